"""GPU parity of the linear layer (det_gemm): the HIP MFMA path against the
FP64 oracle, and bitwise invariance of dX and dW across every layout of the
same logical rows.  Sizes span several 128 x 128 output tiles with ragged
tails in rows, outputs and inputs, and more than one dW group."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests import parity_utils as pu
from invariant_rmsnorm_backward_amd import adapters, binding, contract, harness, inputs, layouts

pytestmark = pytest.mark.gpu
CONTRACT = contract.load_contract()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _wl(name, k, n, lengths, pad_rows=0):
    return inputs.scaled(inputs.workload_linear(), name, hidden=k, lengths=lengths,
                         pad_rows=pad_rows, out_features=n)


def _reference(wl):
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_wmat(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl))
    dx, dw, dwa = oracle.linear_bwd_bf16(xb, wb, dyb)
    return {"dX": dx, "dW": dw, "y": oracle.linear_fwd_bf16(xb, wb)}, dwa


CASES = {
    # name: (k in, n out, lengths, chunk)
    "k200_n136_ragged": (200, 136, [300, 257, 150], 100),
    "k256_n384": (256, 384, [128, 129, 64], 64),
    "k1024_n512": (1024, 512, [333, 211], 128),
    "k72_n8_thin": (72, 8, [77, 60], 33),
    "k8_n200_tiny_k": (8, 200, [50, 13], 17),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_det_gemm_parity_and_invariance(case):
    k, n, lengths, chunk = CASES[case]
    wl = _wl(f"lin_{case}", k, n, lengths)
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    ref, _ = _reference(wl)
    cells = layouts.standard_matrix(wl, chunk)
    print(f"[linear] {case}: {len(cells)} cells", flush=True)
    rep = harness.assert_gradient_batch_invariant("det_gemm", cells, CONTRACT, data=data,
                                                  reference=ref, raise_on_red=False)
    if not rep.strict:
        print(rep.to_json()[:4000], flush=True)
    assert rep.strict, rep.first_failure
    assert all(v.max_abs == 0.0 for v in rep.invariance_reports)


def test_det_gemm_edge_tiles_of_a_padded_tile_grid():
    """Output grids that 4 x 8 super-blocks of 256 x 256 tiles do not tile are
    launched as whole super-blocks, with the workgroups past the grid's edge
    exiting at once: y (64 x 31 tiles) and dW (31 x 8 tiles) here, with a
    ragged last tile column.  y and dX on the first and last tile rows and
    columns and at random entries, and dW (within the canonical order's error
    bound), against single FP64 oracle outputs; a layout with padding rows in
    front (another row grid) gives the same bits."""
    T, N, K = 16384, 7928, 2048
    wl = _wl("lin_padded_grid", K, N, [T])
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    out = adapters.LinearAdapter().run_cell(layouts.full(wl), data)
    # 37 padding rows first, every real row 37 places down (another row grid):
    # the same bits
    out_p = adapters.LinearAdapter().run_cell(layouts.padded(wl, T + 37, "left"), data)
    for name in ("y", "dX", "dW"):
        assert np.array_equal(out[name].view(np.uint8), out_p[name].view(np.uint8)), name
    assert bool(out_p["pad_rows_clean"][0])
    xb, wb, dyb = (inputs.bf16_bits(t) for t in (data.x, data.w, data.dy))
    rng = np.random.default_rng(31)
    n_s = 64
    edge_r = np.array([0, 255, 256, T - 256, T - 1, 0, T - 1, 7000])
    edge_n = np.array([0, N - 1, N - 120, N - 1, 0, 31 * 256 - 257, N - 256, 4000])
    ry = np.concatenate([edge_r, rng.integers(0, T, n_s)])
    ny = np.concatenate([edge_n, rng.integers(0, N, n_s)])
    rx = np.concatenate([edge_r, rng.integers(0, T, n_s)])
    kx = np.concatenate([[0, K - 1, 255, 256, K - 256, 1024, 0, K - 1], rng.integers(0, K, n_s)])
    nw = np.concatenate([edge_n, rng.integers(0, N, n_s)])
    kw = np.concatenate([[0, K - 1, 255, 256, K - 256, 1024, K - 1, 0], rng.integers(0, K, n_s)])
    m = len(ry)
    kind = np.concatenate([np.full(m, 3, np.int32), np.zeros(m, np.int32), np.ones(m, np.int32),
                           np.full(m, 2, np.int32)])
    ia = np.concatenate([ry, rx, nw, nw]).astype(np.int64)
    ib = np.concatenate([ny, kx, kw, kw]).astype(np.int64)
    ref = oracle.linear_sample_bf16(xb, wb, dyb, kind, ia, ib)
    y_ref, dx_ref, dw_ref, dwa = ref[:m], ref[m:2 * m], ref[2 * m:3 * m], ref[3 * m:]
    y_got = harness.bf16_bits_to_f32(out["y"][ry, ny]).astype(np.float64)
    dx_got = harness.bf16_bits_to_f32(out["dX"][rx, kx]).astype(np.float64)
    dw_got = out["dW"][nw, kw].astype(np.float64)
    assert CONTRACT.accuracy_passes(y_got, y_ref, "y")
    assert CONTRACT.accuracy_passes(dx_got, dx_ref, "dX")
    assert CONTRACT.accuracy_passes(dw_got, dw_ref, "dW")
    assert np.all(np.abs(dw_got - dw_ref) <= (1024 + 2) * 2.0 ** -24 * dwa + 1e-30)


def test_det_gemm_two_groups_and_the_group_tree():
    """More than 16384 logical rows: two dW groups joined by the tree, for one
    call, for staged chunks, and for a first call that holds group 0 whole and
    ends at its last row (its chain runs from the call's own buffer, whose
    rows end where the group does)."""
    wl = _wl("lin_two_groups", 64, 72, [9000, 7384, 700])
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    ref, dwa = _reference(wl)
    cells = [layouts.full(wl), layouts.chunked_packed(wl, chunk=4000),
             layouts.permuted(wl),
             layouts.chunked_packed(wl, sizes=[16384, 700], name="BN/chunked_group_whole")]
    rep = harness.assert_gradient_batch_invariant("det_gemm", cells, CONTRACT, data=data,
                                                  reference=ref, raise_on_red=False)
    assert rep.strict, rep.first_failure
    out = adapters.LinearAdapter().run_cell(cells[0], data)
    err = np.abs(out["dW"].astype(np.float64) - ref["dW"])
    # error bound of the canonical order: one rounding per 16-row step of a
    # group chain (1024 steps) plus the tree, relative to the sum of |terms|
    assert np.all(err <= (1024 + 2) * 2.0 ** -24 * dwa + 1e-30)


def test_det_gemm_padding_rows_are_never_read():
    wl = _wl("lin_pad", 128, 128, [100, 60, 31], pad_rows=40)
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    ref, _ = _reference(wl)
    cells = [layouts.full(wl), layouts.packed_with_padding(wl), layouts.padded(wl, 230, "left")]
    rep = harness.assert_gradient_batch_invariant("det_gemm", cells, CONTRACT, data=data,
                                                  reference=ref, raise_on_red=False)
    assert rep.strict, rep.first_failure
    out = adapters.LinearAdapter().run_cell(cells[1], data)
    assert bool(out["pad_rows_clean"][0])


def test_det_gemm_accumulator_protocol():
    wl = _wl("lin_proto", 64, 64, [100])
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    T = wl.n_logical
    acc = binding.GemmDwAccumulator(T, 64, 64)
    half = layouts.chunked_packed(wl, sizes=[60, 40]).calls
    l0 = binding.Layout(half[0].row_logical, T)
    l1 = binding.Layout(half[1].row_logical, T)
    acc.contrib(data.x[:60], data.dy[:60], l0)
    with pytest.raises(binding.RmsNormError) as ei:
        acc.contrib(data.x[:60], data.dy[:60], l0)
    assert ei.value.code == binding.ECOVERAGE
    with pytest.raises(binding.RmsNormError) as ei:
        acc.finalize()
    assert ei.value.code == binding.ECOVERAGE
    acc.contrib(data.x[60:], data.dy[60:], l1)
    d1 = acc.finalize().cpu().numpy()
    d2 = acc.finalize().cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    with pytest.raises(binding.RmsNormError) as ei:
        acc.contrib(data.x[60:], data.dy[60:], l1)
    assert ei.value.code == binding.ESTATE
    acc.reset()
    acc.contrib(data.x, data.dy)
    d3 = acc.finalize().cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d3.view(np.uint32))
    acc.close()
    # zero logical rows: dW = 0
    acc0 = binding.GemmDwAccumulator(0, 64, 64)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    acc0.contrib(e, e)
    assert bool((acc0.finalize() == 0).all())
    acc0.close()


def test_det_gemm_rows_are_independent_of_the_call():
    """The same row gives the same dX and y bits alone, in a small call and
    inside the full batch (tile position and row count do not matter)."""
    wl = _wl("lin_rows", 384, 256, [700])
    data = adapters.make_linear_inputs(wl, device="cuda", gen_device="cpu")
    full_dx = binding.gemm_bwd_dx(data.dy, data.w)
    full_y = binding.gemm_fwd(data.x, data.w)
    for a, b in ((0, 1), (5, 6), (129, 300), (650, 700)):
        dx = binding.gemm_bwd_dx(data.dy[a:b].contiguous(), data.w)
        y = binding.gemm_fwd(data.x[a:b].contiguous(), data.w)
        assert torch.equal(dx.view(torch.int16), full_dx[a:b].view(torch.int16))
        assert torch.equal(y.view(torch.int16), full_y[a:b].view(torch.int16))


@pytest.mark.parametrize("k,n,lengths,chunk", [(1024, 512, [333, 211], 128), (4096, 256, [300, 97], 64),
                                               (128, 256, [150, 77, 9], 32)])
def test_norm_linear_chain_is_invariant_in_every_tensor(k, n, lengths, chunk):
    """RMSNorm -> linear, forward and backward, call by call in every layout:
    every intermediate and every gradient bitwise equal to the B=N run, and
    the per-op gradients within the contract of each op's own oracle."""
    wl = _wl(f"chain_k{k}_n{n}", k, n, lengths)
    data = adapters.make_chain_inputs(wl, device="cuda", gen_device="cpu")
    cells = layouts.standard_matrix(wl, chunk)
    ad = adapters.NormLinearChainAdapter()
    rep = harness.assert_gradient_batch_invariant(ad, cells, CONTRACT, data=data,
                                                  raise_on_red=False)
    assert rep.strict, (rep.first_failure, rep.chain_attribution)
    assert rep.chain_attribution == {}
    assert {v.tensor for v in rep.invariance_reports} == set(ad.tensor_order)
    # the chain against an oracle chain of its own: FP64 ops, bf16 rounding between them
    # done on the oracle side (row-local outputs only: the sums over rows inherit the
    # occasional one-ulp difference of a rounded intermediate, and each op's dW /
    # dweight is checked against its own oracle in the single-op tests)
    out = ad.run_cell(cells[0], data)
    xb = inputs.bf16_bits(data.x.cpu())
    wb = inputs.bf16_bits(data.w.cpu())
    Wb = inputs.bf16_bits(data.wmat.cpu())
    dyb = inputs.bf16_bits(data.dy.cpu())
    y1, _ = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    y1b = oracle.round_bf16(y1)
    y2 = oracle.linear_fwd_bf16(y1b, Wb)
    dX, _, _ = oracle.linear_bwd_bf16(y1b, Wb, dyb)
    dx, _, _ = oracle.rmsnorm_bwd_bf16(xb, wb, oracle.round_bf16(dX), wl.eps)
    for name, want, tol in (("rms_norm.y", y1, "y"), ("det_gemm.y", y2, "y"),
                            ("det_gemm.dX", dX, "dX"), ("rms_norm.dx", dx, "dx")):
        got = harness.bf16_bits_to_f32(out[name])
        assert CONTRACT.accuracy_passes(got, want, tol), name
        # and the bf16 outputs, element by element, within one bf16 ulp of FP64
        frac = pu.bf16_ulp_fraction(np.asarray(out[name]), want)
        print(f"[chain] k{k} n{n}: {name} within 1 bf16 ulp of FP64: {frac:.5f}", flush=True)
        assert frac > 0.99, (name, frac)


@pytest.mark.parametrize("k,n,lengths", [
    (64, 72, [9000, 7384, 700]),       # 128 x 128 output tiles, two dW groups
    (512, 384, [12000, 4500, 1200]),   # 256 x 256 output tiles, two dW groups
])
def test_det_gemm_dw_bits_equal_the_exact_sum(k, n, lengths):
    """Small-integer x and dY (|x|, |dY| <= 3): every product and every partial
    sum of dW = dY^T X is an integer below 2^24, so every FP32 addition in any
    order is exact and the canonical order must give the FP64 oracle's value
    bit for bit, whatever the tile shape, the group split and the layout.
    A dropped, repeated or misplaced row, a wrong group join or a tile that
    reads outside its block changes an integer and fails here."""
    wl = _wl(f"lin_exact_k{k}_n{n}", k, n, lengths)
    T = wl.n_logical
    g = torch.Generator().manual_seed(0x6D0E + k)
    xi = torch.randint(-3, 4, (T, k), generator=g).to(torch.bfloat16)
    gi = torch.randint(-3, 4, (T, n), generator=g).to(torch.bfloat16)
    data = adapters.LinearInputs(wl.name, wl, xi.cuda(), inputs.gen_wmat(wl, device="cuda"),
                                 gi.cuda(), inputs.n_active(wl))
    xb = xi.view(torch.int16).numpy().view(np.uint16)
    gb = gi.view(torch.int16).numpy().view(np.uint16)
    wb = inputs.bf16_bits(inputs.gen_wmat(wl))
    _, dw_ref, _ = oracle.linear_bwd_bf16(xb, wb, gb)
    assert np.abs(dw_ref).max() < 2.0 ** 24 and np.all(dw_ref == np.round(dw_ref))
    want = dw_ref.astype(np.float32)
    cells = [layouts.full(wl), layouts.chunked_packed(wl, chunk=3001), layouts.permuted(wl),
             layouts.singleton_aggregate(wl), layouts.padded(wl, T + 77, "left")]
    for cell in cells:
        out = adapters.LinearAdapter().run_cell(cell, data)
        assert np.array_equal(out["dW"].view(np.uint32), want.view(np.uint32)), cell.name
