"""GPU parity: the HIP path against the FP64 oracle, and bitwise invariance
across every layout of the same logical rows.  Sizes span several 64-row
blocks and a ragged tail, and every kernel variant (lane groups, one
wavefront per row with and without lane masks, two wavefronts per row)."""
import numpy as np
import pytest
import torch

import oracle
from invariant_rmsnorm_backward_amd import adapters, binding, contract, harness, inputs, layouts
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu
CONTRACT = contract.load_contract()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


# Tests that take this fixture run on each of the backward's work
# distributions (tests/parity_utils.py, BWD_PATHS).
@pytest.fixture(params=sorted(pu.BWD_PATHS))
def bwd_path(request):
    with pu.forced_path(request.param):
        yield request.param


def _run(op, cells, data, ref, name):
    print(f"[parity] {name}: {len(cells)} cells", flush=True)
    rep = harness.assert_gradient_batch_invariant(op, cells, CONTRACT, data=data, reference=ref,
                                                  raise_on_red=False)
    if not rep.strict:
        print(rep.to_json()[:4000], flush=True)
    assert rep.strict, rep.first_failure
    return rep


def _check_call_log(adapter_calls, cells):
    by_cell = {}
    for cname, _, rows in adapter_calls:
        by_cell.setdefault(cname, []).append(rows)
    for c in cells:
        assert by_cell[c.name] == c.call_shapes, c.name
    assert len(by_cell["BN/full"]) == 1


WIDE_CASES = {
    # name: (base workload, hidden, lengths, chunk)
    "h4096": (inputs.workload_h4096, 4096, [300, 257, 150], 100),
    "h8192": (inputs.workload_h8192, 8192, [130, 333, 61], 128),
    "h5120": (inputs.workload_h5120, 5120, [200, 100, 50, 30, 77], 64),
    "h512": (inputs.workload_h4096, 512, [70, 45, 129], 50),
    "h1000_masked": (inputs.workload_h4096, 1000, [70, 45], 33),
    "h2048": (inputs.workload_h4096, 2048, [64, 64, 65], 64),
    "h3072": (inputs.workload_h4096, 3072, [150, 97, 64], 48),
    "h6144_two_waves": (inputs.workload_h8192, 6144, [99, 30], 40),
    "h9000_two_waves_masked": (inputs.workload_h8192, 9000, [77, 60], 64),
    "h10240_max": (inputs.workload_h8192, 10240, [90, 41], 64),
    "h40_masked": (inputs.workload_h8, 40, [70, 45, 3], 17),
    "h16": (inputs.workload_h8, 16, [70, 45, 3], 17),
    "h128": (inputs.workload_h8, 128, [130, 2, 61], 32),
    "h256": (inputs.workload_h8, 256, [130, 61], 32),
}


@pytest.mark.parametrize("case", sorted(WIDE_CASES))
def test_rms_norm_parity_and_invariance(case, bwd_path):
    base, H, lengths, chunk = WIDE_CASES[case]
    wl = inputs.scaled(base(), f"{case}_t{sum(lengths)}", hidden=H, lengths=lengths, pad_rows=0)
    data = pu.make_data(wl)
    ref = pu.oracle_reference(wl)
    cells = pu.standard_cells(wl, chunk)
    ad = adapters.RmsNormAdapter()
    rep = _run(ad, cells, data, ref, f"{case} ({bwd_path})")
    _check_call_log(ad.call_log, cells)
    # element by element: more than 99% of the bf16 outputs within one bf16
    # ulp of FP64 (the contract's bound above is looser than one ulp)
    out = ad.run_cell(cells[0], data)
    for t in ("y", "dx"):
        frac = pu.bf16_ulp_fraction(out[t], ref[t])
        print(f"[parity] {case}: {t} within 1 bf16 ulp of FP64: {frac:.5f}", flush=True)
        assert frac > 0.99, (t, frac)
    assert rep.active_token_denominator == inputs.n_active(wl)


def test_page_matrix_h8_t59():
    """The hidden=8, 59-row matrix of the page: every cell bitwise equal."""
    wl = inputs.workload_h8()
    data = pu.make_data(wl)
    ref = pu.oracle_reference(wl)
    cells = layouts.page_matrix(wl)
    ad = adapters.RmsNormAdapter()
    rep = _run(ad, cells, data, ref, "page_matrix_h8")
    _check_call_log(ad.call_log, cells)
    names = {c.name for c in rep.cells}
    assert {"BN/full", "BN/chunked", "B1-singleton_aggregate/full", "BN/padded_right",
            "BN/padded_left", "BN/permuted"} <= names
    assert all(v.max_abs == 0.0 for v in rep.invariance_reports)


def test_qk_norm_parity_and_invariance():
    wq = inputs.scaled(inputs.workload_qk("q"), "qk_q_small", lengths=[100, 37, 64])
    wk = inputs.scaled(inputs.workload_qk("k"), "qk_k_small", lengths=[100, 37, 64])
    data = adapters.QkInputs("qk_small", pu.make_data(wq), pu.make_data(wk))
    rq, rk = pu.oracle_reference(wq), pu.oracle_reference(wk)
    ref = {"dq": rq["dx"], "dk": rk["dx"], "dweight_q": rq["dweight"], "dweight_k": rk["dweight"],
           "yq": rq["y"], "yk": rk["y"], "rstd_q": rq["rstd"], "rstd_k": rk["rstd"]}
    _run("qk_norm", pu.qk_cells(wq, wk, 16), data, ref, "qk_norm")
    # the same cells with Q and K of every call in one launch per phase
    _run("qk_norm_pair", pu.qk_cells(wq, wk, 16), data, ref, "qk_norm_pair")


def test_masked_padded_permuted_packing_h5120():
    """25% padding rows between permuted samples, mask density 0.5."""
    wl = inputs.scaled(inputs.workload_h5120(), "h5120_packed_small", lengths=[200, 100, 50, 30, 77],
                       pad_rows=150)
    data = pu.make_data(wl)
    ref = pu.oracle_reference(wl)
    cells = [layouts.full(wl), layouts.packed_with_padding(wl), layouts.singleton_aggregate(wl)]
    rep = _run("rms_norm", cells, data, ref, "h5120_packed")
    assert rep.cells[1].n_pad_rows == 150


def test_inactive_rows_do_not_change_dweight_bits():
    wl = inputs.scaled(inputs.workload_h5120(), "h5120_inactive", hidden=1024, lengths=[150, 90])
    data = pu.make_data(wl)
    s, p, _ = inputs.logical_keys(wl)
    inactive = torch.from_numpy(~inputs.active_mask(wl, s, p)).cuda()
    assert bool(inactive.any())
    ad = adapters.RmsNormAdapter()
    base = ad.run_cell(layouts.full(wl), data)
    x2 = data.x.clone()
    x2[inactive] = (x2[inactive].float() * -3.0 + 0.5).to(torch.bfloat16)
    data2 = adapters.NormInputs(data.name, wl, x2, data.w, data.dy, data.eps,
                                data.active_token_denominator)
    pert = ad.run_cell(layouts.permuted(wl), data2)
    assert np.array_equal(base["dweight"].view(np.uint32), pert["dweight"].view(np.uint32))
    act = ~inactive.cpu().numpy()
    assert np.array_equal(base["dx"][act], pert["dx"][act])


@pytest.mark.parametrize("H,lengths", [(8, [59]), (128, [200, 77]), (4096, [130, 70]),
                                       (5120, [100, 29]), (1000, [64, 1]), (8192, [66, 70]),
                                       (9000, [40, 41]), (8, [40000]), (16, [70000, 33001])])
def test_dweight_is_the_canonical_order_bit_for_bit(H, lengths, bwd_path):
    """Tree conformance: given the same FP32 rstd, the GPU dweight equals the
    oracle's FP32 emulation of CDO-v2 bit for bit, for one call and for
    chunked calls."""
    wl = inputs.scaled(inputs.workload_h4096(), f"cdo_h{H}", hidden=H, lengths=lengths)
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl))
    _, rstd64 = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    rstd32 = rstd64.astype(np.float32)
    want = oracle.cdo_v2_dweight_f32(xb, dyb, rstd32)
    data = pu.make_data(wl)
    T = wl.n_logical
    for cell in (layouts.full(wl), layouts.chunked_packed(wl, chunk=23),
                 layouts.padded(wl, T + 5, "left")):
        acc = binding.DwAccumulator(T, H)
        for call in cell.calls:
            if call.row_logical is None:
                xc, dyc, lay = data.x, data.dy, None
            else:
                rl = torch.from_numpy(call.row_logical.astype(np.int64)).cuda()
                real = rl >= 0
                xc = torch.zeros((call.rows, H), dtype=torch.bfloat16, device="cuda")
                dyc = torch.zeros_like(xc)
                xc[real] = data.x[rl[real]]
                dyc[real] = data.dy[rl[real]]
                lay = binding.Layout(call.row_logical, T)
            binding.dw_contrib(xc, dyc, pu.physical_rstd(rstd32, call), acc, lay)
        got = acc.finalize().cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (H, cell.name)
    print(f"[cdo] H={H} ({bwd_path}): GPU dweight == CDO-v2 emulation bit for bit", flush=True)


@pytest.mark.parametrize("H,T,chunk", [(8, 40000, 8192), (16, 131000, 30000), (8, 262000, 65536),
                                         (8, 524288, 131072), (8, 524352, 131072),
                                         (1024, 70000, 16384)])
def test_block_tree_over_many_blocks_is_the_canonical_tree(H, T, chunk):
    """The cross-block tree over more than 512 block partials runs level by
    level (512 leaves per workgroup, then the tree over their roots padded
    with +0.0): dweight equals the oracle's FP32 emulation of CDO-v2 bit for
    bit at 625, 2047, 4094, 8192 and 8193 blocks (two levels) and
    at 1094 blocks of hidden 1024, for one call and for large chunks."""
    wl = inputs.scaled(inputs.workload_h4096(), f"tree_h{H}_t{T}", hidden=H, lengths=[T])
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl))
    _, rstd64 = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    rstd32 = rstd64.astype(np.float32)
    want = oracle.cdo_v2_dweight_f32(xb, dyb, rstd32)
    data = pu.make_data(wl)
    rstd_d = torch.from_numpy(rstd32).cuda()
    print(f"[tree] H={H} T={T}: {(T + 63) // 64} blocks", flush=True)
    for cell in (layouts.full(wl), layouts.chunked_packed(wl, chunk=chunk)):
        acc = binding.DwAccumulator(T, H)
        for call in cell.calls:
            if call.row_logical is None:
                binding.dw_contrib(data.x, data.dy, rstd_d, acc)
            else:
                rl = torch.from_numpy(call.row_logical.astype(np.int64)).cuda()
                lay = binding.Layout(call.row_logical, T)
                binding.dw_contrib(data.x[rl].contiguous(), data.dy[rl].contiguous(),
                                   rstd_d[rl].contiguous(), acc, lay)
        got = acc.finalize().cpu().numpy()
        torch.cuda.synchronize()
        acc.close()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (H, T, cell.name)


@pytest.mark.parametrize("H", [24, 128, 520, 1024, 1032, 4096, 5120, 9000])
def test_padding_rows_are_written_as_positive_zero(H):
    """Padding rows are never read (they hold NaN here) and come out as +0.0
    bits in y and dx, with rstd +0.0, also where the weight is negative (a
    computed (0*rstd)*w would be -0.0 there); real rows match the unpadded call."""
    wl = inputs.scaled(inputs.workload_h4096(), f"pads_h{H}", hidden=H, lengths=[70, 59])
    data = pu.make_data(wl)
    T = wl.n_logical
    w = -data.w                                   # negative weights
    rl = np.full(T + 40, -1, dtype=np.int32)
    real_at = np.sort(np.random.default_rng(H).choice(T + 40, size=T, replace=False))
    rl[real_at] = np.arange(T, dtype=np.int32)
    lay = binding.Layout(rl, T)
    nan = torch.full((T + 40, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx = torch.from_numpy(real_at.astype(np.int64)).cuda()
    x, dy = nan.clone(), nan.clone()
    x[idx] = data.x
    dy[idx] = data.dy
    y, rstd = binding.fwd(x, w, data.eps, lay)
    dx = binding.bwd(x, w, dy, rstd, lay)
    y0, r0 = binding.fwd(data.x, w, data.eps)
    dx0 = binding.bwd(data.x, w, data.dy, r0)
    pad = torch.from_numpy(np.flatnonzero(rl < 0).astype(np.int64)).cuda()
    assert torch.equal(y[pad].view(torch.int16), torch.zeros_like(y[pad]).view(torch.int16)), H
    assert torch.equal(dx[pad].view(torch.int16), torch.zeros_like(dx[pad]).view(torch.int16)), H
    assert torch.equal(rstd[pad].view(torch.int32), torch.zeros_like(rstd[pad]).view(torch.int32)), H
    assert torch.equal(y[idx].view(torch.int16), y0.view(torch.int16)), H
    assert torch.equal(rstd[idx].view(torch.int32), r0.view(torch.int32)), H
    assert torch.equal(dx[idx].view(torch.int16), dx0.view(torch.int16)), H
    lay.close()


@pytest.mark.parametrize("nbytes", [16, 4096, 3 * (1 << 20) + 16 * 37])
def test_stream_copy_copies_every_byte(nbytes):
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros(nbytes // 4 + 8, dtype=torch.int32, device="cuda")
    binding.rmsnorm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, binding.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(dst[: nbytes // 4], src)
    assert not dst[nbytes // 4:].any()            # nothing past the end is written


# the last size needs two grid-stride passes (16,384 workgroups x 1024 units each)
@pytest.mark.parametrize("nbytes", [16, 4096, 3 * (1 << 20) + 16 * 37, 16 * (16384 * 1024 + 37)])
def test_stream_2r1w_writes_the_xor_of_every_unit(nbytes):
    a = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    b = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    c = torch.zeros(nbytes // 4 + 8, dtype=torch.int32, device="cuda")
    binding.rmsnorm_stream_2r1w(a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, binding.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(c[: nbytes // 4], a ^ b)
    assert not c[nbytes // 4:].any()              # nothing past the end is written


def _bf16_scaled(bits: np.ndarray, log2: int) -> np.ndarray:
    """bf16 bit patterns times 2**log2, exactly (exponent field shifted);
    zeros stay zero and a value that would leave the normal range becomes a
    zero of its sign (inputs only: the oracle sees the same bits)."""
    b = bits.astype(np.int32)
    exp = (b >> 7) & 0xFF
    new_exp = exp + log2
    keep = (exp != 0) & (new_exp >= 1) & (new_exp <= 254)
    out = b & 0x8000
    out[keep] = (b[keep] & ~(0xFF << 7)) | (new_exp[keep] << 7)
    return out.astype(np.uint16)


@pytest.mark.parametrize("H", [128, 1024, 4096, 5120])
def test_degenerate_rows_match_the_oracle(H, bwd_path):
    """Rows the method treats specially or that stress FP32, planted in the
    inputs and checked against the FP64 oracle on the same bits in every
    layout cell: an all-zero row (rstd = eps^-1/2, y = 0), a constant row, a
    row scaled by 2^40 and one by 2^-60 (squares near the bottom of FP32), a
    row with a zero upstream gradient (contributes exactly 0), and a row with
    one 2^20 outlier.  The rstd-recompute backward meets the same rows."""
    wl = inputs.scaled(inputs.workload_h4096(), f"degen_h{H}", hidden=H, lengths=[70, 59])
    xb = inputs.bf16_bits(inputs.gen_x(wl)).copy()
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl)).copy()
    xb[0] = 0
    xb[1] = 0x4040                                        # 3.0 in every column
    xb[2] = _bf16_scaled(xb[2], 40)
    xb[3] = _bf16_scaled(xb[3], -60)
    dyb[4] = 0
    xb[5, 7] = 0x4980                                     # 2^20
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    data = adapters.NormInputs(wl.name, wl, dev(xb), dev(wb), dev(dyb), wl.eps, inputs.n_active(wl))
    y, rstd = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    dx, dw, _ = oracle.rmsnorm_bwd_bf16(xb, wb, dyb, wl.eps)
    assert abs(rstd[0] - wl.eps ** -0.5) <= 1e-9 * wl.eps ** -0.5 and not y[0].any()
    ref = {"y": y, "rstd": rstd, "dx": dx, "dweight": dw}
    cells = pu.standard_cells(wl, 37)
    _run("rms_norm", cells, data, ref, f"degenerate h{H} ({bwd_path})")
    # the one-ulp gate over all rows, and row by row over the planted ones
    out = adapters.RmsNormAdapter().run_cell(cells[0], data)
    for t in ("y", "dx"):
        frac = pu.bf16_ulp_fraction(out[t], ref[t])
        rows = [pu.bf16_ulp_fraction(out[t][r], ref[t][r]) for r in range(6)]
        print(f"[degenerate] h{H}: {t} within 1 bf16 ulp: {frac:.5f}, planted rows "
              f"{[round(v, 4) for v in rows]}", flush=True)
        assert frac > 0.99 and min(rows) > 0.99, (t, frac, rows)
    if bwd_path == "fused":   # the rstd-recompute backward always takes the fused kernel
        _run("rms_norm_recompute", cells, data, ref, f"degenerate h{H} (rstd rebuilt)")


def test_fused_dweight_equals_dweight_only_path():
    wl = inputs.scaled(inputs.workload_h4096(), "fused_vs_contrib", lengths=[300, 100])
    data = pu.make_data(wl)
    T, H = data.x.shape
    a1 = binding.DwAccumulator(T, H)
    y, rstd = binding.fwd(data.x, data.w, data.eps)
    binding.bwd(data.x, data.w, data.dy, rstd, acc=a1)
    d1 = a1.finalize().cpu().numpy()
    a2 = binding.DwAccumulator(T, H)
    binding.dw_contrib(data.x, data.dy, rstd, a2)
    d2 = a2.finalize().cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))


@pytest.mark.parametrize("case", ["h4096", "h5120", "h512", "h1000_masked", "h6144_two_waves",
                                  "h9000_two_waves_masked"])
def test_two_pass_backward_is_bitwise_the_fused_one(case):
    """Every cell (partial blocks, spills, padding, permutations) gives the
    same dx, dweight, y and rstd bits on both work distributions, so a cell
    whose calls take different paths stays invariant."""
    base, H, lengths, chunk = WIDE_CASES[case]
    wl = inputs.scaled(base(), f"{case}_paths", hidden=H, lengths=lengths, pad_rows=0)
    data = pu.make_data(wl)
    cells = pu.standard_cells(wl, chunk)
    outs = {}
    for path in pu.BWD_PATHS:
        with pu.forced_path(path):
            ad = adapters.RmsNormAdapter()
            outs[path] = [ad.run_cell(c, data) for c in cells]
    for other in ("stream", "two_pass"):
        for c, a, b in zip(cells, outs["fused"], outs[other]):
            for t in ("dx", "dweight", "y", "rstd"):
                assert np.array_equal(a[t].view(np.uint8), b[t].view(np.uint8)), (case, other, c.name, t)
    # one call over every row: dx with the dweight fold, dx alone and the
    # dweight contributions alone, on each path
    T = wl.n_logical
    _, rstd = binding.fwd(data.x, data.w, data.eps)
    got = {}
    for path in pu.BWD_PATHS:
        with pu.forced_path(path):
            acc = binding.DwAccumulator(T, H)
            dx_fold = binding.bwd(data.x, data.w, data.dy, rstd, acc=acc).view(torch.int16).cpu()
            dw_fold = acc.finalize().view(torch.int32).cpu()
            dw_again = acc.finalize().view(torch.int32).cpu()   # a repeated finalize: same value
            acc.reset()
            binding.dw_contrib(data.x, data.dy, rstd, acc)
            got[path] = (binding.bwd(data.x, data.w, data.dy, rstd).view(torch.int16).cpu(),
                         acc.finalize().view(torch.int32).cpu(), dx_fold, dw_fold, dw_again)
            acc.close()
    for other in ("stream", "two_pass"):
        for i, what in enumerate(("dx", "dw_contrib", "dx_fold", "dw_fold", "dw_refinalized")):
            assert torch.equal(got["fused"][i], got[other][i]), (case, other, what)
    print(f"[paths] {case}: fused == stream == two-pass bitwise over {len(cells)} cells", flush=True)


# Caps on the block-owning workgroups of the fused backward: with a cap the
# workgroups each walk many canonical blocks in turn (prefetching the next
# block's first row across the current block's tree).
GROUP_CAPS = (1, 3, 7)


@pytest.mark.parametrize("case", ["h4096", "h2048", "h3072", "h5120", "h512", "h1000_masked"])
def test_workgroup_cap_changes_no_bit(case):
    """Every cell (complete blocks, spilled partial blocks, padding rows,
    permutations) gives the same dx, dweight, y and rstd bits whatever the
    number of workgroups the fused backward runs with, and so do dx alone,
    the dweight contributions alone and the rstd-recompute backward."""
    base, H, lengths, chunk = WIDE_CASES[case]
    wl = inputs.scaled(base(), f"{case}_caps", hidden=H, lengths=lengths, pad_rows=0)
    data = pu.make_data(wl)
    cells = pu.standard_cells(wl, chunk)
    T = wl.n_logical
    print(f"[caps] {case}: hidden {H}, {T} rows, {len(cells)} cells, caps {GROUP_CAPS}", flush=True)
    outs, single = {}, {}
    prev_thr = binding.rmsnorm_set_split_threshold(0)    # the fused kernel for every call
    try:
        for cap in (0,) + GROUP_CAPS:
            prev = binding.rmsnorm_set_workgroup_cap(cap)
            try:
                ad = adapters.RmsNormAdapter()
                outs[cap] = [ad.run_cell(c, data) for c in cells]
                _, rstd = binding.fwd(data.x, data.w, data.eps)
                acc = binding.DwAccumulator(T, H)
                binding.dw_contrib(data.x, data.dy, rstd, acc)
                dw_only = acc.finalize().view(torch.int32).cpu()
                acc.reset()
                dx_rc = binding.bwd_recompute(data.x, data.w, data.dy, data.eps, acc=acc)
                dw_rc = acc.finalize().view(torch.int32).cpu()
                acc.close()
                dx_only = binding.bwd(data.x, data.w, data.dy, rstd)
                single[cap] = (dx_only.view(torch.int16).cpu(), dw_only,
                               dx_rc.view(torch.int16).cpu(), dw_rc)
            finally:
                binding.rmsnorm_set_workgroup_cap(prev)
    finally:
        binding.rmsnorm_set_split_threshold(prev_thr)
    for cap in GROUP_CAPS:
        for c, a, b in zip(cells, outs[0], outs[cap]):
            for t in ("dx", "dweight", "y", "rstd"):
                assert np.array_equal(a[t].view(np.uint8), b[t].view(np.uint8)), (case, cap, c.name, t)
        for i, (a, b) in enumerate(zip(single[0], single[cap])):
            assert torch.equal(a, b), (case, cap, ("dx", "dw_contrib", "dx_rc", "dw_rc")[i])
    # the recompute backward equals the saved-rstd one
    assert torch.equal(single[0][0], single[0][2]) and torch.equal(single[0][1], single[0][3])


def test_run_to_run_repeatability():
    wl = inputs.scaled(inputs.workload_h4096(), "repeat", lengths=[700, 300])
    data = pu.make_data(wl)
    ad = adapters.RmsNormAdapter()
    first = ad.run_cell(layouts.chunked_packed(wl, chunk=97), data)
    for _ in range(5):
        again = ad.run_cell(layouts.chunked_packed(wl, chunk=97), data)
        for k in first:
            assert np.array_equal(first[k], again[k]), k


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_small_and_ragged_row_counts(T, bwd_path):
    wl = inputs.scaled(inputs.workload_h4096(), f"ragged_{T}", hidden=768, lengths=[T])
    data = pu.make_data(wl)
    ref = pu.oracle_reference(wl)
    cells = [layouts.full(wl), layouts.chunked_packed(wl, chunk=7),
             layouts.padded(wl, T + 64, "right")]
    _run("rms_norm", cells, data, ref, f"ragged_{T}")


def test_zero_rows_and_empty_calls():
    H = 4096
    x = torch.zeros((3, H), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    y, rstd = binding.fwd(x, w, 1e-6)
    torch.cuda.synchronize()
    want = np.full(3, 1.0 / np.sqrt(np.float64(np.float32(1e-6))))    # eps^-1/2, closed form
    assert CONTRACT.accuracy_passes(rstd.cpu().numpy(), want, "rstd")
    assert bool((y.float() == 0).all())
    # rows == 0 is a successful no-op, with and without an accumulator
    e = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    binding.fwd(e, w, 1e-6)
    acc = binding.DwAccumulator(0, H)
    binding.bwd(e, w, e, torch.empty(0, device="cuda"), acc=acc)
    dw = acc.finalize()
    torch.cuda.synchronize()
    assert bool((dw == 0).all())


def test_accumulator_protocol_errors():
    H, T = 512, 100
    wl = inputs.scaled(inputs.workload_h4096(), "proto", hidden=H, lengths=[T])
    data = pu.make_data(wl)
    y, rstd = binding.fwd(data.x, data.w, data.eps)
    acc = binding.DwAccumulator(T, H)
    half = layouts.chunked_packed(wl, sizes=[60, 40]).calls
    lay0 = binding.Layout(half[0].row_logical, T)
    binding.dw_contrib(data.x[:60], data.dy[:60], rstd[:60], acc, lay0)
    with pytest.raises(binding.RmsNormError) as ei:          # the same rows again
        binding.dw_contrib(data.x[:60], data.dy[:60], rstd[:60], acc, lay0)
    assert ei.value.code == binding.ECOVERAGE
    with pytest.raises(binding.RmsNormError) as ei:          # rows 60..99 missing
        acc.finalize()
    assert ei.value.code == binding.ECOVERAGE
    lay1 = binding.Layout(half[1].row_logical, T)
    with pytest.raises(binding.RmsNormError) as ei:          # layout rows != call rows
        binding.dw_contrib(data.x[:41], data.dy[:41], rstd[:41], acc, lay1)
    assert ei.value.code == binding.ELAYOUT
    binding.dw_contrib(data.x[60:], data.dy[60:], rstd[60:], acc, lay1)
    d1 = acc.finalize().cpu().numpy()
    with pytest.raises(binding.RmsNormError) as ei:          # after finalize
        binding.dw_contrib(data.x[60:], data.dy[60:], rstd[60:], acc, lay1)
    assert ei.value.code == binding.ESTATE
    d2 = acc.finalize().cpu().numpy()                        # finalize again: same bits
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    acc.reset()
    binding.dw_contrib(data.x, data.dy, rstd, acc)
    d3 = acc.finalize().cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d3.view(np.uint32))


def test_generator_cpu_gpu_agree():
    wl = inputs.scaled(inputs.workload_h5120(), "gen_agree", hidden=1024, lengths=[300, 211])
    for f in (inputs.gen_x, inputs.gen_dy):
        a = f(wl, device="cpu")
        b = f(wl, device="cuda").cpu()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f.__name__
    assert torch.equal(inputs.gen_w(wl).view(torch.int16),
                       inputs.gen_w(wl, device="cuda").cpu().view(torch.int16))


def test_cli_sweeps_are_green(tmp_path):
    from invariant_rmsnorm_backward_amd import cli
    out = tmp_path / "sweep.json"
    assert cli.main(["sweep", "--workload", "rmsnorm_h8_t59", "--workload", "qknorm_d128_t16384",
                     "--workload", "rmsnorm_h5120_packed131072",
                     "--workload", "linear_h4096_o4096_t32768",
                     "--workload", "chain_rmsnorm_linear_h4096_o4096_t32768",
                     "--workload", "rmsnorm_h5120_packed131072+recompute",
                     "--small", "--json", str(out)]) == 0
    assert cli.main(["check", "--workload", "rmsnorm_h4096_t32768", "--cell", "BN/chunked",
                     "--small"]) == 0
    import json
    reps = json.loads(out.read_text())
    assert len(reps) == 6 and all(r["strict"] for r in reps)


class PerCallFoldOnGpu(adapters.RmsNormAdapter):
    """Negative control on the GPU: dx, y and rstd from the library, but
    dweight summed the way the pages' historical finding describes -- each
    call reduces its own rows (torch's GPU reduction over the call's
    physical rows, whose order follows the call's shape) and the per-call
    partials are added in call order.  The harness must judge it red."""
    name = "rms_norm_per_call_fold"
    aggregation_order = "per-call physical fold"

    def run_cell(self, cell, data):
        out = super().run_cell(cell, data)
        x, dy = data.x.float(), data.dy.float()
        rstd = torch.from_numpy(out["rstd"]).cuda()
        dw = torch.zeros(x.shape[1], dtype=torch.float32, device="cuda")
        for call in cell.calls:
            if call.row_logical is None:
                rows = torch.arange(x.shape[0], device="cuda")
            else:
                rl = torch.from_numpy(call.row_logical.astype(np.int64)).cuda()
                rows = rl[rl >= 0]
            dw = dw + (dy[rows] * x[rows] * rstd[rows, None]).sum(dim=0)
        torch.cuda.synchronize()
        out["dweight"] = dw.cpu().numpy()
        return out


def test_a_per_call_dweight_fold_on_the_gpu_is_red():
    """The harness catches a shape-dependent dweight computed on the GPU
    ("WS1 C4 (#270) closeout evidence", the matrix is falsifiable; the
    historical finding that RMSNorm dweight is not chunk/batch decomposable):
    the chunked and singleton-aggregate cells are red on dweight and the
    first failure names it, while dx (row-local) stays bitwise invariant."""
    wl = inputs.scaled(inputs.workload_h4096(), "negctl_h1024", hidden=1024,
                       lengths=[300, 257, 150, 90])
    data = pu.make_data(wl)
    cells = pu.standard_cells(wl, 100)
    rep = harness.assert_gradient_batch_invariant(PerCallFoldOnGpu(), cells, CONTRACT, data=data,
                                                  raise_on_red=False)
    by = {c.name: c.status for c in rep.cells}
    print(f"[negative control] cell verdicts: {by}", flush=True)
    assert not rep.strict and rep.first_failure["tensor"] == "dweight"
    assert by["BN/chunked"] == harness.RED_VERDICT
    assert by["B1-singleton_aggregate/full"] == harness.RED_VERDICT
    assert all(v.bitwise_equal for v in rep.invariance_reports if v.tensor == "dx")
    # the library's own adapter on the same data and cells is green
    rep_ok = harness.assert_gradient_batch_invariant(adapters.RmsNormAdapter(), cells, CONTRACT,
                                                     data=data, raise_on_red=False)
    assert rep_ok.strict


def test_bounded_spill_area_refuses_when_full_and_matches_unbounded():
    """rmsnorm_dw_acc_create_bounded: a call that needs a spill slot beyond the
    bound is refused with RMSNORM_ESPILL before anything is enqueued and
    leaves the accumulator as it was; with room for exactly the blocks the
    calls split, dweight is bit for bit the unbounded accumulator's, on each
    backward path."""
    H = 1024
    wl = inputs.scaled(inputs.workload_h4096(), "spill_bound_h1024", hidden=H, lengths=[700, 311])
    data = pu.make_data(wl)
    T = wl.n_logical
    x, w, dy = data.x, data.w, data.dy
    _, rstd = binding.fwd(x, w, data.eps)
    # 100-row pieces: blocks 1, 3, 4, 6, ... straddle piece boundaries
    pieces = [(a, min(a + 100, T)) for a in range(0, T, 100)]
    need = {a // 64 for a, b in pieces if a % 64} | {(b - 1) // 64 for a, b in pieces if b % 64 and b < T}
    assert len(need) > 2

    def run(acc, pieces_):
        lays = []
        for a, b in pieces_:
            lay = binding.Layout(np.arange(a, b, dtype=np.int32), T)
            lays.append(lay)
            binding.bwd(x[a:b].contiguous(), w, dy[a:b].contiguous(), rstd[a:b].contiguous(), lay, acc)
        return lays

    for path in pu.BWD_PATHS:
        with pu.forced_path(path):
            ref = binding.DwAccumulator(T, H)
            lays = run(ref, pieces)
            dw_ref = ref.finalize().view(torch.int32).cpu()
            exact = binding.DwAccumulator(T, H, max_spill_rows=64 * len(need))
            lays += run(exact, pieces)
            dw_exact = exact.finalize().view(torch.int32).cpu()
            assert torch.equal(dw_ref, dw_exact), path
            # one slot short: the call that needs the missing slot is refused
            short = binding.DwAccumulator(T, H, max_spill_rows=64 * (len(need) - 1))
            refused_at = None
            for i, (a, b) in enumerate(pieces):
                lay = binding.Layout(np.arange(a, b, dtype=np.int32), T)
                lays.append(lay)
                try:
                    binding.bwd(x[a:b].contiguous(), w, dy[a:b].contiguous(), rstd[a:b].contiguous(),
                                lay, short)
                except binding.RmsNormError as e:
                    assert e.code == binding.ESPILL, e
                    refused_at = i
                    break
            assert refused_at is not None
            # nothing of the refused call was recorded: finalize reports its rows missing
            with pytest.raises(binding.RmsNormError) as ei:
                short.finalize()
            assert ei.value.code == binding.ECOVERAGE
            torch.cuda.synchronize()
            for acc in (ref, exact, short):
                acc.close()
            for lay in lays:
                lay.close()
    print(f"[spill bound] {len(need)} slots: exact bound == unbounded on every path, one short refused",
          flush=True)


@pytest.mark.parametrize("H", [128, 1000, 1024, 4096, 5120, 8192])
def test_whole_block_calls_equal_the_planned_path(H):
    """A call whose rows are whole canonical blocks in logical order runs the
    forward without the map and the backward without a device plan; the same
    rows with one padding row appended take the planned path.  Both give the
    same y, rstd, dx and dweight bits on every backward path, and the same
    dweight as one identity call."""
    wl = inputs.scaled(inputs.workload_h4096(), f"whole_blocks_h{H}", hidden=H, lengths=[400, 300])
    data = pu.make_data(wl)
    T = wl.n_logical
    x, w, dy = data.x, data.w, data.dy
    pieces = [(0, 128), (128, 384), (384, T)]          # block-aligned starts; the last ends at T
    nan_row = torch.full((1, H), float("nan"), dtype=x.dtype, device=x.device)
    _, rstd_all = binding.fwd(x, w, data.eps)
    one = binding.DwAccumulator(T, H)
    binding.bwd(x, w, dy, rstd_all, None, one)
    dw_one = one.finalize().view(torch.int32).cpu()
    one.close()
    lays = []
    for path in pu.BWD_PATHS:
        with pu.forced_path(path):
            dws = []
            for padded in (False, True):
                acc = binding.DwAccumulator(T, H)
                outs = []
                for a, b in pieces:
                    rl = np.arange(a, b, dtype=np.int32)
                    xc, dyc = x[a:b].contiguous(), dy[a:b].contiguous()
                    if padded:
                        rl = np.concatenate([rl, np.array([-1], dtype=np.int32)])
                        xc, dyc = torch.cat([xc, nan_row]), torch.cat([dyc, nan_row])
                    lay = binding.Layout(rl, T)
                    y, rstd = binding.fwd(xc, w, data.eps, lay)
                    dx = binding.bwd(xc, w, dyc, rstd, lay, acc)
                    n = b - a
                    outs.append((y[:n].view(torch.int16).cpu(), rstd[:n].view(torch.int32).cpu(),
                                 dx[:n].view(torch.int16).cpu()))
                    if padded:
                        assert not bool(dx[n:].view(torch.int16).any()), path
                    lays.append(lay)
                dws.append((acc.finalize().view(torch.int32).cpu(), outs))
                torch.cuda.synchronize()
                acc.close()
            (dw_w, out_w), (dw_p, out_p) = dws
            assert torch.equal(dw_w, dw_p), path
            assert torch.equal(dw_w, dw_one), path
            for (yw, rw, dxw), (yp, rp, dxp) in zip(out_w, out_p):
                assert torch.equal(yw, yp) and torch.equal(rw, rp) and torch.equal(dxw, dxp), path
    for lay in lays:
        lay.close()
    print(f"[whole blocks] hidden {H}: planned and plan-free calls bitwise equal on every path", flush=True)
