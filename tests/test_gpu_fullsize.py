"""Full-size workloads in the launch configuration bench.py times.

Every workload runs through the C-ABI on its real shape: bitwise invariance
across its layouts (B=N, N x B=1 aggregate, chunked prefill in both
readings, packed with padding/permutation/mask), dweight against the FP64
oracle over all rows (accumulated in row chunks from CPU-generated inputs),
and dx / y / rstd against the oracle on sampled rows (row-local, so each
sampled row is computed alone)."""
import time

import numpy as np
import pytest
import torch

import oracle
from invariant_rmsnorm_backward_amd import adapters, binding, contract, harness, inputs, layouts
from tests import parity_utils as pu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
CONTRACT = contract.load_contract()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _log(msg):
    print(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _oracle_dweight(wl, chunk=8192):
    """FP64 oracle dweight over all logical rows, accumulated per row chunk."""
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    acc = np.zeros(wl.hidden, dtype=np.float64)
    T = wl.n_logical
    n_act = inputs.n_active(wl)
    for a in range(0, T, chunk):
        rows = np.arange(a, min(a + chunk, T))
        xb = inputs.bf16_bits(inputs.gen_x(wl, rows))
        dyb = inputs.bf16_bits(inputs.gen_dy(wl, rows, denominator=n_act))
        _, dw, _ = oracle.rmsnorm_bwd_bf16(xb, wb, dyb, wl.eps)
        acc += dw
        if (a // chunk) % 8 == 0:
            _log(f"{wl.name}: oracle rows {a + len(rows)}/{T}")
    return acc


def _sample_rows(T, n=200, seed=7):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    pick |= {0, 63, 64, T - 1, T // 2}
    return np.array(sorted(r for r in pick if 0 <= r < T))


def _check_sampled_rows(wl, out, rows):
    """dx, y, rstd of the sampled logical rows against the oracle."""
    n_act = inputs.n_active(wl)
    xb = inputs.bf16_bits(inputs.gen_x(wl, rows))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl, rows, denominator=n_act))
    y, rstd = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    dx, _, _ = oracle.rmsnorm_bwd_bf16(xb, wb, dyb, wl.eps)
    for name, want in (("dx", dx), ("y", y), ("rstd", rstd)):
        got = out[name][rows]
        got = harness.bf16_bits_to_f32(got) if got.dtype == np.uint16 else got
        assert CONTRACT.accuracy_passes(got, want, name), (wl.name, name)
    frac = pu.bf16_ulp_fraction(out["dx"][rows], dx)
    _log(f"{wl.name}: sampled rows {len(rows)}: dx within 1 bf16 ulp {frac:.5f}")
    assert frac > 0.99


def _gpu_data(wl):
    """Logical inputs generated on the GPU (the CPU/GPU generators agree bit
    for bit; test_generator_cpu_gpu_agree) -- the oracle side regenerates its
    rows on the CPU."""
    return adapters.make_inputs(wl, device="cuda")


def _invariance(op, cells, data, name):
    _log(f"{name}: {len(cells)} cells, calls per cell {[len(c.calls) for c in cells]}")
    rep = harness.assert_gradient_batch_invariant(op, cells, CONTRACT, data=data, raise_on_red=False)
    assert rep.strict, rep.first_failure
    return rep


def test_h4096_t32768_bn_vs_singletons_and_chunks():
    wl = inputs.workload_h4096()
    data = _gpu_data(wl)
    cells = [layouts.full(wl), layouts.singleton_aggregate(wl),
             layouts.chunked_per_sample(wl, chunk=512, name="BN/chunked_512"),
             layouts.permuted(wl)]
    ad = adapters.RmsNormAdapter()
    _invariance(ad, cells, data, wl.name)
    out = ad.run_cell(cells[0], data)
    dw = _oracle_dweight(wl)
    assert CONTRACT.accuracy_passes(out["dweight"], dw, "dweight")
    _check_sampled_rows(wl, out, _sample_rows(wl.n_logical))


def test_h8192_varlen_chunked_prefill():
    wl = inputs.workload_h8192()
    _log(f"{wl.name}: T = {wl.n_logical}, lengths {wl.lengths}")
    data = _gpu_data(wl)
    cells = [layouts.full(wl), layouts.chunked_packed(wl, chunk=512, name="BN/chunked_512"),
             layouts.chunked_per_sample(wl, chunk=512, name="BN/chunked_512_per_sample")]
    ad = adapters.RmsNormAdapter()
    _invariance(ad, cells, data, wl.name)
    out = ad.run_cell(cells[0], data)
    del data
    dw = _oracle_dweight(wl)
    assert CONTRACT.accuracy_passes(out["dweight"], dw, "dweight")
    _check_sampled_rows(wl, out, _sample_rows(wl.n_logical))


def test_qk_norm_d128_t16384():
    wq, wk = inputs.workload_qk("q"), inputs.workload_qk("k")
    data = adapters.QkInputs("qknorm_d128_t16384", _gpu_data(wq), _gpu_data(wk))
    cells = [adapters.PairCell(a.name, a, b) for a, b in zip(
        [layouts.full(wq), layouts.singleton_aggregate(wq),
         layouts.chunked_packed(wq, chunk=512, name="BN/chunked_512"),
         layouts.chunked_per_sample(wq, chunk=512, name="BN/chunked_512_per_sample")],
        [layouts.full(wk), layouts.singleton_aggregate(wk),
         layouts.chunked_packed(wk, chunk=512, name="BN/chunked_512"),
         layouts.chunked_per_sample(wk, chunk=512, name="BN/chunked_512_per_sample")])]
    ad = adapters.QkNormAdapter()
    _invariance(ad, cells, data, "qknorm_d128_t16384")
    out = ad.run_cell(cells[0], data)
    for side, wl, dxk, dwk in (("q", wq, "dq", "dweight_q"), ("k", wk, "dk", "dweight_k")):
        dw = _oracle_dweight(wl, chunk=65536)
        assert CONTRACT.accuracy_passes(out[dwk], dw, "dweight"), side
        _check_sampled_rows(wl, {"dx": out[dxk], "y": out["y" + side], "rstd": out["rstd_" + side]},
                            _sample_rows(wl.n_logical))


def test_h5120_packed_padded_permuted_masked():
    wl = inputs.workload_h5120()
    data = _gpu_data(wl)
    cells = [layouts.full(wl), layouts.packed_with_padding(wl), layouts.singleton_aggregate(wl)]
    assert cells[1].calls[0].rows == 131072 and cells[1].calls[0].n_pad == 32768
    ad = adapters.RmsNormAdapter()
    _invariance(ad, cells, data, wl.name)
    out = ad.run_cell(cells[0], data)
    del data
    dw = _oracle_dweight(wl)
    assert CONTRACT.accuracy_passes(out["dweight"], dw, "dweight")
    _check_sampled_rows(wl, out, _sample_rows(wl.n_logical))


def test_linear_h4096_o4096_t32768_sampled():
    """det_gemm at its full size (32768 rows, 4096 -> 4096): dX and dW bitwise
    across B=N, 8 x B=1 and chunked-512 calls; sampled dX and dW entries
    against the FP64 oracle, each computed alone, and within the error bound
    of the canonical order."""
    wl = inputs.workload_linear()
    data = adapters.make_linear_inputs(wl, device="cuda")
    cells = [layouts.full(wl), layouts.singleton_aggregate(wl),
             layouts.chunked_packed(wl, chunk=512, name="BN/chunked_512")]
    _invariance("det_gemm", cells, data, wl.name)
    out = adapters.LinearAdapter().run_cell(cells[0], data)
    xb = inputs.bf16_bits(data.x)
    wb = inputs.bf16_bits(data.w)
    dyb = inputs.bf16_bits(data.dy)
    rng = np.random.default_rng(11)
    T, N, K = wl.n_logical, wl.out_features, wl.hidden
    n_s = 96
    r = np.concatenate([[0, T - 1, 16383, 16384], rng.integers(0, T, n_s)])
    kk = np.concatenate([[0, K - 1, 255, 256], rng.integers(0, K, n_s)])
    nn = np.concatenate([[0, N - 1, 127, 128], rng.integers(0, N, n_s)])
    m = len(r)
    # y over the vocabulary side: the corners of the grid and the tiles on its
    # last row and column of 256 x 256 tiles, plus random entries
    ry = np.concatenate([[0, T - 1, T - 1, 0, T - 256, 255], rng.integers(0, T, n_s)])
    ny = np.concatenate([[0, N - 1, 0, N - 1, N - 256, N - 257], rng.integers(0, N, n_s)])
    kind = np.concatenate([np.zeros(m, np.int32), np.ones(m, np.int32), np.full(m, 2, np.int32),
                           np.full(len(ry), 3, np.int32)])
    ia = np.concatenate([r, nn, nn, ry]).astype(np.int64)
    ib = np.concatenate([kk, kk, kk, ny]).astype(np.int64)
    _log(f"{wl.name}: {len(kind)} oracle samples")
    ref = oracle.linear_sample_bf16(xb, wb, dyb, kind, ia, ib)
    dx_ref, dw_ref, dwa, y_ref = ref[:m], ref[m:2 * m], ref[2 * m:3 * m], ref[3 * m:]
    dx_got = harness.bf16_bits_to_f32(out["dX"][r, kk]).astype(np.float64)
    dw_got = out["dW"][nn, kk].astype(np.float64)
    y_got = harness.bf16_bits_to_f32(out["y"][ry, ny]).astype(np.float64)
    assert CONTRACT.accuracy_passes(dx_got, dx_ref, "dX")
    assert CONTRACT.accuracy_passes(dw_got, dw_ref, "dW")
    assert CONTRACT.accuracy_passes(y_got, y_ref, "y")
    # one rounding per 16-row step of a group chain (1024 steps) plus the tree
    assert np.all(np.abs(dw_got - dw_ref) <= (1024 + 2) * 2.0 ** -24 * dwa + 1e-30)
    _log(f"{wl.name}: sampled dX/dW match the oracle; max |dW err| / |dW| scale "
         f"{float(np.max(np.abs(dw_got - dw_ref)) / max(np.max(np.abs(dw_ref)), 1e-30)):.2e}")


def test_lmhead_v32000_h4096_t32768_sampled():
    """The LM-head weight gradient at its real shape: det_gemm with N = the
    32,000-token vocabulary, K = 4096, on 32768 rows (two dW groups).  dX and
    dW bitwise across B=N, 8 x B=1 and chunked-512 calls (the B=N call runs
    both group chains at once, the others stage the rows of the groups they
    split); sampled y, dX and dW entries against the FP64 oracle (y on every
    edge of the vocabulary-wide tile grid), dW within the error bound of the
    canonical order."""
    wl = inputs.workload_lmhead()
    data = adapters.make_linear_inputs(wl, device="cuda")
    cells = [layouts.full(wl), layouts.singleton_aggregate(wl),
             layouts.chunked_packed(wl, chunk=512, name="BN/chunked_512")]
    _invariance("det_gemm", cells, data, wl.name)
    out = adapters.LinearAdapter().run_cell(cells[0], data)
    xb = inputs.bf16_bits(data.x)
    wb = inputs.bf16_bits(data.w)
    dyb = inputs.bf16_bits(data.dy)
    del data
    rng = np.random.default_rng(13)
    T, N, K = wl.n_logical, wl.out_features, wl.hidden
    n_s = 96
    r = np.concatenate([[0, T - 1, 16383, 16384], rng.integers(0, T, n_s)])
    kk = np.concatenate([[0, K - 1, 255, 256], rng.integers(0, K, n_s)])
    nn = np.concatenate([[0, N - 1, 31999 - 255, 256], rng.integers(0, N, n_s)])
    m = len(r)
    kind = np.concatenate([np.zeros(m, np.int32), np.ones(m, np.int32), np.full(m, 2, np.int32)])
    ia = np.concatenate([r, nn, nn]).astype(np.int64)
    ib = np.concatenate([kk, kk, kk]).astype(np.int64)
    _log(f"{wl.name}: {3 * m} oracle samples")
    ref = oracle.linear_sample_bf16(xb, wb, dyb, kind, ia, ib)
    dx_ref, dw_ref, dwa = ref[:m], ref[m:2 * m], ref[2 * m:]
    dx_got = harness.bf16_bits_to_f32(out["dX"][r, kk]).astype(np.float64)
    dw_got = out["dW"][nn, kk].astype(np.float64)
    assert CONTRACT.accuracy_passes(dx_got, dx_ref, "dX")
    assert CONTRACT.accuracy_passes(dw_got, dw_ref, "dW")
    assert np.all(np.abs(dw_got - dw_ref) <= (1024 + 2) * 2.0 ** -24 * dwa + 1e-30)
    _log(f"{wl.name}: sampled dX/dW match the oracle; max |dW err| / |dW| scale "
         f"{float(np.max(np.abs(dw_got - dw_ref)) / max(np.max(np.abs(dw_ref)), 1e-30)):.2e}")


def test_embedding_v32000_d4096_t32768_sampled_columns():
    """det_embedding at full size (32768 rows, 32000 x 4096 table, Zipf ids):
    dE bitwise across B=N, 8 x B=1 and chunked-512 calls; on sampled columns,
    dE against the FP64 oracle and bit for bit against the EDO-v1 emulation."""
    wl = inputs.workload_embedding()
    data = adapters.make_embedding_inputs(wl, device="cuda")
    cells = [layouts.full(wl), layouts.singleton_aggregate(wl),
             layouts.chunked_packed(wl, chunk=512, name="BN/chunked_512")]
    _invariance("embedding", cells, data, wl.name)
    out = adapters.EmbeddingAdapter().run_cell(cells[0], data)
    cols = np.array([0, 1, 7, 8, 1023, 1024, 2047, 4095] + list(range(100, 4000, 397)))
    dyb = inputs.bf16_bits(data.dy)
    _log(f"{wl.name}: oracle on {len(cols)} columns")
    ref, _ = oracle.embedding_bwd_bf16(data.ids, dyb, wl.vocab, cols=cols)
    got = out["dE"][:, cols]
    assert CONTRACT.accuracy_passes(got, ref, "dE")
    want = oracle.edo_v1_f32(data.ids, np.ascontiguousarray(dyb[:, cols]), wl.vocab)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    tb = inputs.bf16_bits(data.table)
    rows = _sample_rows(wl.n_logical)
    assert np.array_equal(out["y"][rows], tb[data.ids[rows]])
    # the one-call backward: every bit of dE as the accumulator path
    acc = binding.EmbeddingDwAccumulator(data.ids, wl.vocab, wl.hidden)
    one = acc.backward(data.dy)
    torch.cuda.synchronize()
    acc.close()
    assert np.array_equal(one.cpu().numpy().view(np.uint32), out["dE"].view(np.uint32))
    _log(f"{wl.name}: sampled columns match, one-call backward bitwise; "
         f"{int((np.bincount(data.ids) > 0).sum())} tokens occur")
