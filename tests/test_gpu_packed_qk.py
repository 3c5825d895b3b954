"""Per-head norm inside a packed QKV tensor (no copy of Q or K out of it):
every output matches the FP64 oracle within the tolerance contract (also
with a padded, permuted token order inside the packed tensor), every output
bit equals the contiguous path on the extracted rows, the rows of other
heads (V) are never written, and dweight stays bitwise invariant across
layouts of the packed rows."""
import numpy as np
import pytest
import torch

from invariant_rmsnorm_backward_amd import binding, inputs, layouts

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FA5   # a NaN pattern: any write to a V position changes it


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _side(side, lengths):
    return inputs.scaled(inputs.workload_qk(side), f"packed_{side}", lengths=lengths)


def _packed(wq, wk, d, fill=None):
    """qkv[T, (Hq + 2 Hk) d] with the Q and K rows of the workloads in place."""
    T = wq.n_tokens
    hq, hk = wq.heads, wk.heads
    ts = (hq + 2 * hk) * d
    qkv = torch.full((T, ts), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if fill is not None:
        q, k = fill
        qkv[:, : hq * d] = q.view(T, hq * d)
        qkv[:, hq * d: (hq + hk) * d] = k.view(T, hk * d)
    return qkv, ts


@pytest.mark.parametrize("lengths", [[100, 37, 64], [1], [70, 3]])
def test_packed_qk_norm_equals_the_contiguous_path(lengths):
    wq, wk = _side("q", lengths), _side("k", lengths)
    d, T = wq.hidden, wq.n_tokens
    xq, xk = inputs.gen_x(wq, device="cuda"), inputs.gen_x(wk, device="cuda")
    gq, gk = inputs.gen_dy(wq, device="cuda"), inputs.gen_dy(wk, device="cuda")
    wvq, wvk = inputs.gen_w(wq, device="cuda"), inputs.gen_w(wk, device="cuda")
    x, ts = _packed(wq, wk, d, (xq, xk))
    dy, _ = _packed(wq, wk, d, (gq, gk))
    y, _ = _packed(wq, wk, d)
    dx, _ = _packed(wq, wk, d)
    st = binding.current_stream()
    for side, xs, gs, wv, heads, col0 in (("q", xq, gq, wvq, wq.heads, 0),
                                          ("k", xk, gk, wvk, wk.heads, wq.heads * d)):
        rows = T * heads
        # contiguous reference path
        acc_c = binding.DwAccumulator(rows, d)
        yc, rc = binding.fwd(xs, wvq if side == "q" else wvk, wq.eps)
        dxc = binding.bwd(xs, wv, gs, rc, acc=acc_c)
        dwc = acc_c.finalize()
        # packed path
        rp = torch.empty(rows, dtype=torch.float32, device="cuda")
        acc_p = binding.DwAccumulator(rows, d)
        xb, yb, gb, db = (t.view(torch.int16)[:, col0:].view(torch.bfloat16) for t in (x, y, dy, dx))
        binding.rmsnorm_fwd_packed(xb.data_ptr(), wv.data_ptr(), yb.data_ptr(), rp.data_ptr(), T,
                                   heads, d, ts, wq.eps, None, st)
        binding.rmsnorm_bwd_dx_packed(xb.data_ptr(), wv.data_ptr(), gb.data_ptr(), rp.data_ptr(),
                                      db.data_ptr(), T, heads, d, ts, None, acc_p.handle, st)
        dwp = acc_p.finalize()
        torch.cuda.synchronize()
        sl = slice(col0, col0 + heads * d)
        assert torch.equal(y.view(torch.int16)[:, sl].reshape(rows, d), yc.view(torch.int16)), side
        assert torch.equal(dx.view(torch.int16)[:, sl].reshape(rows, d), dxc.view(torch.int16)), side
        assert torch.equal(rp.view(torch.int32), rc.view(torch.int32)), side
        assert torch.equal(dwp.view(torch.int32), dwc.view(torch.int32)), side
        acc_c.close()
        acc_p.close()
    v0 = (wq.heads + wk.heads) * d
    for t in (y, dx):
        assert bool((t.view(torch.int16)[:, v0:] == SENTINEL).all())   # V never written


def test_packed_rows_with_a_layout_are_invariant():
    """Padding tokens and a permuted token order inside the packed tensor:
    the same dweight bits as the plain call, padded rows zero."""
    wq = _side("q", [40, 29])
    d, T, heads = wq.hidden, wq.n_tokens, wq.heads
    xs, gs, wv = inputs.gen_x(wq, device="cuda"), inputs.gen_dy(wq, device="cuda"), inputs.gen_w(wq, device="cuda")
    st = binding.current_stream()
    acc0 = binding.DwAccumulator(T * heads, d)
    _, r0 = binding.fwd(xs, wv, wq.eps)
    binding.bwd(xs, wv, gs, r0, acc=acc0)
    dw0 = acc0.finalize().clone()
    # tokens permuted, 5 padding tokens interleaved; each token keeps its heads together
    perm = np.random.default_rng(3).permutation(T)
    tok = np.concatenate([perm[:20], [-1] * 3, perm[20:], [-1] * 2])
    rl = np.where(tok[:, None] < 0, -1, tok[:, None] * heads + np.arange(heads)[None, :]).reshape(-1)
    P = len(tok)
    ts = heads * d + 64                       # a gap after each token's heads
    x = torch.zeros((P, ts), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros_like(x)
    y = torch.full((P, ts), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dx = y.clone()
    real = tok >= 0
    x[torch.from_numpy(np.nonzero(real)[0]).cuda(), : heads * d] = xs.view(T, heads * d)[torch.from_numpy(tok[real]).cuda()]
    g[torch.from_numpy(np.nonzero(real)[0]).cuda(), : heads * d] = gs.view(T, heads * d)[torch.from_numpy(tok[real]).cuda()]
    lay = binding.Layout(rl.astype(np.int32), T * heads)
    r = torch.empty(P * heads, dtype=torch.float32, device="cuda")
    acc = binding.DwAccumulator(T * heads, d)
    binding.rmsnorm_fwd_packed(x.data_ptr(), wv.data_ptr(), y.data_ptr(), r.data_ptr(), P, heads, d,
                               ts, wq.eps, lay.handle, st)
    binding.rmsnorm_bwd_dx_packed(x.data_ptr(), wv.data_ptr(), g.data_ptr(), r.data_ptr(),
                                  dx.data_ptr(), P, heads, d, ts, lay.handle, acc.handle, st)
    dw = acc.finalize()
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))
    pad = torch.from_numpy(np.nonzero(~real)[0]).cuda()
    assert bool((y.view(torch.int16)[pad, : heads * d] == 0).all())
    assert bool((dx.view(torch.int16)[pad, : heads * d] == 0).all())
    assert bool((y.view(torch.int16)[:, heads * d:] == SENTINEL).all())   # the gap is never written
    lay.close()
    acc.close()
    acc0.close()


def _oracle_side(wl):
    """FP64 oracle of one side (logical rows t * heads + h), from CPU inputs."""
    import oracle
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    gb = inputs.bf16_bits(inputs.gen_dy(wl))
    y, rstd = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    dx, dw, _ = oracle.rmsnorm_bwd_bf16(xb, wb, gb, wl.eps)
    return {"y": y, "rstd": rstd, "dx": dx, "dweight": dw}


@pytest.mark.parametrize("lengths,layout", [([100, 37, 64], "identity"), ([70, 3, 41], "padded_permuted")])
def test_packed_qk_norm_matches_the_oracle(lengths, layout):
    """Q and K inside one packed QKV tensor (32 + 8 + 8 heads of 128), run in
    place, against the FP64 oracle element by element: y, dx (bf16) and
    rstd, dweight_q, dweight_k (FP32) within the tolerance contract, and more
    than 99% of y and dx within one bf16 ulp of FP64.  The padded, permuted
    case puts the tokens in a seeded order with padding tokens between them
    inside the packed tensor; its outputs are gathered back to logical order."""
    from tests import parity_utils as pu
    from invariant_rmsnorm_backward_amd import contract
    con = contract.load_contract()
    wq, wk = _side("q", lengths), _side("k", lengths)
    d, T = wq.hidden, wq.n_tokens
    hq, hk = wq.heads, wk.heads
    if layout == "identity":
        tok = np.arange(T)
    else:
        perm = np.random.default_rng(11).permutation(T)
        tok = np.concatenate([[-1] * 2, perm[: T // 2], [-1] * 5, perm[T // 2:], [-1]])
    P = len(tok)
    real = tok >= 0
    ts = (hq + 2 * hk) * d
    st = binding.current_stream()
    phys = torch.from_numpy(np.nonzero(real)[0]).cuda()
    logi = torch.from_numpy(tok[real]).cuda()

    def packed(q, k):
        t = torch.zeros((P, ts), dtype=torch.bfloat16, device="cuda")
        t[phys, : hq * d] = q.view(T, hq * d)[logi]
        t[phys, hq * d: (hq + hk) * d] = k.view(T, hk * d)[logi]
        return t

    x = packed(inputs.gen_x(wq, device="cuda"), inputs.gen_x(wk, device="cuda"))
    dy = packed(inputs.gen_dy(wq, device="cuda"), inputs.gen_dy(wk, device="cuda"))
    y = torch.full((P, ts), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dx = y.clone()
    inv = np.empty(T, dtype=np.int64)
    inv[tok[real]] = np.nonzero(real)[0]
    for side, wl, heads, col0 in (("q", wq, hq, 0), ("k", wk, hk, hq * d)):
        ref = _oracle_side(wl)
        wv = inputs.gen_w(wl, device="cuda")
        rows_log = T * heads
        rl = np.where(tok[:, None] < 0, -1, tok[:, None] * heads + np.arange(heads)[None, :]).reshape(-1)
        lay = None if layout == "identity" else binding.Layout(rl.astype(np.int32), rows_log)
        r = torch.empty(P * heads, dtype=torch.float32, device="cuda")
        acc = binding.DwAccumulator(rows_log, d)
        xb, yb, gb, db = (t.view(torch.int16)[:, col0:].view(torch.bfloat16) for t in (x, y, dy, dx))
        lh = None if lay is None else lay.handle
        binding.rmsnorm_fwd_packed(xb.data_ptr(), wv.data_ptr(), yb.data_ptr(), r.data_ptr(), P,
                                   heads, d, ts, wl.eps, lh, st)
        binding.rmsnorm_bwd_dx_packed(xb.data_ptr(), wv.data_ptr(), gb.data_ptr(), r.data_ptr(),
                                      db.data_ptr(), P, heads, d, ts, lh, acc.handle, st)
        dw = acc.finalize()
        torch.cuda.synchronize()
        # gather the physical outputs to logical row order t * heads + h
        sl = slice(col0, col0 + heads * d)
        order = torch.from_numpy(inv).cuda()
        y_log = y.view(torch.int16)[:, sl][order].reshape(rows_log, d).cpu().numpy().view(np.uint16)
        dx_log = dx.view(torch.int16)[:, sl][order].reshape(rows_log, d).cpu().numpy().view(np.uint16)
        r_log = r.view(P, heads)[order].reshape(rows_log).cpu().numpy()
        got = {"y": (y_log.astype(np.uint32) << 16).view(np.float32).astype(np.float64),
               "dx": (dx_log.astype(np.uint32) << 16).view(np.float32).astype(np.float64),
               "rstd": r_log.astype(np.float64), "dweight": dw.cpu().numpy().astype(np.float64)}
        names = {"y": f"y{side}", "dx": f"d{side}", "rstd": f"rstd_{side}", "dweight": f"dweight_{side}"}
        for t in ("y", "dx", "rstd", "dweight"):
            assert con.accuracy_passes(got[t], ref[t], names[t]), (side, layout, t)
        for t, bits in (("y", y_log), ("dx", dx_log)):
            frac = pu.bf16_ulp_fraction(bits, ref[t])
            print(f"[packed-qk] {side} {layout}: {t} within 1 bf16 ulp of FP64: {frac:.5f}", flush=True)
            assert frac > 0.99, (side, layout, t, frac)
        if not real.all():
            pad = torch.from_numpy(np.nonzero(~real)[0]).cuda()
            assert bool((y.view(torch.int16)[pad, sl] == 0).all())
            assert bool((dx.view(torch.int16)[pad, sl] == 0).all())
        acc.close()
        if lay is not None:
            lay.close()
    v0 = (hq + hk) * d
    for t in (y, dx):
        assert bool((t.view(torch.int16)[:, v0:] == SENTINEL).all())   # V never written


@pytest.mark.parametrize("lengths,layout", [([100, 37, 64], "identity"), ([70, 3, 41], "padded_permuted")])
def test_packed_pair_launch_equals_two_calls_and_the_oracle(lengths, layout):
    """rmsnorm_fwd_packed_pair / rmsnorm_bwd_dx_packed_pair run Q and K in one
    launch each: y, rstd, dx and both dweights bit for bit those of the two
    single packed calls, V never written, and the pair's outputs against the
    FP64 oracle (tolerance contract and the one-ulp gate)."""
    from tests import parity_utils as pu
    from invariant_rmsnorm_backward_amd import contract
    con = contract.load_contract()
    wq, wk = _side("q", lengths), _side("k", lengths)
    d, T = wq.hidden, wq.n_tokens
    hq, hk = wq.heads, wk.heads
    if layout == "identity":
        tok = np.arange(T)
    else:
        perm = np.random.default_rng(12).permutation(T)
        tok = np.concatenate([[-1] * 3, perm[: T // 3], [-1] * 4, perm[T // 3:], [-1] * 2])
    P = len(tok)
    real = tok >= 0
    ts = (hq + 2 * hk) * d
    st = binding.current_stream()
    phys = torch.from_numpy(np.nonzero(real)[0]).cuda()
    logi = torch.from_numpy(tok[real]).cuda()

    def packed(q, k):
        t = torch.zeros((P, ts), dtype=torch.bfloat16, device="cuda")
        t[phys, : hq * d] = q.view(T, hq * d)[logi]
        t[phys, hq * d: (hq + hk) * d] = k.view(T, hk * d)[logi]
        return t

    x = packed(inputs.gen_x(wq, device="cuda"), inputs.gen_x(wk, device="cuda"))
    dy = packed(inputs.gen_dy(wq, device="cuda"), inputs.gen_dy(wk, device="cuda"))
    sides = (("q", wq, hq, 0), ("k", wk, hk, hq * d))
    ws = {s: inputs.gen_w(wl, device="cuda") for s, wl, _, _ in sides}
    lays = {}
    for s, wl, heads, _ in sides:
        rl = np.where(tok[:, None] < 0, -1, tok[:, None] * heads + np.arange(heads)[None, :]).reshape(-1)
        lays[s] = None if layout == "identity" else binding.Layout(rl.astype(np.int32), T * heads)
    lh = {s: (None if lays[s] is None else lays[s].handle) for s in lays}
    col = lambda t, c0: t.view(torch.int16)[:, c0:].view(torch.bfloat16)
    out = {}
    for mode in ("single", "pair"):
        y = torch.full((P, ts), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        dx = y.clone()
        r = {s: torch.empty(P * h, dtype=torch.float32, device="cuda") for s, _, h, _ in sides}
        acc = {s: binding.DwAccumulator(T * h, d) for s, _, h, _ in sides}
        if mode == "single":
            for s, wl, heads, c0 in sides:
                binding.rmsnorm_fwd_packed(col(x, c0).data_ptr(), ws[s].data_ptr(), col(y, c0).data_ptr(),
                                           r[s].data_ptr(), P, heads, d, ts, wl.eps, lh[s], st)
                binding.rmsnorm_bwd_dx_packed(col(x, c0).data_ptr(), ws[s].data_ptr(),
                                              col(dy, c0).data_ptr(), r[s].data_ptr(),
                                              col(dx, c0).data_ptr(), P, heads, d, ts, lh[s],
                                              acc[s].handle, st)
        else:
            fa = [(col(x, c0).data_ptr(), ws[s].data_ptr(), col(y, c0).data_ptr(), r[s].data_ptr(),
                   heads, ts, lh[s]) for s, _, heads, c0 in sides]
            binding.rmsnorm_fwd_packed_pair(fa[0], fa[1], P, d, wq.eps, st)
            ba = [(col(x, c0).data_ptr(), ws[s].data_ptr(), col(dy, c0).data_ptr(), r[s].data_ptr(),
                   col(dx, c0).data_ptr(), heads, ts, lh[s], acc[s].handle) for s, _, heads, c0 in sides]
            binding.rmsnorm_bwd_dx_packed_pair(ba[0], ba[1], P, d, st)
        dw = {s: acc[s].finalize() for s in acc}
        torch.cuda.synchronize()
        out[mode] = (y, dx, r, dw)
        for a in acc.values():
            a.close()
    (y1, dx1, r1, dw1), (y2, dx2, r2, dw2) = out["single"], out["pair"]
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    for s in ("q", "k"):
        assert torch.equal(r1[s].view(torch.int32), r2[s].view(torch.int32)), s
        assert torch.equal(dw1[s].view(torch.int32), dw2[s].view(torch.int32)), s
    v0 = (hq + hk) * d
    for t in (y2, dx2):
        assert bool((t.view(torch.int16)[:, v0:] == SENTINEL).all())   # V never written
    # the pair against the oracle, in logical row order t * heads + h
    inv = np.empty(T, dtype=np.int64)
    inv[tok[real]] = np.nonzero(real)[0]
    order = torch.from_numpy(inv).cuda()
    for s, wl, heads, c0 in sides:
        ref = _oracle_side(wl)
        rows_log = T * heads
        sl = slice(c0, c0 + heads * d)
        y_log = y2.view(torch.int16)[:, sl][order].reshape(rows_log, d).cpu().numpy().view(np.uint16)
        dx_log = dx2.view(torch.int16)[:, sl][order].reshape(rows_log, d).cpu().numpy().view(np.uint16)
        got = {"y": (y_log.astype(np.uint32) << 16).view(np.float32).astype(np.float64),
               "dx": (dx_log.astype(np.uint32) << 16).view(np.float32).astype(np.float64),
               "rstd": r2[s].view(P, heads)[order].reshape(rows_log).cpu().numpy().astype(np.float64),
               "dweight": dw2[s].cpu().numpy().astype(np.float64)}
        names = {"y": f"y{s}", "dx": f"d{s}", "rstd": f"rstd_{s}", "dweight": f"dweight_{s}"}
        for t in ("y", "dx", "rstd", "dweight"):
            assert con.accuracy_passes(got[t], ref[t], names[t]), (s, layout, t)
        for t, bits in (("y", y_log), ("dx", dx_log)):
            assert pu.bf16_ulp_fraction(bits, ref[t]) > 0.99, (s, layout, t)
    print(f"[packed-pair] {layout}: pair launch == two calls bitwise, oracle within contract", flush=True)
    for lay in lays.values():
        if lay is not None:
            lay.close()
