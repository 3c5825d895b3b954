"""Per-head norm inside a packed QKV tensor (no copy of Q or K out of it):
every output bit equals the contiguous path on the extracted rows, the
rows of other heads (V) are never written, and dweight stays bitwise
invariant across layouts of the packed rows."""
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
