"""GPU: a whole step -- every call's forward and backward into one dweight
accumulator, then the finalize -- captured once in a HIP graph (through
torch.cuda.graph, on the capturing stream) and replayed.  Every replay,
with eager work and synchronisations between the replays, gives the bits of
the same step run eagerly.  The calls enqueue kernels only; a finalize with
blocks split across calls also uploads its spill list and is not captured
here, so the chunks hold whole 64-row blocks."""
import numpy as np
import pytest
import torch

from invariant_rmsnorm_backward_amd import binding, inputs, layouts
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


# (hidden, chunk sizes over the 6144 rows): the two-pass one-launch backward
# (12 calls of 8 blocks), the fused backward with a layout (one call of 96
# blocks; resident block owners at hidden 4096), two calls of 48 blocks at
# hidden 5120, and the lane-group kernels of the per-head norm.
# The last case rebuilds rstd in the backward (no saved statistic; those
# calls always take the fused kernel).
CASES = [(4096, [512] * 12, False), (4096, [6144], False), (5120, [3072, 3072], False),
         (128, [1024] * 6, False), (4096, [512] * 12, True)]


@pytest.mark.parametrize("H,sizes,recompute", CASES)
def test_graph_replay_of_a_chunked_step_matches_eager(H, sizes, recompute):
    wl = inputs.scaled(inputs.workload_h4096(), f"graph_h{H}", hidden=H, lengths=[3072, 2048, 1024])
    data = pu.make_data(wl)
    T = wl.n_logical
    cell = layouts.chunked_packed(wl, sizes)
    assert all(c.rows % 64 == 0 for c in cell.calls)          # whole blocks: no spills
    calls = []
    for c in cell.calls:
        a, b = int(c.row_logical[0]), int(c.row_logical[-1]) + 1
        calls.append(dict(x=data.x[a:b], dy=data.dy[a:b], y=torch.empty_like(data.x[a:b]),
                          rstd=torch.empty(b - a, dtype=torch.float32, device="cuda"),
                          dx=torch.empty_like(data.x[a:b]), lay=binding.Layout(c.row_logical, T)))

    def step(acc, dw):
        for c in calls:
            binding.fwd(c["x"], data.w, data.eps, c["lay"], y=c["y"], rstd=c["rstd"])
            if recompute:
                binding.bwd_recompute(c["x"], data.w, c["dy"], data.eps, c["lay"], acc, dx=c["dx"])
            else:
                binding.bwd(c["x"], data.w, c["dy"], c["rstd"], c["lay"], acc, dx=c["dx"])
        acc.finalize(dweight=dw)

    # eager reference
    acc_e = binding.DwAccumulator(T, H)
    dw_e = torch.empty(H, dtype=torch.float32, device="cuda")
    step(acc_e, dw_e)
    torch.cuda.synchronize()
    ref = [(_bits(c["y"]), _bits(c["rstd"]), _bits(c["dx"])) for c in calls] + [_bits(dw_e)]

    # capture (after a warm-up step on the same accumulator, reset)
    acc_g = binding.DwAccumulator(T, H)
    dw_g = torch.empty(H, dtype=torch.float32, device="cuda")
    step(acc_g, dw_g)
    acc_g.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(acc_g, dw_g)
    torch.cuda.synchronize()
    print(f"[graph] H={H}: {len(calls)} calls captured", flush=True)

    for rep in range(3):
        for c in calls:                                   # clear the outputs eagerly
            c["y"].zero_()
            c["rstd"].zero_()
            c["dx"].zero_()
        dw_g.zero_()
        acc_e.reset()                                     # eager work between the replays
        step(acc_e, dw_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [(_bits(c["y"]), _bits(c["rstd"]), _bits(c["dx"])) for c in calls] + [_bits(dw_g)]
        for i, (a, b) in enumerate(zip(ref[:-1], got[:-1])):
            for name, u, v in zip(("y", "rstd", "dx"), a, b):
                assert torch.equal(u, v), (H, rep, i, name)
        assert torch.equal(ref[-1], got[-1]), (H, rep, "dweight")
    del g
    for c in calls:
        c["lay"].close()
    acc_e.close()
    acc_g.close()


def test_finalize_with_split_blocks_is_refused_under_capture():
    """A finalize that has spilled blocks to rebuild uploads their list from a
    pinned host buffer; under stream capture it returns RMSNORM_EUNSUPPORTED
    (nothing is recorded), and the same finalize outside the capture gives
    the one-call dweight bits."""
    H = 4096
    wl = inputs.scaled(inputs.workload_h4096(), "graph_split_h4096", hidden=H, lengths=[100, 60])
    data = pu.make_data(wl)
    T = wl.n_logical
    cell = layouts.chunked_packed(wl, [100, 60])              # block 1 is split across the calls
    acc = binding.DwAccumulator(T, H)
    lays = []
    for c in cell.calls:
        a, b = int(c.row_logical[0]), int(c.row_logical[-1]) + 1
        lay = binding.Layout(c.row_logical, T)
        lays.append(lay)
        _, r = binding.fwd(data.x[a:b], data.w, data.eps, lay)
        binding.bwd(data.x[a:b], data.w, data.dy[a:b], r, lay, acc)
    torch.cuda.synchronize()
    dw = torch.empty(H, dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(g):
        dw.zero_()
        try:
            acc.finalize(dweight=dw)
        except binding.RmsNormError as e:
            refused = e
    torch.cuda.synchronize()
    assert refused is not None and refused.code == binding.EUNSUPPORTED, refused
    acc.finalize(dweight=dw)                                   # outside the capture
    acc1 = binding.DwAccumulator(T, H)
    _, r1 = binding.fwd(data.x, data.w, data.eps)
    binding.bwd(data.x, data.w, data.dy, r1, acc=acc1)
    dw1 = acc1.finalize()
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), dw1.view(torch.int32))
    del g
    for lay in lays:
        lay.close()
    acc.close()
    acc1.close()
