"""rmsnorm_bwd_noalloc (the allocation-free one-call backward) against the
accumulator path it stands in for: rmsnorm_bwd_dx with an accumulator, then
rmsnorm_dw_finalize, on the same inputs.  dx and dweight must be equal bit
for bit, on two calls in a row on one stream (the second with a smaller
input, so that it runs over scratch the first call left behind) and for
every kernel path (fused, two-pass, small hidden)."""
import dataclasses

import pytest
import torch

from invariant_rmsnorm_backward_amd import binding, inputs

pytestmark = pytest.mark.gpu


def _data(rows, hidden, seed):
    wl = dataclasses.replace(inputs.scaled(inputs.workload_h4096(), f"noalloc_h{hidden}_t{rows}",
                                           hidden=hidden, lengths=[rows]), seed=seed)
    x = inputs.gen_x(wl, device="cuda")
    w = inputs.gen_w(wl, device="cuda")
    dy = inputs.gen_dy(wl, device="cuda")
    _, rstd = binding.fwd(x, w, wl.eps)
    return x, w, dy, rstd


def _reference(x, w, dy, rstd):
    rows, hidden = x.shape
    acc = binding.DwAccumulator(rows, hidden)
    dx = binding.bwd(x, w, dy, rstd, acc=acc)
    dw = acc.finalize()
    torch.cuda.synchronize()
    acc.close()
    return dx, dw


def _noalloc(x, w, dy, rstd):
    rows, hidden = x.shape
    dx = torch.empty_like(x)
    dw = torch.empty(hidden, dtype=torch.float32, device="cuda")
    binding.rmsnorm_bwd_noalloc(x.data_ptr(), w.data_ptr(), dy.data_ptr(), rstd.data_ptr(),
                                dx.data_ptr(), dw.data_ptr(), rows, hidden,
                                binding.current_stream())
    return dx, dw


def _same(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("first,second", [
    ((8192, 4096), (3000, 4096)),      # fused, then 47 blocks over the same scratch (two-pass
                                       # here, stream-owner in the accumulator reference)
    ((6400, 8192), (700, 1024)),       # wide fused, then a narrower shape
    ((20000, 128), (333, 64)),         # small-hidden kernel
])
def test_noalloc_equals_the_accumulator_path_on_two_calls_in_a_row(first, second):
    binding.load()
    runs = []
    for k, (rows, hidden) in enumerate((first, second)):
        data = _data(rows, hidden, 0x5A110C00 + k)
        got = _noalloc(*data)
        torch.cuda.synchronize()
        want = _reference(*data)
        runs.append((got, want))
    for (got_dx, got_dw), (want_dx, want_dw) in runs:
        assert _same(got_dx, want_dx)
        assert _same(got_dw, want_dw)


def test_noalloc_at_the_full_headline_size_and_empty_input():
    binding.load()
    x, w, dy, rstd = _data(32768, 4096, 0x5A110C10)
    got_dx, got_dw = _noalloc(x, w, dy, rstd)
    torch.cuda.synchronize()
    want_dx, want_dw = _reference(x, w, dy, rstd)
    assert _same(got_dx, want_dx) and _same(got_dw, want_dw)
    # rows == 0: dweight of the empty multiset is +0.0
    dw = torch.full((4096,), 7.0, dtype=torch.float32, device="cuda")
    binding.rmsnorm_bwd_noalloc(0, w.data_ptr(), 0, 0, 0, dw.data_ptr(), 0, 4096,
                                binding.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(dw.view(torch.int32), torch.zeros(4096, dtype=torch.int32, device="cuda"))
