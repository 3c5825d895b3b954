"""GPU: the rstd-recompute backward (rmsnorm_bwd_dx_recompute) rebuilds rstd
from x in the forward's order, so dx and dweight are bit for bit those of
rmsnorm_bwd_dx given the forward's saved rstd -- for every kernel shape (lane
groups; one wavefront per row with and without lane masks; two wavefronts per
row, with and without masks) and every layout family of the standard matrix,
padding rows included.  The forward without a saved rstd gives the same y."""
import numpy as np
import pytest
import torch

from invariant_rmsnorm_backward_amd import binding, contract, harness, inputs, layouts
from tests import parity_utils as pu

pytestmark = pytest.mark.gpu
EPS = 1e-6

# hidden: sample lengths (every case spans several 64-row blocks and a ragged tail)
CASES = {
    8: [40, 29], 64: [70, 13], 256: [65, 64], 24: [50, 31], 520: [66, 61], 1024: [64, 77],
    1032: [90, 40], 1536: [70, 70], 2048: [64, 65], 4096: [130, 70], 5120: [77, 64],
    8192: [64, 70], 10240: [65, 20],
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _same(a, b):
    return torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.view(torch.int16 if b.element_size() == 2 else torch.int32))


def _physical(t, call, pad_value):
    """One call's rows of a logical-order device tensor; padding rows hold pad_value."""
    if call.row_logical is None:
        return t
    rl = torch.from_numpy(call.row_logical.astype(np.int64)).to(t.device)
    out = t[rl.clamp(min=0)].clone()
    out[rl < 0] = pad_value
    return out


@pytest.mark.parametrize("hidden", sorted(CASES))
def test_recompute_backward_is_the_saved_rstd_backward(hidden):
    wl = inputs.scaled(inputs.workload_h4096(), f"rc_h{hidden}", hidden=hidden,
                       lengths=CASES[hidden])
    T = wl.n_logical
    x = inputs.gen_x(wl, device="cuda")
    x[3] = 0                                   # a zero row: rstd = eps^-1/2
    w = inputs.gen_w(wl, device="cuda")
    dy = inputs.gen_dy(wl, device="cuda")
    y, rstd = binding.fwd(x, w, EPS)
    y2, none = binding.fwd(x, w, EPS, save_rstd=False)
    assert none is None and _same(y, y2)
    cells = layouts.standard_matrix(wl, chunk=48)
    print(f"[recompute] hidden {hidden}: {T} rows, {len(cells)} cells", flush=True)
    for cell in cells:
        a1, a2 = binding.DwAccumulator(T, hidden), binding.DwAccumulator(T, hidden)
        for call in cell.calls:
            xp = _physical(x, call, float("nan"))       # padding rows must never be read
            dyp = _physical(dy, call, float("nan"))
            rp = _physical(rstd, call, float("nan"))
            lay = None if call.row_logical is None else binding.Layout(call.row_logical, T)
            d1 = binding.bwd(xp, w, dyp, rp, lay, a1)
            d2 = binding.bwd_recompute(xp, w, dyp, EPS, lay, a2)
            assert _same(d1, d2), (cell.name, call.name)
        g1, g2 = a1.finalize(), a2.finalize()
        assert _same(g1, g2), cell.name
        a1.close()
        a2.close()


def test_recompute_with_eps_zero_and_without_accumulator():
    wl = inputs.scaled(inputs.workload_h4096(), "rc_eps0", hidden=4096, lengths=[70, 65])
    x = inputs.gen_x(wl, device="cuda")
    w = inputs.gen_w(wl, device="cuda")
    dy = inputs.gen_dy(wl, device="cuda")
    _, rstd = binding.fwd(x, w, 0.0)
    assert _same(binding.bwd(x, w, dy, rstd), binding.bwd_recompute(x, w, dy, 0.0))


def test_recompute_argument_errors():
    wl = inputs.scaled(inputs.workload_h4096(), "rc_err", hidden=64, lengths=[10])
    x = inputs.gen_x(wl, device="cuda")
    w = inputs.gen_w(wl, device="cuda")
    dx = torch.empty_like(x)
    for eps in (-1.0, float("nan"), float("inf")):
        with pytest.raises(binding.RmsNormError) as ei:
            binding.rmsnorm_bwd_dx_recompute(x.data_ptr(), w.data_ptr(), x.data_ptr(), eps,
                                             dx.data_ptr(), 10, 64, None, None, None)
        assert ei.value.code == binding.EINVAL
    with pytest.raises(binding.RmsNormError) as ei:
        binding.rmsnorm_bwd_dx_recompute(x.data_ptr(), w.data_ptr(), x.data_ptr(), 1e-6, None,
                                         10, 64, None, None, None)
    assert ei.value.code == binding.EINVAL


def test_recompute_adapter_through_the_harness():
    """rms_norm_recompute over every layout family of a padded, permuted,
    masked workload: bitwise invariant and within the contract of the oracle."""
    wl = inputs.scaled(inputs.workload_h5120(), "rc_h5120_small", lengths=[200, 100, 50, 30, 77],
                       pad_rows=150)
    data = pu.make_data(wl)
    ref = pu.oracle_reference(wl)
    ref = {k: v for k, v in ref.items() if k in ("dx", "dweight", "y")}
    cells = pu.standard_cells(wl, 64)
    print(f"[recompute] harness: {len(cells)} cells", flush=True)
    rep = harness.assert_gradient_batch_invariant("rms_norm_recompute", cells,
                                                  contract.load_contract(), data=data,
                                                  reference=ref, raise_on_red=False)
    if not rep.strict:
        print(rep.to_json()[:3000], flush=True)
    assert rep.strict, rep.first_failure
