"""The harness can fail: synthetic CPU operators show that an operator whose
result follows the physical layout is judged red and one that sees only
logical identity green, that the one-call cell really is one call, that
chunked cells really split it and that padding rows reach the operator
("WS1 C4 (#270) closeout evidence", section "The matrix is falsifiable")."""
import numpy as np
import pytest

from invariant_rmsnorm_backward_amd import contract, harness, inputs, layouts

CONTRACT = contract.load_contract()


class _Data:
    def __init__(self, wl):
        self.name = wl.name
        self.wl = wl
        self.x = inputs.gen_x(wl).float().numpy()
        self.dy = inputs.gen_dy(wl).float().numpy()
        self.active_token_denominator = inputs.n_active(wl)


class _SyntheticOp(harness.GradientAdapter):
    """dweight_j = sum over rows of dy*x (FP32), dx = dy (row-local)."""
    name = "synthetic"
    aggregation_order = "synthetic"

    def physical(self, call, data, fill=np.nan):
        return (layouts.gather_physical(data.x, call, fill),
                layouts.gather_physical(data.dy, call, fill))

    def restore(self, call, out_phys, T):
        out = np.zeros((T,) + out_phys.shape[1:], dtype=out_phys.dtype)
        rl = np.arange(call.rows) if call.row_logical is None else call.row_logical
        out[rl[rl >= 0]] = out_phys[rl >= 0]
        return out


class PhysicalChunkLeftFold(_SyntheticOp):
    """The prior-art failure: each call left-folds its rows in physical order,
    and per-call results are added in call order."""
    name = "negative_control_physical_fold"

    def run_cell(self, cell, data):
        T = data.x.shape[0]
        dw = np.zeros(data.x.shape[1], dtype=np.float32)
        dx = np.zeros_like(data.dy)
        for call in cell.calls:
            self.call_log.append((cell.name, call.name, call.rows))
            x, dy = self.physical(call, data)
            part = np.zeros_like(dw)
            rl = np.arange(call.rows) if call.row_logical is None else call.row_logical
            for p in range(call.rows):
                if rl[p] >= 0:
                    part = (part + (dy[p] * x[p]).astype(np.float32)).astype(np.float32)
            dw = (dw + part).astype(np.float32)
            dx += self.restore(call, np.where(rl[:, None] >= 0, dy, 0), T)
        return {"dx": dx.astype(np.float32), "dweight": dw}


class LogicalOrderOp(_SyntheticOp):
    """Contributions keyed by logical row, summed in logical order at the end."""
    name = "logical_identity_only"

    def run_cell(self, cell, data):
        T, H = data.x.shape
        contrib = np.zeros((T, H), dtype=np.float32)
        dx = np.zeros_like(data.dy)
        for call in cell.calls:
            self.call_log.append((cell.name, call.name, call.rows))
            x, dy = self.physical(call, data)
            c = (dy * x).astype(np.float32)
            contrib += self.restore(call, np.nan_to_num(c), T)
            rl = np.arange(call.rows) if call.row_logical is None else call.row_logical
            dx += self.restore(call, np.where(rl[:, None] >= 0, dy, 0), T)
        dw = np.zeros(H, dtype=np.float32)
        for l in range(T):
            dw = (dw + contrib[l]).astype(np.float32)
        return {"dx": dx.astype(np.float32), "dweight": dw}


class LayoutBlindOp(LogicalOrderOp):
    """Ignores the physical layout (runs B=N once per cell): a tautology."""
    name = "layout_blind"

    def run_cell(self, cell, data):
        return super().run_cell(layouts.full(data.wl), data)


class DropsDweightWhenChunked(LogicalOrderOp):
    """Correct everywhere, except that chunked cells return no dweight."""
    name = "drops_dweight_when_chunked"

    def run_cell(self, cell, data):
        out = super().run_cell(cell, data)
        if cell.name.startswith("BN/chunked"):
            del out["dweight"]
        return out


class ExtraTensorWhenChunked(LogicalOrderOp):
    """Correct everywhere, except that chunked cells return a tensor the
    reference cell does not have."""
    name = "extra_tensor_when_chunked"

    def run_cell(self, cell, data):
        out = super().run_cell(cell, data)
        if cell.name.startswith("BN/chunked"):
            out["stray"] = np.zeros(3, dtype=np.float32)
        return out


def _wl():
    return inputs.scaled(inputs.workload_h4096(), "synthetic_h64", hidden=64,
                         lengths=[11, 7, 13, 9, 5, 14])


def test_layout_sensitive_operator_is_red():
    wl = _wl()
    rep = harness.assert_gradient_batch_invariant(
        PhysicalChunkLeftFold(), layouts.page_matrix(wl), CONTRACT, data=_Data(wl),
        raise_on_red=False)
    by = {c.name: c.status for c in rep.cells}
    assert by["BN/chunked"] == harness.RED_VERDICT
    assert by["B1-singleton_aggregate/full"] == harness.RED_VERDICT
    assert by["BN/permuted"] == harness.RED_VERDICT
    assert not rep.strict and rep.first_failure["tensor"] == "dweight"
    # dx is row-local, so it stays bitwise invariant even for this operator
    assert all(v.bitwise_equal for v in rep.invariance_reports if v.tensor == "dx")
    with pytest.raises(harness.GradientInvarianceError) as ei:
        harness.assert_gradient_batch_invariant(PhysicalChunkLeftFold(), layouts.page_matrix(wl),
                                                CONTRACT, data=_Data(wl))
    assert "dweight" in str(ei.value)


def test_logical_identity_operator_is_green_and_calls_are_physical():
    wl = _wl()
    op = LogicalOrderOp()
    cells = layouts.page_matrix(wl)
    rep = harness.assert_gradient_batch_invariant(op, cells, CONTRACT, data=_Data(wl))
    assert rep.strict and all(c.status == harness.GREEN for c in rep.cells)
    calls = {}
    for cname, _, rows in op.call_log:
        calls.setdefault(cname, []).append(rows)
    assert calls["BN/full"] == [59]                          # B=N is one batched call
    assert len(calls["BN/chunked"]) == 10                    # chunking splits it
    assert calls["BN/padded_right"] == [80]                  # padding reaches the op
    assert len(calls["B1-singleton_aggregate/full"]) == 6
    assert rep.active_token_denominator == 59
    assert len(rep.singleton_aggregate_reports) > 0


def test_layout_blind_adapter_is_caught_by_the_call_log():
    wl = _wl()
    op = LayoutBlindOp()
    cells = layouts.page_matrix(wl)
    harness.assert_gradient_batch_invariant(op, cells, CONTRACT, data=_Data(wl))
    rows_seen = sorted({rows for _, _, rows in op.call_log})
    # every call was the full batch: the chunked and padded cells never reached the op
    assert rows_seen == [59]
    assert [c.call_shapes for c in cells if c.name == "BN/chunked"][0] != [59]


def test_unknown_operator_is_a_categorised_red():
    wl = _wl()
    rep = harness.assert_gradient_batch_invariant("fused_logp", [layouts.full(wl)], CONTRACT,
                                                  data=_Data(wl), raise_on_red=False)
    assert rep.cells[0].status == harness.RED_NO_BACKWARD and not rep.strict


def test_adapter_without_backward_is_red_no_backward():
    wl = _wl()
    rep = harness.assert_gradient_batch_invariant(harness.GradientAdapter(), layouts.page_matrix(wl),
                                                  CONTRACT, data=_Data(wl), raise_on_red=False)
    assert {c.status for c in rep.cells} == {harness.RED_NO_BACKWARD}


def test_required_ops_are_enumerable():
    from invariant_rmsnorm_backward_amd import adapters
    assert set(adapters.GRADIENT_ADAPTERS) == {"rms_norm", "rms_norm_recompute", "qk_norm",
                                              "qk_norm_pair", "det_gemm", "rms_norm+det_gemm",
                                              "embedding"}
    for name, cls in adapters.GRADIENT_ADAPTERS.items():
        a = cls()
        assert a.name == name and len(a.grad_names) >= 1 and len(a.forward_names) >= 1


def test_accuracy_and_invariance_are_separate():
    wl = _wl()
    data = _Data(wl)
    ref = {"dweight": (data.dy.astype(np.float64) * data.x).sum(0) * 1.001}   # 0.1% off
    rep = harness.assert_gradient_batch_invariant(LogicalOrderOp(), layouts.page_matrix(wl),
                                                  CONTRACT, data=data, reference=ref,
                                                  raise_on_red=False)
    assert all(c.status == harness.GREEN for c in rep.cells)     # invariance green
    assert [v.passed for v in rep.accuracy_reports] == [False]   # accuracy red
    assert not rep.strict
    assert rep.first_failure["kind"] == "gradient_accuracy"


def test_no_private_thresholds_in_tests():
    import os
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    for f in os.listdir(here):
        if f.startswith("test_gpu") and f.endswith(".py"):
            text = open(os.path.join(here, f)).read()
            assert not re.search(r"assert_allclose|atol\s*=|rtol\s*=", text), f


def test_cli_list_and_blocked_hardware_without_gpu(capsys):
    import torch
    from invariant_rmsnorm_backward_amd import cli
    assert cli.main(["list"]) == 0
    out = capsys.readouterr().out
    assert "rmsnorm_h8_t59" in out and "BN/chunked: 10 call(s), rows 59" in out
    if not torch.cuda.is_available():
        assert cli.main(["sweep", "--workload", "rmsnorm_h8_t59"]) == 1
        assert "blocked_hardware" in capsys.readouterr().out


class _SyntheticChain(_SyntheticOp):
    """Three stages in chain order: a row-local forward, a layout-sensitive
    parameter gradient (left fold in physical order, per call), and a
    row-local input gradient; optionally an earlier layout-sensitive stage."""
    name = "synthetic_chain"
    tensor_order = ("a.y", "a.stat", "b.dW", "c.dx")

    def __init__(self, early_red=False):
        super().__init__()
        self.early_red = early_red

    def run_cell(self, cell, data):
        T, H = data.x.shape
        y = np.zeros_like(data.x)
        dx = np.zeros_like(data.dy)
        dW = np.zeros(H, dtype=np.float32)
        stat = np.zeros(1, dtype=np.float32)
        contrib = np.zeros((T, H), dtype=np.float32)
        for call in cell.calls:
            self.call_log.append((cell.name, call.name, call.rows))
            x, dy = self.physical(call, data)
            rl = np.arange(call.rows) if call.row_logical is None else call.row_logical
            real = rl >= 0
            y += self.restore(call, np.where(real[:, None], 2 * x, 0), T)
            dx += self.restore(call, np.where(real[:, None], dy, 0), T)
            part = np.zeros(H, dtype=np.float32)
            for p in range(call.rows):
                if rl[p] >= 0:
                    part = (part + (dy[p] * x[p]).astype(np.float32)).astype(np.float32)
            dW = (dW + part).astype(np.float32)
            if self.early_red:
                s1 = np.float32(0)
                for p in range(call.rows):
                    if rl[p] >= 0:
                        s1 = np.float32(s1 + np.float32(x[p, 0] * 1e-3))
                stat = (stat + s1).astype(np.float32)
            else:
                contrib += self.restore(call, np.nan_to_num(x[:, :1] * 1e-3).astype(np.float32)
                                        * np.ones((1, H), np.float32), T)
        if not self.early_red:
            s = np.float32(0)
            for l in range(T):
                s = np.float32(s + contrib[l, 0])
            stat[0] = s
        return {"c.dx": dx.astype(np.float32), "b.dW": dW, "a.y": y.astype(np.float32), "a.stat": stat}


def test_chain_drift_is_attributed_to_the_first_drifting_tensor():
    wl = _wl()
    rep = harness.assert_gradient_batch_invariant(_SyntheticChain(), layouts.page_matrix(wl),
                                                  CONTRACT, data=_Data(wl), raise_on_red=False)
    assert rep.chain_attribution["BN/chunked"] == "b.dW"
    assert rep.first_failure["tensor"] == "b.dW"
    by = {c.name: c for c in rep.cells}
    assert by["BN/chunked"].first_drift == "b.dW" and by["BN/full"].first_drift is None
    # an earlier drifting stage takes the attribution, whatever the dict order
    rep2 = harness.assert_gradient_batch_invariant(_SyntheticChain(early_red=True),
                                                   layouts.page_matrix(wl), CONTRACT,
                                                   data=_Data(wl), raise_on_red=False)
    assert rep2.chain_attribution["BN/chunked"] == "a.stat"
    assert "a.y" not in rep2.chain_attribution.values()


@pytest.mark.parametrize("op", [DropsDweightWhenChunked(), ExtraTensorWhenChunked()])
def test_a_missing_or_extra_tensor_is_red(op):
    """A cell that omits a gradient the reference cell has (or returns one it
    lacks) is a red verdict on that tensor, not a green cell or an exception."""
    wl = _wl()
    rep = harness.assert_gradient_batch_invariant(op, layouts.page_matrix(wl), CONTRACT,
                                                  data=_Data(wl), raise_on_red=False)
    by = {c.name: c for c in rep.cells}
    bad = "dweight" if isinstance(op, DropsDweightWhenChunked) else "stray"
    assert by["BN/chunked"].status == harness.RED_VERDICT
    assert by["BN/chunked"].first_drift == bad
    assert by["BN/permuted"].status == harness.GREEN
    assert not rep.strict and rep.first_failure["tensor"] == bad
