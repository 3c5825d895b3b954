"""Gradient-invariance harness: ``assert_gradient_batch_invariant``.

Shape of the API and semantics follow "[WS1 Closeout][Backward] Reusable
gradient-invariance harness and operator adapters" (Suggested API, Scope,
Acceptance criteria) and "WS1 C4 (#270) closeout evidence" (Acceptance map,
"The matrix is falsifiable"):

  * one comparison semantic: the upstream gradient, loss reduction,
    active-token denominator and aggregation order are fixed by the caller's
    logical inputs and recorded in the report, never invented per test;
  * accuracy (against a reference VJP supplied by the caller) is reported
    separately from invariance (across layouts of the same logical rows);
  * invariance is bitwise after logical aggregation; accuracy uses the
    tolerance contract; there are no private thresholds;
  * adapters run the operator on each cell's *physical* layout and restore
    token gradients to logical order through the cell's row map; the call log
    proves that B=N is one call, that chunking splits it and that padding
    reaches the operator;
  * diagnostics per named gradient: max abs / max rel / mean / p99 drift and
    the first failing op / tensor / cell; for a multi-op chain the adapter
    lists its tensors in chain order and every red cell is attributed to the
    first tensor that drifts ("Phase 4: Add single-card operator comparisons
    and drift attribution", Scope);
  * an op without a backward is a categorised red (``red_no_backward``), not a
    stack trace; the report's ``strict`` flag is set only when every cell is
    green.

The harness computes none of RMSNorm's arithmetic: adapters call the HIP
library, and the reference for accuracy is handed in by the caller.
"""
from __future__ import annotations

import dataclasses
import json
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from .contract import ToleranceContract
from .layouts import Cell

GREEN, RED_VERDICT, RED_NO_BACKWARD, BLOCKED_HARDWARE, SKIPPED = (
    "green", "red_verdict", "red_no_backward", "blocked_hardware", "skipped")


class MissingBackwardError(RuntimeError):
    """The operator exposes no backward for a required gradient."""


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class TensorVerdict:
    op: str
    tensor: str
    kind: str                    # "gradient_invariance" | "gradient_accuracy"
    config: str                  # the cell compared (vs the reference cell or the reference VJP)
    passed: bool
    bitwise_equal: bool
    n_mismatch: int
    max_abs: float
    max_rel: float
    mean_abs: float
    p99_abs: float


@dataclasses.dataclass
class CellResult:
    name: str
    status: str
    call_rows: List[int]
    n_pad_rows: int
    verdicts: List[TensorVerdict] = dataclasses.field(default_factory=list)
    first_drift: Optional[str] = None   # first differing tensor in the adapter's tensor order


@dataclasses.dataclass
class GradientInvarianceReport:
    op: str
    workload: str
    reference_cell: str
    loss_reduction: str
    active_token_denominator: int
    aggregation_order: str
    contract_version: str
    accuracy_reports: List[TensorVerdict]
    invariance_reports: List[TensorVerdict]
    singleton_aggregate_reports: List[TensorVerdict]
    cells: List[CellResult]
    first_failure: Optional[dict]
    strict: bool
    provenance: dict
    chain_attribution: Dict[str, str] = dataclasses.field(default_factory=dict)

    def to_json(self) -> str:
        return json.dumps(dataclasses.asdict(self), indent=1, default=float)

    @property
    def green(self) -> bool:
        return all(c.status in (GREEN, SKIPPED) for c in self.cells) and all(
            v.passed for v in self.accuracy_reports)


class GradientInvarianceError(AssertionError):
    def __init__(self, report: GradientInvarianceReport):
        ff = report.first_failure or {}
        super().__init__(
            f"gradient invariance red for op={ff.get('op')} tensor={ff.get('tensor')} "
            f"config={ff.get('config')} ({ff.get('kind')}): max_abs={ff.get('max_abs')}")
        self.report = report


# ------------------------------------------------------------------ adapters
class GradientAdapter:
    """Runs one operator on every call of a cell and returns its outputs in
    logical order: bf16 tensors as raw uint16 bits, FP32 tensors as float32.

    ``call_log`` records (cell, call, rows) for every operator invocation."""
    name = "abstract"
    grad_names: Sequence[str] = ()
    forward_names: Sequence[str] = ()

    def __init__(self):
        self.call_log: List[tuple] = []

    def run_cell(self, cell: Cell, data) -> Dict[str, np.ndarray]:
        raise MissingBackwardError(f"{self.name} has no backward")

    def provenance(self) -> dict:
        return {}


def _drift(got: np.ndarray, ref: np.ndarray, float_view: Callable) -> dict:
    g = float_view(got).astype(np.float64)
    r = float_view(ref).astype(np.float64)
    d = np.abs(g - r)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(r != 0, d / np.abs(r), np.where(d == 0, 0.0, np.inf))
    finite = d[np.isfinite(d)]
    return dict(max_abs=float(np.nanmax(d)) if d.size else 0.0,
                max_rel=float(np.nanmax(rel)) if rel.size else 0.0,
                mean_abs=float(finite.mean()) if finite.size else 0.0,
                p99_abs=float(np.percentile(finite, 99)) if finite.size else 0.0)


def _float_view(arr: np.ndarray):
    return bf16_bits_to_f32 if arr.dtype == np.uint16 else (lambda a: a)


def _bits(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return arr
    if arr.dtype == np.float32:
        return arr.view(np.uint32)
    if arr.dtype == np.float64:
        return arr.view(np.uint64)
    return arr


def assert_gradient_batch_invariant(op, configs: Sequence[Cell], contract: ToleranceContract, *,
                                    data, reference: Optional[Dict[str, np.ndarray]] = None,
                                    reference_cell: str = "BN/full",
                                    raise_on_red: bool = True) -> GradientInvarianceReport:
    """Runs ``op`` on every cell of ``configs`` and compares.

    op         : adapter name registered in ``GRADIENT_ADAPTERS`` or an adapter
    configs    : cells (physical layouts) of one logical row multiset
    contract   : the tolerance contract (the only source of thresholds)
    data       : the logical inputs the adapter needs (see the adapters)
    reference  : expected outputs in logical order from a reference VJP, for
                 the accuracy reports (optional)
    Returns the report if every required cell is green, else raises
    ``GradientInvarianceError`` carrying the report (unless raise_on_red=False).
    """
    from . import adapters  # registry lives next to the HIP adapters
    if isinstance(op, str):
        factory = adapters.GRADIENT_ADAPTERS.get(op)
        adapter = factory() if factory is not None else None
        op_name = op
    else:
        adapter, op_name = op, op.name
    workload = getattr(data, "name", "?")
    denom = int(getattr(data, "active_token_denominator", 0))

    cells_out: List[CellResult] = []
    inv: List[TensorVerdict] = []
    acc: List[TensorVerdict] = []
    first = None

    def note(v: TensorVerdict):
        nonlocal first
        if not v.passed and first is None:
            first = dataclasses.asdict(v)

    names = [c.name for c in configs]
    if reference_cell not in names:
        raise ValueError(f"reference cell {reference_cell!r} missing from configs")

    if adapter is None:
        for c in configs:
            cells_out.append(CellResult(c.name, RED_NO_BACKWARD, c.call_shapes,
                                        sum(k.n_pad for k in c.calls)))
        first = dict(op=op_name, tensor=None, config=names[0], kind="red_no_backward",
                     max_abs=None)
        report = GradientInvarianceReport(op_name, workload, reference_cell, "?", denom, "?",
                                          contract.version, [], [], [], cells_out, first, False, {})
        if raise_on_red:
            raise GradientInvarianceError(report)
        return report

    results: Dict[str, Dict[str, np.ndarray]] = {}
    status: Dict[str, str] = {}
    for c in configs:
        try:
            results[c.name] = adapter.run_cell(c, data)
            status[c.name] = GREEN
        except MissingBackwardError:
            status[c.name] = RED_NO_BACKWARD
            if first is None:
                first = dict(op=op_name, tensor=None, config=c.name, kind="red_no_backward",
                             max_abs=None)

    ref = results.get(reference_cell)
    order = list(getattr(adapter, "tensor_order", ()) or [])
    attribution: Dict[str, str] = {}
    for c in configs:
        cr = CellResult(c.name, status[c.name], c.call_shapes, sum(k.n_pad for k in c.calls))
        if c.name != reference_cell and status[c.name] == GREEN and ref is not None:
            got_all = results[c.name]
            # every tensor either cell produced: one the other lacks is a drift
            # (a layout that drops a gradient must not be judged green)
            names = list(ref) + [t for t in got_all if t not in ref]
            names_in_order = [t for t in order if t in names] + [t for t in names if t not in order]
            for t in names_in_order:
                if t not in got_all or t not in ref:
                    v = TensorVerdict(op_name, t, "gradient_invariance", c.name, False, False, -1,
                                      max_abs=float("inf"), max_rel=float("inf"),
                                      mean_abs=float("inf"), p99_abs=float("inf"))
                    cr.verdicts.append(v)
                    inv.append(v)
                    note(v)
                    cr.status = RED_VERDICT
                    if cr.first_drift is None:
                        cr.first_drift = t
                        attribution[c.name] = t
                    continue
                got = got_all[t]
                want = ref[t]
                same = contract.invariance_passes(_bits(got), _bits(want))
                if same:   # bitwise equal: every drift statistic is exactly 0
                    mism, drift = 0, dict(max_abs=0.0, max_rel=0.0, mean_abs=0.0, p99_abs=0.0)
                else:
                    mism = int(np.sum(_bits(got) != _bits(want))) if got.shape == want.shape else -1
                    drift = _drift(got, want, _float_view(got)) if got.shape == want.shape else \
                        dict(max_abs=float("inf"), max_rel=float("inf"), mean_abs=float("inf"),
                             p99_abs=float("inf"))
                v = TensorVerdict(op_name, t, "gradient_invariance", c.name, same, same, mism, **drift)
                cr.verdicts.append(v)
                inv.append(v)
                note(v)
                if not same:
                    cr.status = RED_VERDICT
                    if cr.first_drift is None:
                        cr.first_drift = t
                        attribution[c.name] = t
        cells_out.append(cr)

    if reference is not None and ref is not None:
        for t, want in reference.items():
            if t not in ref:
                continue
            got = ref[t]
            g = _float_view(got)(got).astype(np.float64)
            ok = contract.accuracy_passes(g, want, t)
            d = _drift(g, np.asarray(want, dtype=np.float64), lambda a: a)
            v = TensorVerdict(op_name, t, "gradient_accuracy", "reference_vjp", ok, False, -1, **d)
            acc.append(v)
            note(v)

    singleton = [v for v in inv if v.config.startswith("B1-singleton")]
    strict = all(c.status == GREEN for c in cells_out) and all(v.passed for v in acc)
    report = GradientInvarianceReport(
        op=op_name, workload=workload, reference_cell=reference_cell,
        loss_reduction=getattr(data, "loss_reduction", "mean_over_active_tokens"),
        active_token_denominator=denom,
        aggregation_order=getattr(adapter, "aggregation_order", "?"),
        contract_version=contract.version, accuracy_reports=acc, invariance_reports=inv,
        singleton_aggregate_reports=singleton, cells=cells_out, first_failure=first,
        strict=strict, provenance=adapter.provenance(), chain_attribution=attribution)
    if raise_on_red and not strict:
        raise GradientInvarianceError(report)
    return report
