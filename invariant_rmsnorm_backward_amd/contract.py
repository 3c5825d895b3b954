"""The single tolerance contract every comparison goes through.

"[WS1 Closeout][Backward] Reusable gradient-invariance harness and operator
adapters" (Scope and Acceptance criteria) asks that gradient thresholds come
from one resolver only, that invariance be bitwise (atol = 0, rtol = 0) after
logical aggregation, and that only accuracy against a reference VJP use a
tolerance.  ``contract.json`` holds the numbers; nothing else may define one.

Accuracy thresholds: bf16 outputs (dx, y) use rtol 2e-2 with an absolute term
scaled by the reference tensor's max-abs (a literal atol of 2e-2 would be
vacuous for gradients of size ~1/N_active); FP32 dweight uses rtol 1e-5 with
the same scaled absolute term plus a normwise bound; FP32 rstd uses rtol 1e-5.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Dict, Optional

import numpy as np

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "contract.json")


@dataclasses.dataclass(frozen=True)
class AccuracyTolerance:
    rtol: float
    atol_scale: float
    normwise: Optional[float] = None


@dataclasses.dataclass
class ToleranceContract:
    version: str
    invariance_atol: float
    invariance_rtol: float
    accuracy: Dict[str, AccuracyTolerance]

    def accuracy_for(self, tensor: str) -> AccuracyTolerance:
        """Tolerance for a gradient/output name; per-side names such as
        ``dweight_q`` or ``dq`` resolve to their base tensor."""
        base = tensor
        if base.startswith("dweight"):
            base = "dweight"
        elif base in ("dq", "dk"):
            base = "dx"
        elif base in ("yq", "yk"):
            base = "y"
        elif base.startswith("rstd"):
            base = "rstd"
        return self.accuracy[base]

    def accuracy_passes(self, got: np.ndarray, ref: np.ndarray, tensor: str) -> bool:
        tol = self.accuracy_for(tensor)
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        err = np.abs(got - ref)
        ok = bool(np.all(err <= tol.rtol * np.abs(ref) + tol.atol_scale * scale))
        if tol.normwise is not None and ref.size:
            denom = float(np.linalg.norm(ref))
            ok = ok and float(np.linalg.norm(got - ref)) <= tol.normwise * max(denom, 1e-300)
        return ok

    def invariance_passes(self, got_bits: np.ndarray, ref_bits: np.ndarray) -> bool:
        # atol = rtol = 0: the raw bit patterns must be identical
        assert self.invariance_atol == 0.0 and self.invariance_rtol == 0.0
        return got_bits.shape == ref_bits.shape and bool(np.array_equal(got_bits, ref_bits))


def load_contract(path: str = _PATH) -> ToleranceContract:
    with open(path) as f:
        d = json.load(f)
    acc = {k: AccuracyTolerance(v["rtol"], v["atol_scale"], v.get("normwise"))
           for k, v in d["gradient_accuracy"].items() if isinstance(v, dict)}
    inv = d["gradient_invariance"]
    return ToleranceContract(d["version"], float(inv["atol"]), float(inv["rtol"]), acc)
