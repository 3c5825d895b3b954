"""Command line: list workloads, check one cell, or sweep a workload's cells.

    python -m invariant_rmsnorm_backward_amd.cli list
    python -m invariant_rmsnorm_backward_amd.cli check --workload rmsnorm_h8_t59 --cell BN/chunked
    python -m invariant_rmsnorm_backward_amd.cli sweep [--workload NAME ...] [--small] [--json FILE]

A sweep runs the operator (RMSNorm, QK-norm, the linear layer, or the
RMSNorm -> linear chain) on every cell of the workload through the HIP
library and classifies each cell (green / red_verdict / red_no_backward /
blocked_hardware / skipped) against the B=N reference cell, bitwise.  It
exits non-zero unless every non-skipped cell is green ("WS1 C4 (#270)
closeout evidence", Runtime verification); a red cell of a chain names the
first tensor, in chain order, that drifts.  Without a GPU every cell is
blocked_hardware: nothing falls back to another implementation.  Accuracy
against a reference VJP is the test suite's job (it needs the oracle).
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import List

from . import contract, harness, inputs, layouts

SMALL = {  # reduced lengths for quick sweeps (same recipe and seed)
    "rmsnorm_h4096_t32768": dict(lengths=[300, 257, 150]),
    "rmsnorm_h8192_varlen16": dict(lengths=[130, 333, 61]),
    "qknorm_d128_t16384_q": dict(lengths=[100, 37, 64]),
    "qknorm_d128_t16384_k": dict(lengths=[100, 37, 64]),
    "rmsnorm_h5120_packed131072": dict(lengths=[200, 100, 50, 30, 77], pad_rows=150),
    "linear_h4096_o4096_t32768": dict(hidden=256, out_features=384, lengths=[300, 257, 150]),
}
# Multi-op targets: a linear workload run behind an RMSNorm of its input width.
CHAINS = {"chain_rmsnorm_linear_h4096_o4096_t32768": "linear_h4096_o4096_t32768"}
CHUNK = {"rmsnorm_h8_t59": 7, "qknorm": 512}
# An RMSNorm workload name with this suffix runs the rstd-recompute backward.
RECOMPUTE = "+recompute"
# The per-head workload with this suffix runs Q and K in one launch per phase.
PAIR = "+pair"


def _workload(name: str, small: bool) -> inputs.Workload:
    wl = (inputs.ALL_WORKLOADS.get(name) or inputs.LINEAR_WORKLOADS[name])()
    if small and name in SMALL:
        wl = inputs.scaled(wl, wl.name + "_small", **SMALL[name])
    return wl


def _cells(wl: inputs.Workload) -> List[layouts.Cell]:
    if wl.name == "rmsnorm_h8_t59":
        return layouts.page_matrix(wl)
    return layouts.standard_matrix(wl, chunk=64 if wl.n_tokens < 4096 else 512)


def _gpu() -> bool:
    import torch
    return torch.cuda.is_available()


def _run(op_name: str, wls, cells_by_side, names=None):
    """Runs one op over its cells; returns the report (or a blocked one)."""
    from . import adapters
    c = contract.load_contract()
    if op_name in ("qk_norm", "qk_norm_pair"):
        wq, wk = wls
        cq, ck = cells_by_side
        cells = [adapters.PairCell(a.name, a, b) for a, b in zip(cq, ck)]
    else:
        cells = cells_by_side[0]
    if names:
        cells = [x for x in cells if x.name in names or x.name == "BN/full"]
    if not _gpu():
        return None, cells
    if op_name in ("qk_norm", "qk_norm_pair"):
        data = adapters.QkInputs(wls[0].name.rsplit("_", 1)[0], adapters.make_inputs(wls[0]),
                                 adapters.make_inputs(wls[1]))
    elif op_name == "det_gemm":
        data = adapters.make_linear_inputs(wls[0])
    elif op_name == "rms_norm+det_gemm":
        data = adapters.make_chain_inputs(wls[0])
    else:
        data = adapters.make_inputs(wls[0])
    rep = harness.assert_gradient_batch_invariant(op_name, cells, c, data=data, raise_on_red=False)
    return rep, cells


def _targets(names, small):
    out = []
    names = names or ["rmsnorm_h8_t59", "rmsnorm_h4096_t32768", "rmsnorm_h8192_varlen16",
                      "qknorm_d128_t16384", "rmsnorm_h5120_packed131072",
                      "linear_h4096_o4096_t32768", "chain_rmsnorm_linear_h4096_o4096_t32768"]
    for n in names:
        if n in CHAINS:
            wl = _workload(CHAINS[n], small)
            out.append(("rms_norm+det_gemm", n, (wl,), (_cells(wl),)))
        elif n in inputs.LINEAR_WORKLOADS:
            wl = _workload(n, small)
            out.append(("det_gemm", n, (wl,), (_cells(wl),)))
        elif n.endswith(RECOMPUTE):
            base = n[: -len(RECOMPUTE)]
            wl = _workload(base, small)
            out.append(("rms_norm_recompute", n, (wl,), (_cells(wl),)))
        elif n.startswith("qknorm"):
            # "+pair": Q and K of every call in one launch per phase
            base = "qknorm_d128_t16384"
            wq, wk = _workload(base + "_q", small), _workload(base + "_k", small)
            op = "qk_norm_pair" if n.endswith(PAIR) else "qk_norm"
            out.append((op, n, (wq, wk), (_cells(wq), _cells(wk))))
        else:
            wl = _workload(n, small)
            out.append(("rms_norm", n, (wl,), (_cells(wl),)))
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="rmsnorm-bi")
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("list")
    ck = sub.add_parser("check")
    ck.add_argument("--workload", required=True)
    ck.add_argument("--cell", required=True)
    ck.add_argument("--small", action="store_true")
    sw = sub.add_parser("sweep")
    sw.add_argument("--workload", action="append")
    sw.add_argument("--small", action="store_true")
    sw.add_argument("--json")
    args = ap.parse_args(argv)

    if args.cmd == "list":
        for op, name, wls, cells in _targets(None, small=False):
            extra = f" -> {wls[0].out_features}" if wls[0].out_features else ""
            print(f"{name} ({op}): hidden {wls[0].hidden}{extra}, {wls[0].n_logical} logical rows")
            for c in cells[0]:
                print(f"    {c.name}: {len(c.calls)} call(s), rows {sum(c.call_shapes)}")
        return 0

    wanted = [args.workload] if args.cmd == "check" else args.workload
    results, rc = [], 0
    for op, name, wls, cells in _targets(wanted, args.small):
        rep, used = _run(op, wls, cells, names=[args.cell] if args.cmd == "check" else None)
        if rep is None:
            rows = [(c.name, harness.BLOCKED_HARDWARE) for c in used]
            rc = 1
        else:
            rows = [(c.name, c.status) for c in rep.cells]
            rc |= 0 if rep.strict else 1
            results.append(json.loads(rep.to_json()))
        print(f"{name} ({op})")
        for cname, status in rows:
            extra = ""
            if rep is not None and rep.chain_attribution.get(cname):
                extra = f"  (first drift: {rep.chain_attribution[cname]})"
            print(f"    {cname:44s} {status}{extra}")
    if getattr(args, "json", None):
        with open(args.json, "w") as f:
            json.dump(results, f, indent=1)
    return rc


if __name__ == "__main__":
    sys.exit(main())
