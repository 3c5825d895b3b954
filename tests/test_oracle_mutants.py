"""The oracle's pins catch plausible mistakes.

Each case copies ``oracle/rmsnorm_oracle.c`` to a temporary directory, plants
one mistake by a textual edit, builds the copy with gcc and runs every pin
against it on the CPU.  At least one pin must fail for every mutant; the
unmodified source must pass them all.
"""
import inspect
import os

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "dx_drops_dot_term": (" - xr[j] * r * r * dot / (double)H", ""),
    "dx_wrong_sign": ("dyr[j] * w[j] - xr[j] * r * r", "dyr[j] * w[j] + xr[j] * r * r"),
    "eps_outside_sqrt": ("1.0 / sqrt(ss / (double)H + eps)", "1.0 / (sqrt(ss / (double)H) + eps)"),
    "sum_not_mean": ("1.0 / sqrt(ss / (double)H + eps)", "1.0 / sqrt(ss + eps)"),
    "dot_drops_weight": ("dot += dyr[j] * w[j] * xr[j]", "dot += dyr[j] * xr[j]"),
    "dot_wrong_index": ("dot += dyr[j] * w[j] * xr[j]", "dot += dyr[j] * w[H - 1 - j] * xr[j]"),
    "dweight_drops_rstd": ("double t = dyr[j] * xr[j] * r;", "double t = dyr[j] * xr[j];"),
    "dweight_uses_w": ("double t = dyr[j] * xr[j] * r;", "double t = dyr[j] * w[j] * r;"),
    "y_drops_weight": ("yr[j] = xr[j] * r * w[j];", "yr[j] = xr[j] * r;"),
    "pad_rows_read_in_fwd": ("        if (is_pad(row_logical, p)) {\n            for (int64_t j = 0; j < H; ++j) yr[j] = 0.0;",
                             "        if (0) {\n            for (int64_t j = 0; j < H; ++j) yr[j] = 0.0;"),
    "duplicates_accepted": ("        if (inv[l] != -1) return ORACLE_ELAYOUT;\n", ""),
    "cdo_contiguous_streams": ("for (int s = w; s < CDO_BLOCK; s += CDO_STREAMS)",
                               "for (int s = w * 16; s < w * 16 + 16; ++s)"),
    "cdo_descending_fold": ("for (int s = w; s < CDO_BLOCK; s += CDO_STREAMS)",
                            "for (int s = w + CDO_BLOCK - CDO_STREAMS; s >= 0; s -= CDO_STREAMS)"),
    "cdo_sequential_stream_tree": ("P[b] = (q[0] + q[1]) + (q[2] + q[3]);",
                                   "P[b] = ((q[0] + q[1]) + q[2]) + q[3];"),
    "cdo_left_fold_over_blocks": ("dweight[j] = nb > 0 ? cdo_tree(P, nb, 0, npad) : 0.0f;",
                                  "{ float a = 0.0f; for (int64_t b = 0; b < nb; ++b) a = a + P[b]; dweight[j] = a; }"),
    "cdo_contribution_fused": ("float c = prod * rstd[p];\n                    acc = acc + c;",
                               "acc = fmaf(prod, rstd[p], acc);"),
    "cdo_eight_streams": ("#define CDO_STREAMS 4", "#define CDO_STREAMS 8"),
    "cdo_contribution_x_rstd_first": ("float c = prod * rstd[p];", "float c = dyv * (xv * rstd[p]);"),
}


def _run_all_pins(orc):
    failures = []
    for pin in pins.PINS:
        args = [orc]
        if "eps" in inspect.signature(pin).parameters:
            args.append(1e-6)
        try:
            pin(*args)
        except (AssertionError, oracle.OracleError, pytest.fail.Exception) as e:
            failures.append((pin.__name__, type(e).__name__))
    return failures


def _build_variant(tmp_path, name, edit):
    with open(oracle.SRC) as f:
        src = f.read()
    if edit is not None:
        old, new = edit
        assert src.count(old) >= 1, f"mutation anchor for {name} not found"
        src = src.replace(old, new, 1)
    path = os.path.join(str(tmp_path), f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.load_library(oracle.build(path, os.path.join(str(tmp_path), f"lib{name}.so")))


def test_unmodified_source_passes_every_pin(tmp_path):
    assert _run_all_pins(_build_variant(tmp_path, "clean", None)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failures = _run_all_pins(_build_variant(tmp_path, name, MUTANTS[name]))
    assert failures, f"no pin caught the planted mistake {name}"
