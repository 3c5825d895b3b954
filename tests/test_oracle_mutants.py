"""The oracle's pins catch plausible mistakes.

Each case copies an oracle source (``oracle/rmsnorm_oracle.c`` or
``oracle/linear_oracle.c``) to a temporary directory, plants one mistake by a
textual edit, builds the copy with gcc and runs every pin against it on the
CPU.  At least one pin must fail for every mutant; the
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
    "round_bf16_truncates": ("out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "out[i] = (uint16_t)(u >> 16);"),
    "round_bf16_ties_away": ("out[i] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);",
                             "out[i] = (uint16_t)((u + 0x8000u) >> 16);"),
}


LINEAR_MUTANTS = {
    "linear_dx_mirrored_weight_index": ("lin_widen(dy[r * n + o]) * lin_widen(w[o * k + i]);\n            dx",
                                        "lin_widen(dy[r * n + o]) * lin_widen(w[o * k + (k - 1 - i)]);\n            dx"),
    "linear_dw_drops_last_logical_row": ("for (int64_t l = 0; l < n_logical; ++l) {\n        const int64_t p = inv[l];",
                                         "for (int64_t l = 0; l + 1 < n_logical; ++l) {\n        const int64_t p = inv[l];"),
    "linear_dw_wrong_sign": ("dw[o * k + i] += c;", "dw[o * k + i] -= c;"),
    "linear_dw_uses_physical_row_of_wrong_tensor": ("const double c = g * lin_widen(x[p * k + i]);",
                                                    "const double c = g * lin_widen(x[(l < rows ? l : p) * k + i]);"),
    "linear_fwd_transposed_weight": ("s += lin_widen(x[r * k + i]) * lin_widen(w[o * k + i]);",
                                     "s += lin_widen(x[r * k + i]) * lin_widen(w[(i % n) * k + (o % k)]);"),
    "linear_pad_rows_read": ("        const int pad = row_logical && row_logical[r] < 0;\n        for (int64_t i = 0; i < k; ++i) {",
                             "        const int pad = 0;\n        for (int64_t i = 0; i < k; ++i) {"),
}


EMBEDDING_MUTANTS = {
    "edo_blocks_of_32": ("#define EDO_BLOCK 64", "#define EDO_BLOCK 32"),
    "edo_left_fold_over_blocks": ("out[v * dim + j] = edo_tree(q, nb, 0, width);",
                                  "{ float s = 0.0f; for (int64_t b = 0; b < nb; ++b) s = s + q[b]; out[v * dim + j] = s; }"),
    "edo_descending_occurrences": ("acc = acc + emb_widen(dy[occ[a + i] * dim + j]);",
                                   "acc = acc + emb_widen(dy[occ[a + (n - 1 - i)] * dim + j]);"),
    "embedding_bwd_wrong_token": ("dE[v * ncols + c] += g;", "dE[((v + 1) % vocab) * ncols + c] += g;"),
    "embedding_bwd_drops_last_row": ("for (int64_t l = 0; l < n_logical; ++l) {\n        const int64_t p = inv[l];",
                                     "for (int64_t l = 0; l + 1 < n_logical; ++l) {\n        const int64_t p = inv[l];"),
    "embedding_fwd_reads_padding": ("const int pad = row_logical && row_logical[r] < 0;\n        if (!pad && (ids[r]",
                                    "const int pad = 0;\n        if (!pad && (ids[r]"),
}


def _run_all_pins(orc):
    failures = []
    for pin in list(pins.PINS) + list(pins.LINEAR_PINS) + list(pins.EMBEDDING_PINS):
        args = [orc]
        if "eps" in inspect.signature(pin).parameters:
            args.append(1e-6)
        try:
            pin(*args)
        except (AssertionError, oracle.OracleError, pytest.fail.Exception) as e:
            failures.append((pin.__name__, type(e).__name__))
    return failures


def _build_variant(tmp_path, name, edit, which=0):
    """Build the oracle with source ``which`` (index into oracle.SRCS) edited."""
    srcs = []
    for i, src_path in enumerate(oracle.SRCS):
        with open(src_path) as f:
            src = f.read()
        if edit is not None and i == which:
            old, new = edit
            assert src.count(old) >= 1, f"mutation anchor for {name} not found"
            src = src.replace(old, new, 1)
        path = os.path.join(str(tmp_path), f"{name}_{i}.c")
        with open(path, "w") as f:
            f.write(src)
        srcs.append(path)
    return oracle.load_library(oracle.build(srcs, os.path.join(str(tmp_path), f"lib{name}.so")))


def test_unmodified_source_passes_every_pin(tmp_path):
    assert _run_all_pins(_build_variant(tmp_path, "clean", None)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    failures = _run_all_pins(_build_variant(tmp_path, name, MUTANTS[name]))
    assert failures, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(LINEAR_MUTANTS))
def test_linear_mutant_is_caught(tmp_path, name):
    failures = _run_all_pins(_build_variant(tmp_path, name, LINEAR_MUTANTS[name], which=1))
    assert failures, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(EMBEDDING_MUTANTS))
def test_embedding_mutant_is_caught(tmp_path, name):
    failures = _run_all_pins(_build_variant(tmp_path, name, EMBEDDING_MUTANTS[name], which=2))
    assert failures, f"no pin caught the planted mistake {name}"
