"""Shared helpers of the GPU parity tests (imports the oracle: test-only)."""
import contextlib

import numpy as np
import torch

import oracle
from invariant_rmsnorm_backward_amd import adapters, binding, inputs, layouts


def make_data(wl: inputs.Workload) -> adapters.NormInputs:
    """Logical inputs generated on the CPU, copied to the GPU."""
    return adapters.make_inputs(wl, device="cuda", gen_device="cpu")


def oracle_reference(wl: inputs.Workload) -> dict:
    """FP64 oracle outputs in logical order, from CPU-generated inputs."""
    xb = inputs.bf16_bits(inputs.gen_x(wl))
    wb = inputs.bf16_bits(inputs.gen_w(wl))
    dyb = inputs.bf16_bits(inputs.gen_dy(wl))
    y, rstd = oracle.rmsnorm_fwd_bf16(xb, wb, wl.eps)
    dx, dw, _ = oracle.rmsnorm_bwd_bf16(xb, wb, dyb, wl.eps)
    return {"y": y, "rstd": rstd, "dx": dx, "dweight": dw}


def standard_cells(wl: inputs.Workload, chunk: int):
    """Every layout family for one logical multiset."""
    return layouts.standard_matrix(wl, chunk)


def qk_cells(wq, wk, chunk):
    cq = standard_cells(wq, chunk)
    ck = standard_cells(wk, chunk)
    return [adapters.PairCell(a.name, a, b) for a, b in zip(cq, ck)]


def bf16_ulp_fraction(got_bits: np.ndarray, ref64: np.ndarray) -> float:
    """Fraction of bf16 outputs within one bf16 ulp of the FP64 reference."""
    g = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = ref64.astype(np.float64)
    ulp = np.abs(r) * 2.0 ** -7
    return float(np.mean(np.abs(g - r) <= np.maximum(ulp, 1e-30)))


def physical_rstd(rstd_logical: np.ndarray, call) -> torch.Tensor:
    """rstd for one call's physical rows (padding rows get NaN: never read)."""
    if call.row_logical is None:
        return torch.from_numpy(rstd_logical.astype(np.float32)).cuda()
    rl = call.row_logical.astype(np.int64)
    out = np.full(call.rows, np.nan, dtype=np.float32)
    out[rl >= 0] = rstd_logical[rl[rl >= 0]]
    return torch.from_numpy(out).cuda()


# The backward for hidden > 256 has three work distributions with the same
# arithmetic: the fused kernel (workgroups owning whole canonical blocks),
# the stream-owner kernel (one workgroup per fold stream of a block; calls
# with dx and an accumulator) and the two-pass path (dx rows beside 256-column
# dweight units).  Each is forced through the split and stream thresholds.
BWD_PATHS = {"fused": (0, -1), "stream": (1 << 40, 0), "two_pass": (1 << 40, 1 << 41)}


@contextlib.contextmanager
def forced_path(name: str):
    split, stream = BWD_PATHS[name]
    prev_split = binding.rmsnorm_set_split_threshold(split)
    prev_stream = binding.rmsnorm_set_stream_threshold(stream)
    try:
        yield name
    finally:
        binding.rmsnorm_set_stream_threshold(prev_stream)
        binding.rmsnorm_set_split_threshold(prev_split)
