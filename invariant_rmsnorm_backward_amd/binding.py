"""Thin ctypes binding of the C-ABI in ``include/rmsnorm_bi.h``.

The functions named like the C entry points take exactly the C arguments
(device pointers as ints, sizes, a stream handle as int); they only marshal.
The small helpers below them (``fwd``, ``bwd``, ``Layout``, ``DwAccumulator``)
allocate outputs with torch (device memory only) and call those entry points.
Every computation runs in the HIP library; if the library is missing this
module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "librmsnorm_bi.so")

OK, EINVAL, EUNSUPPORTED, ELAYOUT, ECOVERAGE, ESTATE, EHIP, ESPILL = 0, -1, -2, -3, -4, -5, -6, -7
SPILL_TABLE = 32   # blocks a call may hold in part with a bounded accumulator
STATUS_NAMES = {OK: "OK", EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", ELAYOUT: "ELAYOUT",
                ECOVERAGE: "ECOVERAGE", ESTATE: "ESTATE", EHIP: "EHIP", ESPILL: "ESPILL"}

EXPORTED = ("rmsnorm_max_hidden", "rmsnorm_fwd", "rmsnorm_bwd_dx", "rmsnorm_dw_contrib",
            "rmsnorm_dw_finalize", "rmsnorm_layout_create", "rmsnorm_layout_destroy",
            "rmsnorm_layout_check", "rmsnorm_dw_acc_create", "rmsnorm_dw_acc_create_bounded",
            "rmsnorm_dw_acc_reset",
            "rmsnorm_dw_acc_destroy", "rmsnorm_last_error", "rmsnorm_backend_info",
            "rmsnorm_set_split_threshold", "rmsnorm_set_stream_threshold",
            "rmsnorm_set_workgroup_cap", "rmsnorm_stream_copy", "rmsnorm_stream_2r1w",
            "rmsnorm_fwd_packed", "rmsnorm_fwd_packed_pair", "rmsnorm_bwd_dx_packed_pair",
            "rmsnorm_bwd_dx_packed", "rmsnorm_bwd_dx_recompute", "rmsnorm_bwd_noalloc",
            "rmsnorm_bwd_noalloc_max_scratch",
            "det_gemm_fwd", "det_gemm_bwd_dx", "det_gemm_dw_acc_create", "det_gemm_dw_contrib",
            "det_gemm_dw_finalize", "det_gemm_dw_acc_reset", "det_gemm_dw_acc_destroy",
            "det_embedding_fwd", "det_embedding_dw_acc_create", "det_embedding_dw_acc_set_ids",
            "det_embedding_dw_contrib", "det_embedding_dw_finalize", "det_embedding_bwd",
            "det_embedding_dw_acc_reset", "det_embedding_dw_acc_destroy")


class RmsNormError(RuntimeError):
    def __init__(self, code: int, func: str, message: str):
        super().__init__(f"{func} -> {STATUS_NAMES.get(code, code)}: {message}")
        self.code = code
        self.func = func
        self.message = message


_lib = None


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run __graft_entry__.build() or python -m invariant_rmsnorm_backward_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "rmsnorm_max_hidden": ([], I32),
        "rmsnorm_fwd": ([P, P, P, P, I64, I64, ctypes.c_float, P, P], I32),
        "rmsnorm_bwd_dx": ([P, P, P, P, P, I64, I64, P, P, P], I32),
        "rmsnorm_bwd_dx_recompute": ([P, P, P, ctypes.c_float, P, I64, I64, P, P, P], I32),
        "rmsnorm_dw_contrib": ([P, P, P, I64, I64, P, P, P], I32),
        "rmsnorm_bwd_noalloc": ([P, P, P, P, P, P, I64, I64, P], I32),
        "rmsnorm_bwd_noalloc_max_scratch": ([], I64),
        "rmsnorm_dw_finalize": ([P, P, P], I32),
        "rmsnorm_layout_create": ([PP, P, I64, I64, P], I32),
        "rmsnorm_layout_destroy": ([P], I32),
        "rmsnorm_layout_check": ([P, I64, I64, ctypes.POINTER(ctypes.c_int64)], I32),
        "rmsnorm_dw_acc_create": ([PP, I64, I64, P], I32),
        "rmsnorm_dw_acc_create_bounded": ([PP, I64, I64, I64, P], I32),
        "rmsnorm_dw_acc_reset": ([P, P], I32),
        "rmsnorm_dw_acc_destroy": ([P], I32),
        "rmsnorm_last_error": ([], ctypes.c_char_p),
        "rmsnorm_backend_info": ([], ctypes.c_char_p),
        "rmsnorm_set_split_threshold": ([I64, ctypes.POINTER(ctypes.c_int64)], I32),
        "rmsnorm_set_stream_threshold": ([I64, ctypes.POINTER(ctypes.c_int64)], I32),
        "rmsnorm_set_workgroup_cap": ([I64, ctypes.POINTER(ctypes.c_int64)], I32),
        "rmsnorm_stream_copy": ([P, P, I64, P], I32),
        "rmsnorm_stream_2r1w": ([P, P, P, I64, P], I32),
        "rmsnorm_fwd_packed": ([P, P, P, P, I64, I64, I64, I64, ctypes.c_float, P, P], I32),
        "rmsnorm_bwd_dx_packed": ([P, P, P, P, P, I64, I64, I64, I64, P, P, P], I32),
        "rmsnorm_fwd_packed_pair": ([P, P, P, P, I64, I64, P, P, P, P, P, I64, I64, P, I64, I64,
                                     ctypes.c_float, P], I32),
        "rmsnorm_bwd_dx_packed_pair": ([P, P, P, P, P, I64, I64, P, P, P, P, P, P, P, I64, I64, P,
                                        P, I64, I64, P], I32),
        "det_gemm_fwd": ([P, P, P, I64, I64, I64, P, P], I32),
        "det_gemm_bwd_dx": ([P, P, P, I64, I64, I64, P, P], I32),
        "det_gemm_dw_acc_create": ([PP, I64, I64, I64, P], I32),
        "det_gemm_dw_contrib": ([P, P, I64, I64, I64, P, P, P], I32),
        "det_gemm_dw_finalize": ([P, P, P], I32),
        "det_gemm_dw_acc_reset": ([P, P], I32),
        "det_gemm_dw_acc_destroy": ([P], I32),
        "det_embedding_fwd": ([P, P, P, I64, I64, I64, P, P], I32),
        "det_embedding_dw_acc_create": ([PP, P, I64, I64, I64, P], I32),
        "det_embedding_dw_acc_set_ids": ([P, P, P], I32),
        "det_embedding_dw_contrib": ([P, I64, I64, P, P, P], I32),
        "det_embedding_dw_finalize": ([P, P, P], I32),
        "det_embedding_bwd": ([P, I64, I64, P, P, P], I32),
        "det_embedding_dw_acc_reset": ([P, P], I32),
        "det_embedding_dw_acc_destroy": ([P], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int, func: str):
    if rc != OK:
        raise RmsNormError(rc, func, rmsnorm_last_error())


# ------------------------------------------------------------ C entry points
def rmsnorm_max_hidden() -> int:
    return load().rmsnorm_max_hidden()


def rmsnorm_last_error() -> str:
    return load().rmsnorm_last_error().decode()


def rmsnorm_backend_info() -> str:
    return load().rmsnorm_backend_info().decode()


def rmsnorm_fwd(x: int, w: int, y: int, rstd: int, rows: int, hidden: int, eps: float,
                layout: Optional[int], stream: Optional[int]) -> None:
    _check(load().rmsnorm_fwd(x, w, y, rstd, rows, hidden, eps, layout, stream), "rmsnorm_fwd")


def rmsnorm_bwd_dx(x: int, w: int, dy: int, rstd: int, dx: int, rows: int, hidden: int,
                   layout: Optional[int], acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().rmsnorm_bwd_dx(x, w, dy, rstd, dx, rows, hidden, layout, acc, stream),
           "rmsnorm_bwd_dx")


def rmsnorm_bwd_dx_recompute(x: int, w: int, dy: int, eps: float, dx: int, rows: int, hidden: int,
                             layout: Optional[int], acc: Optional[int],
                             stream: Optional[int]) -> None:
    _check(load().rmsnorm_bwd_dx_recompute(x, w, dy, eps, dx, rows, hidden, layout, acc, stream),
           "rmsnorm_bwd_dx_recompute")


def rmsnorm_dw_contrib(x: int, dy: int, rstd: int, rows: int, hidden: int,
                       layout: Optional[int], acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().rmsnorm_dw_contrib(x, dy, rstd, rows, hidden, layout, acc, stream),
           "rmsnorm_dw_contrib")


def rmsnorm_dw_finalize(acc: Optional[int], dweight: int, stream: Optional[int]) -> None:
    _check(load().rmsnorm_dw_finalize(acc, dweight, stream), "rmsnorm_dw_finalize")


def rmsnorm_bwd_noalloc(x: int, w: int, dy: int, rstd: int, dx: int, dweight: int, rows: int,
                        hidden: int, stream: Optional[int]) -> None:
    _check(load().rmsnorm_bwd_noalloc(x, w, dy, rstd, dx, dweight, rows, hidden, stream),
           "rmsnorm_bwd_noalloc")


def rmsnorm_bwd_noalloc_max_scratch() -> int:
    return int(load().rmsnorm_bwd_noalloc_max_scratch())


def rmsnorm_layout_create(row_logical: np.ndarray, n_logical: int, stream: Optional[int]) -> int:
    rl = np.ascontiguousarray(row_logical, dtype=np.int32)
    out = ctypes.c_void_p()
    _check(load().rmsnorm_layout_create(ctypes.byref(out), rl.ctypes.data_as(ctypes.c_void_p),
                                        rl.size, n_logical, stream), "rmsnorm_layout_create")
    return out.value


def rmsnorm_layout_destroy(layout: Optional[int]) -> None:
    _check(load().rmsnorm_layout_destroy(layout), "rmsnorm_layout_destroy")


def rmsnorm_layout_check(row_logical: np.ndarray, n_logical: int) -> dict:
    rl = np.ascontiguousarray(row_logical, dtype=np.int32)
    stats = (ctypes.c_int64 * 5)()
    _check(load().rmsnorm_layout_check(rl.ctypes.data_as(ctypes.c_void_p), rl.size, n_logical,
                                       stats), "rmsnorm_layout_check")
    keys = ("blocks", "complete_blocks", "partial_blocks", "pad_rows", "real_rows")
    return dict(zip(keys, list(stats)))


def rmsnorm_dw_acc_create(n_logical: int, hidden: int, stream: Optional[int]) -> int:
    out = ctypes.c_void_p()
    _check(load().rmsnorm_dw_acc_create(ctypes.byref(out), n_logical, hidden, stream),
           "rmsnorm_dw_acc_create")
    return out.value


def rmsnorm_dw_acc_create_bounded(n_logical: int, hidden: int, max_spill_rows: int,
                                  stream: Optional[int]) -> int:
    out = ctypes.c_void_p()
    _check(load().rmsnorm_dw_acc_create_bounded(ctypes.byref(out), n_logical, hidden,
                                                max_spill_rows, stream),
           "rmsnorm_dw_acc_create_bounded")
    return out.value


def rmsnorm_dw_acc_reset(acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().rmsnorm_dw_acc_reset(acc, stream), "rmsnorm_dw_acc_reset")


def rmsnorm_dw_acc_destroy(acc: Optional[int]) -> None:
    _check(load().rmsnorm_dw_acc_destroy(acc), "rmsnorm_dw_acc_destroy")


# ------------------------------------------------------------------ helpers
def rmsnorm_fwd_packed(x: int, w: int, y: int, rstd: int, tokens: int, heads: int, head_dim: int,
                       token_stride: int, eps: float, layout: Optional[int],
                       stream: Optional[int]) -> None:
    _check(load().rmsnorm_fwd_packed(x, w, y, rstd, tokens, heads, head_dim, token_stride, eps,
                                     layout, stream), "rmsnorm_fwd_packed")


def rmsnorm_bwd_dx_packed(x: int, w: int, dy: int, rstd: int, dx: int, tokens: int, heads: int,
                          head_dim: int, token_stride: int, layout: Optional[int],
                          acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().rmsnorm_bwd_dx_packed(x, w, dy, rstd, dx, tokens, heads, head_dim, token_stride,
                                        layout, acc, stream), "rmsnorm_bwd_dx_packed")


def rmsnorm_fwd_packed_pair(a: tuple, b: tuple, tokens: int, head_dim: int, eps: float,
                            stream: Optional[int]) -> None:
    """a, b = (x, w, y, rstd, heads, token_stride, layout) of each norm (pointers)."""
    _check(load().rmsnorm_fwd_packed_pair(*a, *b, tokens, head_dim, eps, stream),
           "rmsnorm_fwd_packed_pair")


def rmsnorm_bwd_dx_packed_pair(a: tuple, b: tuple, tokens: int, head_dim: int,
                               stream: Optional[int]) -> None:
    """a, b = (x, w, dy, rstd, dx, heads, token_stride, layout, acc) of each norm."""
    _check(load().rmsnorm_bwd_dx_packed_pair(*a, *b, tokens, head_dim, stream),
           "rmsnorm_bwd_dx_packed_pair")


def rmsnorm_set_split_threshold(blocks: int) -> int:
    """Sets the backward's two-pass threshold (in canonical blocks; 0 disables
    the two-pass path, negative restores the default); returns the previous one."""
    prev = ctypes.c_int64(0)
    _check(load().rmsnorm_set_split_threshold(int(blocks), ctypes.byref(prev)),
           "rmsnorm_set_split_threshold")
    return int(prev.value)


def rmsnorm_set_stream_threshold(blocks: int) -> int:
    """Sets the lower bound (in canonical blocks) of the stream-owner backward
    (negative restores the default); returns the previous one."""
    prev = ctypes.c_int64(0)
    _check(load().rmsnorm_set_stream_threshold(int(blocks), ctypes.byref(prev)),
           "rmsnorm_set_stream_threshold")
    return int(prev.value)


def rmsnorm_set_workgroup_cap(groups: int) -> int:
    """Caps the block-owning workgroups of the fused backward (0 or negative
    restores the default, the number the GPU holds at once); returns the
    previous cap (0 = default)."""
    prev = ctypes.c_int64(0)
    _check(load().rmsnorm_set_workgroup_cap(int(groups), ctypes.byref(prev)),
           "rmsnorm_set_workgroup_cap")
    return int(prev.value)


def rmsnorm_stream_copy(src: int, dst: int, nbytes: int, stream: Optional[int]) -> None:
    """Streaming device copy with the kernels' access policy (bandwidth ceiling probe)."""
    _check(load().rmsnorm_stream_copy(src, dst, int(nbytes), stream), "rmsnorm_stream_copy")


def rmsnorm_stream_2r1w(a: int, b: int, c: int, nbytes: int, stream: Optional[int]) -> None:
    """c = a XOR b: two reads per write, the backward's traffic mix (ceiling probe)."""
    _check(load().rmsnorm_stream_2r1w(a, b, c, int(nbytes), stream), "rmsnorm_stream_2r1w")


# ---------------------------------------------------------------- det_gemm
def det_gemm_fwd(x: int, w: int, y: int, rows: int, n: int, k: int, layout: Optional[int],
                 stream: Optional[int]) -> None:
    _check(load().det_gemm_fwd(x, w, y, rows, n, k, layout, stream), "det_gemm_fwd")


def det_gemm_bwd_dx(dy: int, w: int, dx: int, rows: int, n: int, k: int, layout: Optional[int],
                    stream: Optional[int]) -> None:
    _check(load().det_gemm_bwd_dx(dy, w, dx, rows, n, k, layout, stream), "det_gemm_bwd_dx")


def det_gemm_dw_acc_create(n_logical: int, n: int, k: int, stream: Optional[int]) -> int:
    h = ctypes.c_void_p(None)
    _check(load().det_gemm_dw_acc_create(ctypes.byref(h), n_logical, n, k, stream),
           "det_gemm_dw_acc_create")
    return h.value


def det_gemm_dw_contrib(x: int, dy: int, rows: int, n: int, k: int, layout: Optional[int],
                        acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().det_gemm_dw_contrib(x, dy, rows, n, k, layout, acc, stream),
           "det_gemm_dw_contrib")


def det_gemm_dw_finalize(acc: Optional[int], dw: int, stream: Optional[int]) -> None:
    _check(load().det_gemm_dw_finalize(acc, dw, stream), "det_gemm_dw_finalize")


def det_gemm_dw_acc_reset(acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().det_gemm_dw_acc_reset(acc, stream), "det_gemm_dw_acc_reset")


def det_gemm_dw_acc_destroy(acc: Optional[int]) -> None:
    _check(load().det_gemm_dw_acc_destroy(acc), "det_gemm_dw_acc_destroy")


# ------------------------------------------------------------- det_embedding
def det_embedding_fwd(ids: int, table: int, y: int, rows: int, vocab: int, dim: int,
                      layout: Optional[int], stream: Optional[int]) -> None:
    _check(load().det_embedding_fwd(ids, table, y, rows, vocab, dim, layout, stream),
           "det_embedding_fwd")


def det_embedding_dw_acc_create(ids_host: np.ndarray, vocab: int, dim: int,
                                stream: Optional[int]) -> int:
    ids = np.ascontiguousarray(ids_host, dtype=np.int32)
    h = ctypes.c_void_p(None)
    _check(load().det_embedding_dw_acc_create(ctypes.byref(h), ids.ctypes.data_as(ctypes.c_void_p),
                                              ids.size, vocab, dim, stream),
           "det_embedding_dw_acc_create")
    return h.value


def det_embedding_dw_acc_set_ids(acc: Optional[int], ids_host: np.ndarray,
                                 stream: Optional[int]) -> None:
    ids = np.ascontiguousarray(ids_host, dtype=np.int32)
    _check(load().det_embedding_dw_acc_set_ids(acc, ids.ctypes.data_as(ctypes.c_void_p), stream),
           "det_embedding_dw_acc_set_ids")


def det_embedding_dw_contrib(dy: int, rows: int, dim: int, layout: Optional[int],
                             acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().det_embedding_dw_contrib(dy, rows, dim, layout, acc, stream),
           "det_embedding_dw_contrib")


def det_embedding_dw_finalize(acc: Optional[int], dE: int, stream: Optional[int]) -> None:
    _check(load().det_embedding_dw_finalize(acc, dE, stream), "det_embedding_dw_finalize")


def det_embedding_bwd(dy: int, rows: int, dim: int, acc: Optional[int], dE: int,
                      stream: Optional[int]) -> None:
    _check(load().det_embedding_bwd(dy, rows, dim, acc, dE, stream), "det_embedding_bwd")


def det_embedding_dw_acc_reset(acc: Optional[int], stream: Optional[int]) -> None:
    _check(load().det_embedding_dw_acc_reset(acc, stream), "det_embedding_dw_acc_reset")


def det_embedding_dw_acc_destroy(acc: Optional[int]) -> None:
    _check(load().det_embedding_dw_acc_destroy(acc), "det_embedding_dw_acc_destroy")


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


class Layout:
    """Owns a device layout (plan) built from a host row map."""

    def __init__(self, row_logical: np.ndarray, n_logical: int, stream: Optional[int] = None):
        self.row_logical = np.ascontiguousarray(row_logical, dtype=np.int32)
        self.rows = int(self.row_logical.size)
        self.n_logical = int(n_logical)
        self.handle = rmsnorm_layout_create(self.row_logical, self.n_logical,
                                            current_stream() if stream is None else stream)

    def close(self):
        if self.handle:
            rmsnorm_layout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DwAccumulator:
    """Owns a canonical dweight accumulator."""

    def __init__(self, n_logical: int, hidden: int, stream: Optional[int] = None,
                 max_spill_rows: Optional[int] = None):
        """max_spill_rows: bound on the spill area (None: unbounded)."""
        self.n_logical = int(n_logical)
        self.hidden = int(hidden)
        st = current_stream() if stream is None else stream
        if max_spill_rows is None:
            self.handle = rmsnorm_dw_acc_create(self.n_logical, self.hidden, st)
        else:
            self.handle = rmsnorm_dw_acc_create_bounded(self.n_logical, self.hidden,
                                                        int(max_spill_rows), st)

    def reset(self, stream: Optional[int] = None):
        rmsnorm_dw_acc_reset(self.handle, current_stream() if stream is None else stream)

    def finalize(self, dweight=None, stream: Optional[int] = None):
        import torch
        if dweight is None:
            dweight = torch.empty(self.hidden, dtype=torch.float32, device="cuda")
        rmsnorm_dw_finalize(self.handle, dweight.data_ptr(),
                            current_stream() if stream is None else stream)
        return dweight

    def close(self):
        if self.handle:
            rmsnorm_dw_acc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _handle(obj) -> Optional[int]:
    return None if obj is None else obj.handle


def fwd(x, w, eps: float, layout: Optional[Layout] = None, y=None, rstd=None,
        stream: Optional[int] = None, save_rstd: bool = True) -> Tuple:
    """y, rstd = RMSNorm forward of bf16 ``x[rows, hidden]`` (device tensors);
    with save_rstd=False no rstd is written and None is returned for it."""
    import torch
    rows, hidden = x.shape
    y = torch.empty_like(x) if y is None else y
    if save_rstd and rstd is None:
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    rmsnorm_fwd(x.data_ptr(), w.data_ptr(), y.data_ptr(), rstd.data_ptr() if save_rstd else None,
                rows, hidden, float(eps), _handle(layout),
                current_stream() if stream is None else stream)
    return y, (rstd if save_rstd else None)


def bwd(x, w, dy, rstd, layout: Optional[Layout] = None, acc: Optional[DwAccumulator] = None,
        dx=None, stream: Optional[int] = None):
    """dx of bf16 ``x``; with ``acc`` the dweight contributions are folded in."""
    import torch
    rows, hidden = x.shape
    dx = torch.empty_like(x) if dx is None else dx
    rmsnorm_bwd_dx(x.data_ptr(), w.data_ptr(), dy.data_ptr(), rstd.data_ptr(), dx.data_ptr(),
                   rows, hidden, _handle(layout), _handle(acc),
                   current_stream() if stream is None else stream)
    return dx


def bwd_recompute(x, w, dy, eps: float, layout: Optional[Layout] = None,
                  acc: Optional[DwAccumulator] = None, dx=None, stream: Optional[int] = None):
    """dx of bf16 ``x`` with rstd rebuilt from x (bitwise the forward's rstd)."""
    import torch
    rows, hidden = x.shape
    dx = torch.empty_like(x) if dx is None else dx
    rmsnorm_bwd_dx_recompute(x.data_ptr(), w.data_ptr(), dy.data_ptr(), float(eps), dx.data_ptr(),
                             rows, hidden, _handle(layout), _handle(acc),
                             current_stream() if stream is None else stream)
    return dx


def dw_contrib(x, dy, rstd, acc: DwAccumulator, layout: Optional[Layout] = None,
               stream: Optional[int] = None) -> None:
    rows, hidden = x.shape
    rmsnorm_dw_contrib(x.data_ptr(), dy.data_ptr(), rstd.data_ptr(), rows, hidden,
                       _handle(layout), acc.handle, current_stream() if stream is None else stream)


# --------------------------------------------------------- det_gemm helpers
class GemmDwAccumulator:
    """Owns a canonical dW accumulator of a linear layer (n outputs, k inputs)."""

    def __init__(self, n_logical: int, n: int, k: int, stream: Optional[int] = None):
        self.n_logical, self.n, self.k = int(n_logical), int(n), int(k)
        self.handle = det_gemm_dw_acc_create(self.n_logical, self.n, self.k,
                                             current_stream() if stream is None else stream)

    def contrib(self, x, dy, layout: Optional[Layout] = None, stream: Optional[int] = None):
        rows = x.shape[0]
        det_gemm_dw_contrib(x.data_ptr(), dy.data_ptr(), rows, self.n, self.k, _handle(layout),
                            self.handle, current_stream() if stream is None else stream)

    def reset(self, stream: Optional[int] = None):
        det_gemm_dw_acc_reset(self.handle, current_stream() if stream is None else stream)

    def finalize(self, dw=None, stream: Optional[int] = None):
        import torch
        if dw is None:
            dw = torch.empty((self.n, self.k), dtype=torch.float32, device="cuda")
        det_gemm_dw_finalize(self.handle, dw.data_ptr(),
                             current_stream() if stream is None else stream)
        return dw

    def close(self):
        if self.handle:
            det_gemm_dw_acc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gemm_fwd(x, w, layout: Optional[Layout] = None, y=None, stream: Optional[int] = None):
    """y = x W^T for bf16 x[rows, k], W[n, k] (device tensors)."""
    import torch
    rows, k = x.shape
    n = w.shape[0]
    y = torch.empty((rows, n), dtype=x.dtype, device=x.device) if y is None else y
    det_gemm_fwd(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, n, k, _handle(layout),
                 current_stream() if stream is None else stream)
    return y


def gemm_bwd_dx(dy, w, layout: Optional[Layout] = None, dx=None, stream: Optional[int] = None):
    """dX = dY W for bf16 dY[rows, n], W[n, k]."""
    import torch
    rows, n = dy.shape
    k = w.shape[1]
    dx = torch.empty((rows, k), dtype=dy.dtype, device=dy.device) if dx is None else dx
    det_gemm_bwd_dx(dy.data_ptr(), w.data_ptr(), dx.data_ptr(), rows, n, k, _handle(layout),
                    current_stream() if stream is None else stream)
    return dx


# ----------------------------------------------------- det_embedding helpers
class EmbeddingDwAccumulator:
    """Owns a canonical embedding-gradient accumulator for one batch's ids."""

    def __init__(self, ids_host: np.ndarray, vocab: int, dim: int, stream: Optional[int] = None):
        self.n_logical, self.vocab, self.dim = int(len(ids_host)), int(vocab), int(dim)
        self.handle = det_embedding_dw_acc_create(ids_host, self.vocab, self.dim,
                                                  current_stream() if stream is None else stream)

    def set_ids(self, ids_host: np.ndarray, stream: Optional[int] = None):
        det_embedding_dw_acc_set_ids(self.handle, ids_host,
                                     current_stream() if stream is None else stream)

    def contrib(self, dy, layout: Optional[Layout] = None, stream: Optional[int] = None):
        det_embedding_dw_contrib(dy.data_ptr(), dy.shape[0], self.dim, _handle(layout), self.handle,
                                 current_stream() if stream is None else stream)

    def reset(self, stream: Optional[int] = None):
        det_embedding_dw_acc_reset(self.handle, current_stream() if stream is None else stream)

    def finalize(self, dE=None, stream: Optional[int] = None):
        import torch
        if dE is None:
            dE = torch.empty((self.vocab, self.dim), dtype=torch.float32, device="cuda")
        det_embedding_dw_finalize(self.handle, dE.data_ptr(),
                                  current_stream() if stream is None else stream)
        return dE

    def backward(self, dy, dE=None, stream: Optional[int] = None):
        """The one-call backward (all rows in logical order): dE, bitwise as contrib + finalize."""
        import torch
        if dE is None:
            dE = torch.empty((self.vocab, self.dim), dtype=torch.float32, device="cuda")
        det_embedding_bwd(dy.data_ptr(), dy.shape[0], self.dim, self.handle, dE.data_ptr(),
                          current_stream() if stream is None else stream)
        return dE

    def close(self):
        if self.handle:
            det_embedding_dw_acc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def embedding_fwd(ids, table, layout: Optional[Layout] = None, y=None,
                  stream: Optional[int] = None):
    """y = table[ids] for device int32 ids[rows] and bf16 table[vocab, dim]."""
    import torch
    rows = ids.shape[0]
    vocab, dim = table.shape
    y = torch.empty((rows, dim), dtype=table.dtype, device=table.device) if y is None else y
    det_embedding_fwd(ids.data_ptr(), table.data_ptr(), y.data_ptr(), rows, vocab, dim,
                      _handle(layout), current_stream() if stream is None else stream)
    return y
