"""FP64 CPU oracle for RMSNorm forward/backward, the CDO-v2 dweight order,
the backward of a linear layer (dX, dW) and the embedding table gradient
(with an FP32 emulation of its EDO-v1 order).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``invariant_rmsnorm_backward_amd``) and never imports it.

The arithmetic lives in ``rmsnorm_oracle.c``, ``linear_oracle.c`` and
``embedding_oracle.c`` (plain C, FP64, single thread); this module only marshals numpy arrays.  See the C
files' headers for the definitions followed and the pins that check them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "rmsnorm_oracle.c")
SRCS = [SRC, os.path.join(_HERE, "linear_oracle.c"), os.path.join(_HERE, "embedding_oracle.c")]
LIB_PATH = os.path.join(_HERE, "liboracle_rmsnorm.so")

# -ffp-contract=off and no fast-math: each float operation rounds once, as written.
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None


def build(src=None, out: str = LIB_PATH) -> str:
    """Compile an oracle library with gcc; returns its path.  ``src`` replaces
    the RMSNorm source (the pin tests build deliberately broken copies)."""
    srcs = list(SRCS)
    if src is not None:
        srcs = [src] + SRCS[1:] if not isinstance(src, (list, tuple)) else list(src)
    subprocess.run(["gcc", *GCC_FLAGS, *srcs, "-o", out, "-lm"], check=True)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_widen_bf16.argtypes = [P, I64, P]
    lib.oracle_widen_bf16.restype = None
    lib.oracle_round_bf16.argtypes = [P, I64, P]
    lib.oracle_round_bf16.restype = None
    lib.oracle_rmsnorm_fwd.argtypes = [P, P, I64, I64, ctypes.c_double, P, P, P]
    lib.oracle_rmsnorm_fwd.restype = ctypes.c_int
    lib.oracle_rmsnorm_bwd.argtypes = [P, P, P, I64, I64, ctypes.c_double, P, I64, P, P, P]
    lib.oracle_rmsnorm_bwd.restype = ctypes.c_int
    lib.oracle_cdo_v2_dweight_f32.argtypes = [P, P, P, I64, I64, P, I64, P]
    lib.oracle_cdo_v2_dweight_f32.restype = ctypes.c_int
    lib.oracle_linear_fwd.argtypes = [P, P, I64, I64, I64, P, P]
    lib.oracle_linear_fwd.restype = ctypes.c_int
    lib.oracle_linear_bwd.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P, P]
    lib.oracle_linear_bwd.restype = ctypes.c_int
    lib.oracle_linear_sample.argtypes = [P, P, P, I64, I64, I64, I64, P, P, P, P]
    lib.oracle_linear_sample.restype = ctypes.c_int
    lib.oracle_embedding_fwd.argtypes = [P, P, I64, I64, I64, P, P]
    lib.oracle_embedding_fwd.restype = ctypes.c_int
    lib.oracle_embedding_bwd.argtypes = [P, P, I64, I64, I64, P, I64, P, I64, P, P]
    lib.oracle_embedding_bwd.restype = ctypes.c_int
    lib.oracle_edo_v1_f32.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_edo_v1_f32.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or any(os.path.getmtime(LIB_PATH) < os.path.getmtime(f)
                                               for f in SRCS):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


class Oracle:
    """The oracle's Python API over one loaded build of the C source."""

    def __init__(self, lib=None):
        self._fixed = lib

    def _lib(self):
        return self._fixed if self._fixed is not None else _load()

    def widen_bf16(self, bits: np.ndarray) -> np.ndarray:
        """Exact widening of raw bf16 bit patterns (uint16) to float64."""
        b = _c(bits, np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib().oracle_widen_bf16(_ptr(b), b.size, _ptr(out))
        return out

    def round_bf16(self, x: np.ndarray) -> np.ndarray:
        """Raw bf16 patterns (uint16) nearest to finite float64 values."""
        a = _c(x, np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self._lib().oracle_round_bf16(_ptr(a), a.size, _ptr(out))
        return out

    def rmsnorm_fwd(self, x: np.ndarray, w: np.ndarray, eps: float,
                    row_logical: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """FP64 forward on float64 ``x[rows, H]``, ``w[H]``; returns (y, rstd).
        Rows whose ``row_logical`` entry is -1 are padding: y = 0, rstd = 0."""
        x = _c(x, np.float64)
        w = _c(w, np.float64)
        rows, H = x.shape
        rl = None if row_logical is None else _c(row_logical, np.int32)
        y = np.empty_like(x)
        rstd = np.empty(rows, dtype=np.float64)
        _check(self._lib().oracle_rmsnorm_fwd(_ptr(x), _ptr(w), rows, H, float(eps), _ptr(rl),
                                              _ptr(y), _ptr(rstd)), "oracle_rmsnorm_fwd")
        return y, rstd

    def rmsnorm_bwd(self, x: np.ndarray, w: np.ndarray, dy: np.ndarray, eps: float,
                    row_logical: Optional[np.ndarray] = None, n_logical: Optional[int] = None
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """FP64 backward; returns (dx, dweight, dweight_abs).  dweight sums the
        rows this call holds in ascending logical index; dweight_abs is the
        matching sum of absolute contributions (an error scale)."""
        x = _c(x, np.float64)
        w = _c(w, np.float64)
        dy = _c(dy, np.float64)
        rows, H = x.shape
        assert dy.shape == x.shape and w.shape == (H,)
        rl = None if row_logical is None else _c(row_logical, np.int32)
        nl = rows if n_logical is None else int(n_logical)
        dx = np.empty_like(x)
        dw = np.empty(H, dtype=np.float64)
        dwa = np.empty(H, dtype=np.float64)
        _check(self._lib().oracle_rmsnorm_bwd(_ptr(x), _ptr(w), _ptr(dy), rows, H, float(eps),
                                              _ptr(rl), nl, _ptr(dx), _ptr(dw), _ptr(dwa)),
               "oracle_rmsnorm_bwd")
        return dx, dw, dwa

    def rmsnorm_fwd_bf16(self, x_bits, w_bits, eps, row_logical=None):
        """Forward on raw bf16 inputs, widened exactly to FP64."""
        return self.rmsnorm_fwd(self.widen_bf16(x_bits), self.widen_bf16(w_bits), eps, row_logical)

    def rmsnorm_bwd_bf16(self, x_bits, w_bits, dy_bits, eps, row_logical=None, n_logical=None):
        """Backward on raw bf16 inputs, widened exactly to FP64."""
        return self.rmsnorm_bwd(self.widen_bf16(x_bits), self.widen_bf16(w_bits),
                                self.widen_bf16(dy_bits), eps, row_logical, n_logical)

    def cdo_v2_dweight_f32(self, x_bits: np.ndarray, dy_bits: np.ndarray, rstd: np.ndarray,
                           row_logical: Optional[np.ndarray] = None,
                           n_logical: Optional[int] = None) -> np.ndarray:
        """FP32 emulation of the canonical dweight order CDO-v2 (see the C source)."""
        x = _c(x_bits, np.uint16)
        dy = _c(dy_bits, np.uint16)
        r = _c(rstd, np.float32)
        rows, H = x.shape
        rl = None if row_logical is None else _c(row_logical, np.int32)
        nl = rows if n_logical is None else int(n_logical)
        out = np.empty(H, dtype=np.float32)
        _check(self._lib().oracle_cdo_v2_dweight_f32(_ptr(x), _ptr(dy), _ptr(r), rows, H,
                                                     _ptr(rl), nl, _ptr(out)),
               "oracle_cdo_v2_dweight_f32")
        return out

    # ------------------------------------------------------------- linear layer
    def linear_fwd_bf16(self, x_bits, w_bits, row_logical=None) -> np.ndarray:
        """y = x W^T in FP64 from raw bf16 x[rows, K], W[N, K]; padding rows 0."""
        x = _c(x_bits, np.uint16)
        w = _c(w_bits, np.uint16)
        rows, k = x.shape
        n = w.shape[0]
        assert w.shape == (n, k)
        rl = None if row_logical is None else _c(row_logical, np.int32)
        y = np.empty((rows, n), dtype=np.float64)
        _check(self._lib().oracle_linear_fwd(_ptr(x), _ptr(w), rows, n, k, _ptr(rl), _ptr(y)),
               "oracle_linear_fwd")
        return y

    def linear_bwd_bf16(self, x_bits, w_bits, dy_bits, row_logical=None, n_logical=None):
        """(dX, dW, |dW|) in FP64 from raw bf16 x[rows, K], W[N, K], dY[rows, N].
        dX is per physical row (padding rows 0); dW sums the rows the call
        holds in ascending logical index; |dW| is the matching sum of
        absolute terms (an error scale)."""
        x = _c(x_bits, np.uint16)
        w = _c(w_bits, np.uint16)
        dy = _c(dy_bits, np.uint16)
        rows, k = x.shape
        n = w.shape[0]
        assert w.shape == (n, k) and dy.shape == (rows, n)
        rl = None if row_logical is None else _c(row_logical, np.int32)
        nl = rows if n_logical is None else int(n_logical)
        dx = np.empty((rows, k), dtype=np.float64)
        dw = np.empty((n, k), dtype=np.float64)
        dwa = np.empty((n, k), dtype=np.float64)
        _check(self._lib().oracle_linear_bwd(_ptr(x), _ptr(w), _ptr(dy), rows, n, k, _ptr(rl), nl,
                                             _ptr(dx), _ptr(dw), _ptr(dwa)), "oracle_linear_bwd")
        return dx, dw, dwa

    def linear_sample_bf16(self, x_bits, w_bits, dy_bits, kind, ia, ib) -> np.ndarray:
        """Single outputs of an identity-layout call: kind 0 = dX[ia][ib],
        1 = dW[ia][ib], 2 = |dW|[ia][ib], 3 = y[ia][ib]."""
        x = _c(x_bits, np.uint16)
        w = _c(w_bits, np.uint16)
        dy = _c(dy_bits, np.uint16)
        rows, k = x.shape
        n = w.shape[0]
        kd = _c(kind, np.int32)
        a = _c(ia, np.int64)
        b = _c(ib, np.int64)
        out = np.empty(len(kd), dtype=np.float64)
        _check(self._lib().oracle_linear_sample(_ptr(x), _ptr(w), _ptr(dy), rows, n, k, len(kd),
                                                _ptr(kd), _ptr(a), _ptr(b), _ptr(out)),
               "oracle_linear_sample")
        return out

    # ---------------------------------------------------------------- embedding
    def embedding_fwd_bf16(self, ids, table_bits, row_logical=None) -> np.ndarray:
        """y = table[ids] (FP64) for the call's rows; padding rows 0."""
        i = _c(ids, np.int32)
        t = _c(table_bits, np.uint16)
        vocab, dim = t.shape
        rl = None if row_logical is None else _c(row_logical, np.int32)
        y = np.empty((len(i), dim), dtype=np.float64)
        _check(self._lib().oracle_embedding_fwd(_ptr(i), _ptr(t), len(i), vocab, dim, _ptr(rl),
                                                _ptr(y)), "oracle_embedding_fwd")
        return y

    def embedding_bwd_bf16(self, ids, dy_bits, vocab, row_logical=None, n_logical=None, cols=None):
        """(dE, |dE|) in FP64, [vocab, len(cols) or dim], summed over the rows the
        call holds in ascending logical index."""
        i = _c(ids, np.int32)
        dy = _c(dy_bits, np.uint16)
        rows, dim = dy.shape
        rl = None if row_logical is None else _c(row_logical, np.int32)
        nl = rows if n_logical is None else int(n_logical)
        cl = None if cols is None else _c(cols, np.int64)
        nc = dim if cols is None else len(cl)
        dE = np.empty((vocab, nc), dtype=np.float64)
        dEa = np.empty((vocab, nc), dtype=np.float64)
        _check(self._lib().oracle_embedding_bwd(_ptr(i), _ptr(dy), rows, vocab, dim, _ptr(rl), nl,
                                                _ptr(cl), nc, _ptr(dE), _ptr(dEa)),
               "oracle_embedding_bwd")
        return dE, dEa

    def edo_v1_f32(self, ids, dy_bits, vocab) -> np.ndarray:
        """FP32 emulation of the canonical embedding-gradient order EDO-v1 on
        logical-order ids[n_logical] and dy[n_logical, dim]."""
        i = _c(ids, np.int32)
        dy = _c(dy_bits, np.uint16)
        n, dim = dy.shape
        out = np.empty((vocab, dim), dtype=np.float32)
        _check(self._lib().oracle_edo_v1_f32(_ptr(i), _ptr(dy), n, vocab, dim, _ptr(out)),
               "oracle_edo_v1_f32")
        return out


def load_library(path: str) -> Oracle:
    """Bind another build of the oracle source (the pin tests use this on
    deliberately broken copies)."""
    return Oracle(_bind(ctypes.CDLL(path)))


_default = Oracle()
widen_bf16 = _default.widen_bf16
round_bf16 = _default.round_bf16
rmsnorm_fwd = _default.rmsnorm_fwd
rmsnorm_bwd = _default.rmsnorm_bwd
rmsnorm_fwd_bf16 = _default.rmsnorm_fwd_bf16
rmsnorm_bwd_bf16 = _default.rmsnorm_bwd_bf16
cdo_v2_dweight_f32 = _default.cdo_v2_dweight_f32
linear_fwd_bf16 = _default.linear_fwd_bf16
linear_bwd_bf16 = _default.linear_bwd_bf16
linear_sample_bf16 = _default.linear_sample_bf16
embedding_fwd_bf16 = _default.embedding_fwd_bf16
embedding_bwd_bf16 = _default.embedding_bwd_bf16
edo_v1_f32 = _default.edo_v1_f32
