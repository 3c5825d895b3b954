"""Seeded synthetic inputs: workload shapes and counter-based tensor generators.

This module is shared by the HIP path's tests/benchmark and by the oracle's
tests.  It holds none of RMSNorm's arithmetic: it only defines *what the
inputs are* (shapes, sample lengths, padding/mask structure and the bits of
x, w and dy), keyed by logical identity (sample_id, token_pos[, head], col)
so that every physical layout of the same logical multiset sees the same
bits ("[WS1 Closeout][Backward] Reusable gradient-invariance harness and
operator adapters", section Scope: the upstream gradient and active-token
denominator are fixed across configs; "WS1 C4 (#270) closeout evidence",
Acceptance map: dy depends on nothing but the logical identity of the row).

Generator: the SplitMix64 output function (Steele, Lea, Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014) applied to a packed
64-bit counter.  Tensors are generated with integer torch ops plus single
correctly rounded float conversions and one float32 multiply, so CPU and GPU
generation give the same bits (checked by a GPU test).

Distributions (the input recipe):
  x  : Irwin-Hall sum of four 16-bit uniforms, standardised -> approx N(0,1)
       (support +-3.46), rounded to bf16 (round to nearest even)
  w  : U[0.5, 1.5) from 24 bits, rounded to bf16
  dy : active * U[-1, 1) / N_active, rounded to bf16; N_active = number of
       active tokens of the whole logical multiset (mean over active tokens)
  mask (density < 1): Bernoulli(density) per (sample, pos)
  W  (linear-layer workloads, [out, in]): U[-1, 1) / sqrt(in), rounded to bf16
  ids (embedding workloads): token of each logical row drawn from a Zipf law
       P(rank k) ~ 1/k^s over the vocabulary (inverse CDF of a 53-bit uniform)
  E  (embedding table, [vocab, dim]): U[-1, 1) * 2^-5, rounded to bf16
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

MASK64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# Tensor tags of the counter (8 bits).
TAG_X, TAG_W, TAG_DY, TAG_MASK, TAG_LEN, TAG_COMP, TAG_PERM, TAG_PADCOMP = 1, 2, 3, 4, 5, 6, 7, 8
TAG_WMAT = 9       # weight matrix of a linear-layer workload
TAG_TABLE, TAG_IDS = 10, 11   # embedding table and token ids of an embedding workload
TAG_K_OFFSET = 16  # K-side tensors of a QK-norm workload use tag + 16


def _signed(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


# ----------------------------------------------------------------- scalar (host)
def mix64(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def seed_mix(seed: int) -> int:
    return mix64(seed + _GOLDEN)


def pack_key(tag: int, s: int = 0, p: int = 0, h: int = 0, col: int = 0) -> int:
    """64-bit counter: tag 8b | sample 10b | pos 18b | head 6b | col 16b."""
    assert 0 <= tag < 256 and 0 <= s < 1024 and 0 <= p < (1 << 18)
    assert 0 <= h < 64 and 0 <= col < (1 << 16)
    return (tag << 50) | (s << 40) | (p << 22) | (h << 16) | col


def hash64(seed: int, key: int) -> int:
    return mix64(key ^ seed_mix(seed))


# ------------------------------------------------------------- vector (torch)
def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def mix64_t(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output function on int64 tensors (wrapping arithmetic)."""
    z = (z ^ _lsr(z, 30)) * _signed(_M1)
    z = (z ^ _lsr(z, 27)) * _signed(_M2)
    return z ^ _lsr(z, 31)


def _f32_to_bf16_bits(f: torch.Tensor) -> torch.Tensor:
    """Round finite float32 values to bf16 (nearest even); returns int64 bits."""
    b = f.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    return (b + 0x7FFF + ((b >> 16) & 1)) >> 16


def _bits_to_bf16_tensor(bits: torch.Tensor) -> torch.Tensor:
    b = torch.where(bits >= 32768, bits - 65536, bits).to(torch.int16)
    return b.view(torch.bfloat16)


# ------------------------------------------------------------------ workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: logical samples of tokens, each token one row
    (or ``heads`` rows for a per-head norm), hidden size ``hidden``."""
    name: str
    hidden: int
    lengths: Tuple[int, ...]          # logical sample lengths, in sample_id order
    seed: int
    eps: float = 1e-6
    heads: int = 1                    # rows per token (per-head norm when > 1)
    tag_offset: int = 0               # separates the Q and K tensors of a QK-norm
    mask_density: float = 1.0         # fraction of active tokens
    pad_rows: int = 0                 # padding rows of the packed physical layout
    out_features: int = 0             # linear-layer workloads: N (hidden is the input width K)
    vocab: int = 0                    # embedding workloads: table rows (hidden is the row width)
    zipf_s: float = 1.1               # embedding workloads: token frequency exponent
    description: str = ""

    @property
    def n_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def n_logical(self) -> int:
        return self.n_tokens * self.heads

    @property
    def n_samples(self) -> int:
        return len(self.lengths)

    @property
    def dy_cols(self) -> int:
        """Columns of the upstream gradient: the output width."""
        return self.out_features or self.hidden


def token_offsets(lengths: Sequence[int]) -> np.ndarray:
    """Exclusive prefix sum of the sample lengths (sample_id order)."""
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return off


def _varlen_lengths(seed: int, n: int, lo: int, hi: int) -> Tuple[int, ...]:
    """n integer lengths, uniform on [lo, hi] inclusive."""
    span = hi - lo + 1
    return tuple(lo + (hash64(seed, pack_key(TAG_LEN, s)) >> 33) % span for s in range(n))


def _composition(seed: int, tag: int, total: int, parts: int, positive: bool) -> Tuple[int, ...]:
    """Seeded composition of ``total`` into ``parts`` parts (each > 0 if positive)."""
    cuts: List[int] = []
    seen = set()
    i = 0
    while len(cuts) < parts - 1:
        hv = hash64(seed, pack_key(tag, 0, i))
        i += 1
        if positive:
            c = 1 + (hv >> 33) % (total - 1)
            if c in seen:
                continue
            seen.add(c)
        else:
            c = (hv >> 33) % (total + 1)
        cuts.append(c)
    cuts.sort()
    edges = [0] + cuts + [total]
    return tuple(edges[k + 1] - edges[k] for k in range(parts))


def sample_permutation(seed: int, n: int, tag: int = TAG_PERM) -> np.ndarray:
    """Seeded permutation of sample ids (argsort of per-sample hashes)."""
    keys = [hash64(seed, pack_key(tag, s)) for s in range(n)]
    return np.argsort(np.asarray(keys, dtype=np.uint64), kind="stable").astype(np.int64)


def pad_run_lengths(wl: Workload) -> Tuple[int, ...]:
    """Padding rows after each sample in the packed layout (sum = pad_rows)."""
    if wl.pad_rows == 0:
        return tuple(0 for _ in wl.lengths)
    return _composition(wl.seed, TAG_PADCOMP, wl.pad_rows, wl.n_samples, positive=False)


def _seed(cfg: int) -> int:
    return 0x1A7E0000 + cfg


def workload_h8() -> Workload:
    return Workload("rmsnorm_h8_t59", 8, (11, 7, 13, 9, 5, 14), _seed(1),
                    description="hidden 8, 6 samples, 59 rows")


def workload_h4096() -> Workload:
    return Workload("rmsnorm_h4096_t32768", 4096, (4096,) * 8, _seed(2),
                    description="hidden 4096, 8 x 4096 tokens, all active")


def workload_h8192() -> Workload:
    return Workload("rmsnorm_h8192_varlen16", 8192, _varlen_lengths(_seed(3), 16, 512, 8192),
                    _seed(3), description="hidden 8192, 16 samples of U[512,8192] tokens")


def workload_qk(side: str) -> Workload:
    assert side in ("q", "k")
    heads = 32 if side == "q" else 8
    return Workload(f"qknorm_d128_t16384_{side}", 128, (4096,) * 4, _seed(4), heads=heads,
                    tag_offset=0 if side == "q" else TAG_K_OFFSET,
                    description=f"per-head norm, head_dim 128, {heads} heads, 4 x 4096 tokens")


def workload_h5120() -> Workload:
    return Workload("rmsnorm_h5120_packed131072", 5120,
                    _composition(_seed(5), TAG_COMP, 98304, 64, positive=True), _seed(5),
                    mask_density=0.5, pad_rows=32768,
                    description="hidden 5120, 64 samples (98304 tokens) + 32768 pad rows, "
                                "mask density 0.5")


def scaled(wl: Workload, name: str, hidden: Optional[int] = None,
           lengths: Optional[Sequence[int]] = None, pad_rows: Optional[int] = None,
           out_features: Optional[int] = None, vocab: Optional[int] = None) -> Workload:
    """A smaller variant of a workload (same seed/recipe) for fast parity runs."""
    return dataclasses.replace(wl, name=name, hidden=hidden or wl.hidden,
                               lengths=tuple(lengths) if lengths is not None else wl.lengths,
                               pad_rows=wl.pad_rows if pad_rows is None else pad_rows,
                               out_features=wl.out_features if out_features is None
                               else out_features,
                               vocab=wl.vocab if vocab is None else vocab)


def workload_linear() -> Workload:
    return Workload("linear_h4096_o4096_t32768", 4096, (4096,) * 8, _seed(6), out_features=4096,
                    description="linear layer 4096 -> 4096, 8 x 4096 tokens, all active")


def workload_lmhead() -> Workload:
    """The LM-head projection of a 32,000-token vocabulary on the same rows:
    det_gemm with N = vocabulary (reading R20)."""
    return Workload("lmhead_v32000_h4096_t32768", 4096, (4096,) * 8, _seed(8), out_features=32000,
                    description="LM head 4096 -> 32000 (vocabulary), 8 x 4096 tokens, all active")


def workload_embedding() -> Workload:
    return Workload("embedding_v32000_d4096_t32768", 4096, (4096,) * 8, _seed(7), vocab=32000,
                    description="embedding 32000 x 4096, 8 x 4096 tokens, Zipf(1.1) token ids")


EMBEDDING_WORKLOADS = {
    "embedding_v32000_d4096_t32768": workload_embedding,
}


LINEAR_WORKLOADS = {
    "linear_h4096_o4096_t32768": workload_linear,
    "lmhead_v32000_h4096_t32768": workload_lmhead,
}


ALL_WORKLOADS = {
    "rmsnorm_h8_t59": workload_h8,
    "rmsnorm_h4096_t32768": workload_h4096,
    "rmsnorm_h8192_varlen16": workload_h8192,
    "qknorm_d128_t16384_q": lambda: workload_qk("q"),
    "qknorm_d128_t16384_k": lambda: workload_qk("k"),
    "rmsnorm_h5120_packed131072": workload_h5120,
}


# ----------------------------------------------------------- logical identity
def logical_keys(wl: Workload, rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, ...]:
    """(sample, pos, head) of the given logical rows (default: all), where the
    logical rows enumerate tokens in (sample_id, token_pos) order and, for a
    per-head norm, heads fastest."""
    T = wl.n_logical
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    tok = rows // wl.heads
    head = rows % wl.heads
    off = token_offsets(wl.lengths)
    s = np.searchsorted(off, tok, side="right") - 1
    p = tok - off[s]
    return s, p, head


def active_mask(wl: Workload, s: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Per-token activity (bool); all True when mask_density == 1."""
    if wl.mask_density >= 1.0:
        return np.ones(len(s), dtype=bool)
    key = ((TAG_MASK + wl.tag_offset) << 50) | (s.astype(np.int64) << 40) | (p.astype(np.int64) << 22)
    hv = mix64_t(torch.from_numpy(key ^ _signed(seed_mix(wl.seed))))
    u = (_lsr(hv, 40).numpy().astype(np.float64)) / float(1 << 24)
    return u < wl.mask_density


def n_active(wl: Workload) -> int:
    """Active-token count of the whole logical multiset (the loss denominator)."""
    off = token_offsets(wl.lengths)
    tok = np.arange(wl.n_tokens, dtype=np.int64)
    s = np.searchsorted(off, tok, side="right") - 1
    p = tok - off[s]
    return int(active_mask(wl, s, p).sum())


# ------------------------------------------------------------- tensor makers
def _row_keys(wl: Workload, tag: int, rows: np.ndarray, device) -> torch.Tensor:
    s, p, h = logical_keys(wl, rows)
    k = ((tag + wl.tag_offset) << 50) | (s << 40) | (p << 22) | (h << 16)
    return torch.from_numpy(k.astype(np.int64)).to(device)


def _hash_rows(wl: Workload, tag: int, rows: np.ndarray, device, ncols: Optional[int] = None
               ) -> torch.Tensor:
    rk = _row_keys(wl, tag, rows, device)
    cols = torch.arange(wl.hidden if ncols is None else ncols, dtype=torch.int64, device=device)
    return mix64_t((rk[:, None] | cols[None, :]) ^ _signed(seed_mix(wl.seed)))


_IH4_SCALE = np.float32(1.0 / (2.0 * math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)))


def gen_x(wl: Workload, rows: Optional[np.ndarray] = None, device="cpu",
          chunk: int = 8192) -> torch.Tensor:
    """x[rows, hidden] (bf16) for the given logical rows (default: all)."""
    rows = np.arange(wl.n_logical, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    out = torch.empty((len(rows), wl.hidden), dtype=torch.bfloat16, device=device)
    scale = torch.tensor(_IH4_SCALE, dtype=torch.float32, device=device)
    for a in range(0, len(rows), chunk):
        z = _hash_rows(wl, TAG_X, rows[a:a + chunk], device)
        tot = (z & 0xFFFF) + (_lsr(z, 16) & 0xFFFF) + (_lsr(z, 32) & 0xFFFF) + _lsr(z, 48)
        centred = (2 * tot - 4 * 65535).to(torch.float32)          # exact (< 2^19)
        f = centred * scale                                          # one rounding
        out[a:a + chunk] = _bits_to_bf16_tensor(_f32_to_bf16_bits(f))
    return out


def gen_w(wl: Workload, device="cpu") -> torch.Tensor:
    """w[hidden] (bf16), U[0.5, 1.5)."""
    key = torch.arange(wl.hidden, dtype=torch.int64, device=device) | ((TAG_W + wl.tag_offset) << 50)
    z = mix64_t(key ^ _signed(seed_mix(wl.seed)))
    u = _lsr(z, 40).to(torch.float64) / float(1 << 24)               # exact
    f = (0.5 + u).to(torch.float32)                                   # one rounding
    return _bits_to_bf16_tensor(_f32_to_bf16_bits(f))


def gen_dy(wl: Workload, rows: Optional[np.ndarray] = None, device="cpu",
           chunk: int = 8192, denominator: Optional[int] = None) -> torch.Tensor:
    """Upstream gradient dy[rows, hidden] (bf16) of the loss
    L = (1/N_active) * sum over active tokens of sum_j u * y."""
    rows = np.arange(wl.n_logical, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    n_act = n_active(wl) if denominator is None else int(denominator)
    s, p, _ = logical_keys(wl, rows)
    act = torch.from_numpy(active_mask(wl, s, p).astype(np.float64)).to(device)
    out = torch.empty((len(rows), wl.dy_cols), dtype=torch.bfloat16, device=device)
    for a in range(0, len(rows), chunk):
        z = _hash_rows(wl, TAG_DY, rows[a:a + chunk], device, wl.dy_cols)
        u = (_lsr(z, 40) - (1 << 23)).to(torch.float64) / float(1 << 23)   # exact, [-1, 1)
        g = (u * act[a:a + chunk, None]) / float(n_act)                       # one rounding
        out[a:a + chunk] = _bits_to_bf16_tensor(_f32_to_bf16_bits(g.to(torch.float32)))
    return out


def gen_wmat(wl: Workload, device="cpu") -> torch.Tensor:
    """Weight matrix W[out_features, hidden] (bf16) of a linear-layer workload,
    U[-1, 1) / sqrt(hidden), keyed by (row, column)."""
    assert wl.out_features > 0
    n, k = wl.out_features, wl.hidden
    rows = torch.arange(n, dtype=torch.int64, device=device)
    cols = torch.arange(k, dtype=torch.int64, device=device)
    key = ((TAG_WMAT + wl.tag_offset) << 50) | (rows[:, None] << 22) | cols[None, :]
    z = mix64_t(key ^ _signed(seed_mix(wl.seed)))
    u = (_lsr(z, 40) - (1 << 23)).to(torch.float64) / float(1 << 23)      # exact, [-1, 1)
    f = (u / math.sqrt(k)).to(torch.float32)                             # one rounding
    return _bits_to_bf16_tensor(_f32_to_bf16_bits(f))


def gen_ids(wl: Workload) -> np.ndarray:
    """Token id (int32) of every logical row of an embedding workload: a
    seeded Zipf(s) draw over the vocabulary keyed by (sample, pos)."""
    assert wl.vocab > 0
    s_, p_, _ = logical_keys(wl)
    key = ((TAG_IDS + wl.tag_offset) << 50) | (s_.astype(np.int64) << 40) | (p_.astype(np.int64) << 22)
    z = mix64_t(torch.from_numpy(key ^ _signed(seed_mix(wl.seed))))
    u = (_lsr(z, 11).numpy().astype(np.float64) + 0.5) / float(1 << 53)    # (0, 1)
    w = 1.0 / np.arange(1, wl.vocab + 1, dtype=np.float64) ** wl.zipf_s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    ids = np.searchsorted(cdf, u, side="left")
    return np.minimum(ids, wl.vocab - 1).astype(np.int32)


def gen_table(wl: Workload, device="cpu") -> torch.Tensor:
    """Embedding table E[vocab, hidden] (bf16), U[-1, 1) * 2^-5, keyed by (row, column)."""
    assert wl.vocab > 0
    rows = torch.arange(wl.vocab, dtype=torch.int64, device=device)
    cols = torch.arange(wl.hidden, dtype=torch.int64, device=device)
    out = torch.empty((wl.vocab, wl.hidden), dtype=torch.bfloat16, device=device)
    for a in range(0, wl.vocab, 4096):
        r = rows[a:a + 4096]
        key = ((TAG_TABLE + wl.tag_offset) << 50) | ((r[:, None] >> 18) << 40) | \
              ((r[:, None] & ((1 << 18) - 1)) << 22) | cols[None, :]
        z = mix64_t(key ^ _signed(seed_mix(wl.seed)))
        u = (_lsr(z, 40) - (1 << 23)).to(torch.float64) / float(1 << 23)
        out[a:a + 4096] = _bits_to_bf16_tensor(_f32_to_bf16_bits((u / 32.0).to(torch.float32)))
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16 tensor (copied to host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
