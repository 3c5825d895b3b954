"""Physical layouts of one logical token multiset (the gradient-invariance cells).

A *cell* is one way the same logical samples reach the operator: a list of
operator calls, each with its physical rows and a ``row_logical`` map
(physical row -> canonical logical index, -1 for padding).  The canonical
index of token ``pos`` of sample ``s`` is ``off[s] + pos`` with ``off`` the
exclusive prefix sum of the lengths in sample_id order; for a per-head norm
row ``(token, head)`` is ``token * heads + head``.

Cells follow "WS1 C4 (#270) closeout evidence", section "The matrix is
falsifiable": B=N full is one call, chunked splits the same rows over several
calls, the singleton aggregate issues one call per sample, padding rows reach
the operator, and the permuted cell presents samples in another order.
Readings of the chunk list (the page prints chunk sizes 7,4,7,7,2,7,6,7,7,5
for samples of lengths 11,7,13,9,5,14):
  A ("packed"): cut the packed token stream (sample_id order) at those sizes;
  B ("per_sample"): split each sample into pieces of at most 7 tokens and
     issue samples in the order 0,1,3,2,5,4.
Both reproduce the printed list; both are built and both must be green.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from .inputs import Workload, pad_run_lengths, sample_permutation, token_offsets

PAGE_CHUNK_SIZES = (7, 4, 7, 7, 2, 7, 6, 7, 7, 5)
PAGE_CHUNK_ORDER_B = (0, 1, 3, 2, 5, 4)


@dataclasses.dataclass
class Call:
    name: str
    row_logical: Optional[np.ndarray]   # int32[rows]; None = identity map
    rows: int

    @property
    def n_pad(self) -> int:
        return 0 if self.row_logical is None else int((self.row_logical < 0).sum())


@dataclasses.dataclass
class Cell:
    name: str
    calls: List[Call]
    n_logical: int
    heads: int = 1

    @property
    def call_shapes(self):
        return [c.rows for c in self.calls]


def _expand_heads(tok_logical: np.ndarray, heads: int) -> np.ndarray:
    """Token-level map -> row-level map with ``heads`` rows per token."""
    tok_logical = np.asarray(tok_logical, dtype=np.int64)
    if heads == 1:
        return tok_logical.astype(np.int32)
    h = np.arange(heads, dtype=np.int64)
    rows = np.where(tok_logical[:, None] < 0, -1, tok_logical[:, None] * heads + h[None, :])
    return rows.reshape(-1).astype(np.int32)


def _call(name: str, tok_logical: np.ndarray, heads: int) -> Call:
    rl = _expand_heads(tok_logical, heads)
    return Call(name, rl, len(rl))


def _sample_tokens(wl: Workload, s: int) -> np.ndarray:
    off = token_offsets(wl.lengths)
    return np.arange(off[s], off[s + 1], dtype=np.int64)


def full(wl: Workload) -> Cell:
    """BN/full: one call, identity map."""
    return Cell("BN/full", [Call("all", None, wl.n_logical)], wl.n_logical, wl.heads)


def chunked_packed(wl: Workload, sizes: Optional[Sequence[int]] = None,
                   chunk: Optional[int] = None, name: str = "BN/chunked") -> Cell:
    """Reading A: cut the packed token stream at the given sizes (or every
    ``chunk`` tokens)."""
    T = wl.n_tokens
    if sizes is None:
        assert chunk and chunk > 0
        sizes = [min(chunk, T - a) for a in range(0, T, chunk)]
    assert sum(sizes) == T, "chunk sizes must cover the token stream"
    calls, a = [], 0
    for i, n in enumerate(sizes):
        calls.append(_call(f"c{i}", np.arange(a, a + n), wl.heads))
        a += n
    return Cell(name, calls, wl.n_logical, wl.heads)


def chunked_per_sample(wl: Workload, chunk: int, order: Optional[Sequence[int]] = None,
                       name: str = "BN/chunked_per_sample") -> Cell:
    """Reading B: chunked prefill -- each sample split into pieces of at most
    ``chunk`` tokens, samples issued in ``order``."""
    order = list(range(wl.n_samples)) if order is None else list(order)
    assert sorted(order) == list(range(wl.n_samples))
    calls = []
    for s in order:
        toks = _sample_tokens(wl, s)
        for i, a in enumerate(range(0, len(toks), chunk)):
            calls.append(_call(f"s{s}c{i}", toks[a:a + chunk], wl.heads))
    return Cell(name, calls, wl.n_logical, wl.heads)


def singleton_aggregate(wl: Workload, order: Optional[Sequence[int]] = None,
                        name: str = "B1-singleton_aggregate/full") -> Cell:
    """N x B=1: one call per sample, all aggregated into one dweight."""
    order = list(range(wl.n_samples)) if order is None else list(order)
    calls = [_call(f"s{s}", _sample_tokens(wl, s), wl.heads) for s in order]
    return Cell(name, calls, wl.n_logical, wl.heads)


def padded(wl: Workload, total_tokens: int, side: str) -> Cell:
    """BN/padded_right or BN/padded_left: one call of ``total_tokens`` token
    rows, the real rows in order and the padding after or before them."""
    assert side in ("right", "left")
    T = wl.n_tokens
    assert total_tokens >= T
    pads = np.full(total_tokens - T, -1, dtype=np.int64)
    real = np.arange(T, dtype=np.int64)
    tok = np.concatenate([real, pads] if side == "right" else [pads, real])
    return Cell(f"BN/padded_{side}", [_call("all", tok, wl.heads)], wl.n_logical, wl.heads)


def permuted(wl: Workload, perm: Optional[Sequence[int]] = None, name: str = "BN/permuted") -> Cell:
    """One call with samples in a permuted order (default: seeded shuffle)."""
    perm = sample_permutation(wl.seed, wl.n_samples) if perm is None else np.asarray(perm)
    tok = np.concatenate([_sample_tokens(wl, int(s)) for s in perm])
    return Cell(name, [_call("all", tok, wl.heads)], wl.n_logical, wl.heads)


def packed_with_padding(wl: Workload, perm: Optional[Sequence[int]] = None,
                        name: str = "BN/packed_padded_permuted") -> Cell:
    """One call: samples in permuted order, each followed by its run of
    padding rows (run lengths: a seeded composition of ``wl.pad_rows``)."""
    perm = sample_permutation(wl.seed, wl.n_samples) if perm is None else np.asarray(perm)
    runs = pad_run_lengths(wl)
    parts = []
    for k, s in enumerate(perm):
        parts.append(_sample_tokens(wl, int(s)))
        parts.append(np.full(runs[k], -1, dtype=np.int64))
    tok = np.concatenate(parts)
    return Cell(name, [_call("all", tok, wl.heads)], wl.n_logical, wl.heads)


def page_matrix(wl: Workload, pad_to: int = 80) -> List[Cell]:
    """The cells of the hidden=8 matrix on the page, plus the reverse order
    and the reading-B chunking."""
    rev = list(range(wl.n_samples))[::-1]
    return [
        full(wl),
        chunked_packed(wl, sizes=PAGE_CHUNK_SIZES, name="BN/chunked"),
        chunked_per_sample(wl, chunk=7, order=PAGE_CHUNK_ORDER_B, name="BN/chunked_per_sample"),
        singleton_aggregate(wl),
        singleton_aggregate(wl, order=sample_permutation(wl.seed ^ 0x5A5A, wl.n_samples),
                            name="B1-singleton_aggregate/shuffled_calls"),
        padded(wl, pad_to, "right"),
        padded(wl, pad_to, "left"),
        permuted(wl),
        permuted(wl, perm=rev, name="BN/permuted_reverse"),
    ]


def gather_physical(logical: np.ndarray, call: Call, pad_value=0) -> np.ndarray:
    """Physical input of one call from a logical-order array (rows on axis 0);
    padding rows are filled with ``pad_value``."""
    if call.row_logical is None:
        return logical[: call.rows]
    rl = call.row_logical.astype(np.int64)
    out = np.empty((call.rows,) + logical.shape[1:], dtype=logical.dtype)
    real = rl >= 0
    out[real] = logical[rl[real]]
    out[~real] = pad_value
    return out


def standard_matrix(wl: Workload, chunk: int, pad_extra: int = 37) -> List[Cell]:
    """Every layout family for one logical multiset: B=N, chunked (both
    readings), singleton aggregate (in order and reversed), padded right and
    left, permuted (seeded and reversed), and -- when the workload has padding
    rows -- the packed layout with padding runs."""
    T = wl.n_tokens
    rev = list(range(wl.n_samples))[::-1]
    cells = [
        full(wl),
        chunked_packed(wl, chunk=chunk, name="BN/chunked"),
        chunked_per_sample(wl, chunk=chunk, name="BN/chunked_per_sample"),
        singleton_aggregate(wl),
        singleton_aggregate(wl, order=rev, name="B1-singleton_aggregate/reversed_calls"),
        padded(wl, T + pad_extra, "right"),
        padded(wl, T + pad_extra, "left"),
        permuted(wl),
        permuted(wl, perm=rev, name="BN/permuted_reverse"),
    ]
    if wl.pad_rows:
        cells.append(packed_with_padding(wl))
    return cells

