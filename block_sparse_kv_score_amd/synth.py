"""Seeded synthetic inputs for the decode-step workloads.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic.  Both the HIP path (via its tests and benchmark)
and the float64 oracle consume the exact same bits from here.

Recipe (per workload ``w`` and base seed ``seed``):

* every tensor kind has its own stream, and key/value/logit streams are
  drawn per (b, h) from ``SeedSequence([seed, w.wid, stream, b, h, ...])``
  (PCG64), so any single (b, h) pair can be regenerated alone;
* keys, values and queries are N(0, 1) in float32, rounded once to bfloat16
  (round to nearest even) and kept as uint16 bit patterns;
* heavy-hitter keys: each key row is independently (Bernoulli(heavy_frac))
  scaled by heavy_scale in float32 before the rounding;
* eviction logits are float32 N(0, e_sigma^2);
* prefill tokens and appended tokens come from separate streams; the query
  of decode step t comes from its own stream;
* physical page ids are one seeded random permutation of all pages;
* two-level tables allocate 2^seg_log2-entry segments in a seeded random
  order; packed deferred-RoPE tables place the documents of each sequence in
  a seeded random order.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .workloads import (TABLE_FLAT, TABLE_PACKED_ROPE, TABLE_TWO_LEVEL,
                        Workload)

# stream ids
S_K, S_V, S_E, S_HEAVY = 1, 2, 3, 4
S_K_APP, S_V_APP, S_E_APP, S_HEAVY_APP = 11, 12, 13, 14
S_Q = 20
S_PAGES, S_SEGS, S_DOCS = 30, 31, 32
S_EHEAD = 40
S_QP = 41

PACK_PAGE_BITS = 20   # packed word: page id in bits 0..19
PACK_PAGE_MASK = (1 << PACK_PAGE_BITS) - 1


def rng_for(seed: int, w: Workload, stream: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.wid, stream, *idx])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    uint16 bit patterns.  Inputs here are finite and far from overflow."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# per-(b, h) token streams
# ---------------------------------------------------------------------------

def _tokens(w: Workload, seed: int, b: int, h: int, n: int, appended: bool):
    sk, sv, se, sh = (S_K_APP, S_V_APP, S_E_APP, S_HEAVY_APP) if appended else (S_K, S_V, S_E, S_HEAVY)
    K = rng_for(seed, w, sk, b, h).standard_normal((n, w.D), dtype=np.float32)
    if w.heavy_frac > 0:
        hit = rng_for(seed, w, sh, b, h).random(n) < w.heavy_frac
        K[hit] *= np.float32(w.heavy_scale)
    V = rng_for(seed, w, sv, b, h).standard_normal((n, w.D), dtype=np.float32)
    e = rng_for(seed, w, se, b, h).standard_normal(n, dtype=np.float32) * np.float32(w.e_sigma)
    return f32_to_bf16_bits(K), f32_to_bf16_bits(V), e.astype(np.float32)


def tokens_bh(w: Workload, seed: int, b: int, h: int):
    """Logical token stream of one (b, h): prefill then appended tokens.

    Returns (K bits (T0+A, D) uint16, V bits, e (T0+A,) float32), where row
    T0 + t - 1 is the token appended at decode step t.
    """
    Kp, Vp, ep = _tokens(w, seed, b, h, w.T0, appended=False)
    if w.n_append:
        Ka, Va, ea = _tokens(w, seed, b, h, w.n_append, appended=True)
        return (np.concatenate([Kp, Ka]), np.concatenate([Vp, Va]), np.concatenate([ep, ea]))
    return Kp, Vp, ep


def queries(w: Workload, seed: int, step: int) -> np.ndarray:
    """Query bits (B, Hq, D) uint16 of decode step ``step`` (1-based)."""
    q = rng_for(seed, w, S_Q, step).standard_normal((w.B, w.Hq, w.D), dtype=np.float32)
    return f32_to_bf16_bits(q)


# ---------------------------------------------------------------------------
# page tables
# ---------------------------------------------------------------------------

def prefill_queries(w: Workload, seed: int) -> np.ndarray:
    """The prompt's queries (unrotated), (B, prompt, Hq, D) bf16 bits."""
    q = rng_for(seed, w, S_QP).standard_normal((w.B, w.prompt, w.Hq, w.D), dtype=np.float32)
    return f32_to_bf16_bits(q)


def alibi_slopes(n_heads: int) -> np.ndarray:
    """Per-head ALiBi slopes for the synthetic runs (an input of the
    ALiBi decode, like the queries): 2^(-8 (j + 1) / n_heads), float32."""
    return np.power(2.0, -8.0 * (np.arange(n_heads) + 1.0) / n_heads).astype(np.float32)


def eviction_head_weights(w: Workload, seed: int) -> np.ndarray:
    """Random-init eviction-head weights, fp32 [Hkv, D] ~ N(0, 1/D) (an
    input of the fused QKV append, like the projection rows)."""
    g = rng_for(seed, w, S_EHEAD)
    return (g.standard_normal((w.Hkv, w.D), dtype=np.float32) / np.float32(math.sqrt(w.D))).astype(np.float32)


def qkv_rows(w: Workload, inp: "Inputs", step: int) -> np.ndarray:
    """The fused projection rows of decode step ``step``: per sequence
    [q heads | k heads | v heads] of the appended token, bf16 bits
    [B, (Hq + 2 Hkv) D] (the same query and appended k, v as the separate
    inputs)."""
    pos = w.T0 + step - 1
    q = inp.q(step).reshape(w.B, w.Hq * w.D)
    k = inp.K[:, :, pos].reshape(w.B, w.Hkv * w.D)
    v = inp.V[:, :, pos].reshape(w.B, w.Hkv * w.D)
    return np.ascontiguousarray(np.concatenate([q, k, v], axis=1))


def page_ids(w: Workload, seed: int) -> np.ndarray:
    """(B, Hkv, max_blocks) int32 physical page of each *storage* block: a
    random permutation of range(num_pages)."""
    perm = rng_for(seed, w, S_PAGES).permutation(w.num_pages).astype(np.int32)
    return perm.reshape(w.B, w.Hkv, w.max_blocks)


def doc_order(w: Workload, seed: int, b: int) -> np.ndarray:
    """Deferred-RoPE workload: which stored document sits in each slot of
    sequence b's context (a random permutation of range(n_docs))."""
    return rng_for(seed, w, S_DOCS, b).permutation(w.n_docs).astype(np.int64)


def logical_pages(w: Workload, seed: int) -> np.ndarray:
    """(B, Hkv, max_blocks) page of each *logical* block.  For the packed
    deferred-RoPE workload, logical block i of sequence b is block i % bpd of
    the document in slot i // bpd; documents are stored in document order."""
    pages = page_ids(w, seed)
    if w.table != TABLE_PACKED_ROPE:
        return pages
    bpd = w.doc_len // w.bs
    out = np.empty_like(pages)
    for b in range(w.B):
        order = doc_order(w, seed, b)
        for i in range(w.max_blocks):
            out[b, :, i] = pages[b, :, order[i // bpd] * bpd + i % bpd]
    return out


def block_doc_start(w: Workload) -> np.ndarray:
    """(max_blocks,) first logical block of the document holding block i
    (documents tile the context in slots of doc_len tokens)."""
    bpd = w.doc_len // w.bs
    return (np.arange(w.max_blocks) // bpd) * bpd


def packed_table(w: Workload, seed: int) -> np.ndarray:
    """(B, Hkv, max_blocks) uint32: page id | (document start block << 20)."""
    pages = logical_pages(w, seed).astype(np.uint32)
    start = block_doc_start(w).astype(np.uint32)
    assert int(pages.max()) <= PACK_PAGE_MASK and int(start.max()) < (1 << (32 - PACK_PAGE_BITS))
    return pages | (start[None, None, :] << np.uint32(PACK_PAGE_BITS))


def two_level_tables(w: Workload, seed: int):
    """Directory (dir_entries,) int32 and segments (n_seg, 2^seg_log2) int32
    for key = ((b*Hkv + h) << blocks_log2) | i.  Unused entries are -1."""
    pages = logical_pages(w, seed)
    seg_n = 1 << w.seg_log2
    per_bh = -(-w.max_blocks // seg_n)
    dir_needed = (w.B * w.Hkv << w.blocks_log2) >> w.seg_log2
    assert w.dir_entries >= dir_needed, (w.dir_entries, dir_needed)
    n_seg = w.B * w.Hkv * per_bh
    seg_ids = rng_for(seed, w, S_SEGS).permutation(n_seg).astype(np.int32)
    directory = np.full(w.dir_entries, -1, dtype=np.int32)
    segments = np.full((n_seg, seg_n), -1, dtype=np.int32)
    sid = 0
    for bh in range(w.B * w.Hkv):
        b, h = divmod(bh, w.Hkv)
        for s in range(per_bh):
            d = (bh << (w.blocks_log2 - w.seg_log2)) + s
            directory[d] = seg_ids[sid]
            lo, hi = s * seg_n, min((s + 1) * seg_n, w.max_blocks)
            segments[seg_ids[sid], : hi - lo] = pages[b, h, lo:hi]
            sid += 1
    return directory, segments


# ---------------------------------------------------------------------------
# whole-workload bundle
# ---------------------------------------------------------------------------

@dataclass
class Inputs:
    w: Workload
    seed: int
    K: np.ndarray            # (B, Hkv, T0 + A, D) uint16, logical order
    V: np.ndarray
    e: np.ndarray            # (B, Hkv, T0 + A) float32
    pages: np.ndarray        # (B, Hkv, max_blocks) int32, logical block -> page
    directory: np.ndarray | None = None
    segments: np.ndarray | None = None
    packed: np.ndarray | None = None
    q_pos: np.ndarray | None = None   # (B,) int32 query position (deferred RoPE)
    extra: dict = field(default_factory=dict)

    def q(self, step: int) -> np.ndarray:
        return queries(self.w, self.seed, step)


def generate(w: Workload, seed: int = 0) -> Inputs:
    """All inputs of a workload (every (b, h) pair), generated in parallel."""
    T = w.T0 + w.n_append
    K = np.empty((w.B, w.Hkv, T, w.D), dtype=np.uint16)
    V = np.empty_like(K)
    e = np.empty((w.B, w.Hkv, T), dtype=np.float32)

    def fill(bh):
        b, h = divmod(bh, w.Hkv)
        K[b, h], V[b, h], e[b, h] = tokens_bh(w, seed, b, h)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(w.B * w.Hkv)))
    inp = Inputs(w, seed, K, V, e, logical_pages(w, seed))
    if w.table == TABLE_TWO_LEVEL:
        inp.directory, inp.segments = two_level_tables(w, seed)
    elif w.table == TABLE_PACKED_ROPE:
        inp.packed = packed_table(w, seed)
        inp.q_pos = np.full(w.B, w.T0, dtype=np.int32)
    else:
        assert w.table == TABLE_FLAT
    return inp
