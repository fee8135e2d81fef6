"""Float64 CPU oracle for one NOSA-style block-sparse decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library or its
Python binding and imports neither.

Everything is plain NumPy in float64, one (sequence b, KV head h) pair at a
time, written the slow, definitional way:

* per-token scores over *every* key (no summaries, no pooling shortcuts);
* sub-block mean, then block max;
* selection by explicit sorting of (score, index) pairs and Python sets;
* softmax attention by its textbook definition over the selected tokens.

Sources (web pages; cited by title and section):

[NOSA]  "NOSA: Native and Offloadable Sparse Attention" technical summary
        (gist.science, paper 2510.13602), Methodology part 1 "Algorithm:
        NOSA" -- bullets *dual-selection mechanism*, *locality guarantee*,
        *block-wise implementation*, *ED-DMA*; Methodology part 2 "System:
        NOSI" -- bullet *optimised memory layout* (set differences for block
        swapping).
[SPIN]  "Unifying Sparse Attention with Hierarchical Memory for Scalable
        Long-Context LLM Serving" summary (gist.science, 2604.26837),
        section 2.A (five-operation pipeline, including Offload and
        Retrieve), 2.B (per-head physical pages),
        2.C (two-level index).
[LAZY]  "LazyAttention" technical summary (gist.science, 2606.04302),
        "Technical implementation -- 2. Decoding" and "Mathematical
        equivalence".
[NOVITA] Novita AI blog "How KV sparsity achieves 1.5x acceleration for
        vLLM", "Key techniques -- 2. Attention modifications" (one-pass
        FlashAttention, returning rowmax and l).

Readings where the pages leave a step open are marked READING in the
docstrings below; each is also listed in the design notes.

Pinning status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py`` (library routines, closed forms, brute force and
invariants) except the selection *semantics* choices marked READING, whose
agreement with the GPU is agreement on the reading: parity unpinned beyond
the reading for those choices (disjoint budgets, initial state, new-block
candidacy, no forced local window, tie order, slot placement of the host
tier, the recency bucket and the in-bucket order of the buffer).
"""

from __future__ import annotations

import math
from typing import Iterable

import numpy as np

__all__ = [
    "bf16_to_f64",
    "num_blocks",
    "block_token_range",
    "subblock_token_ranges",
    "query_token_scores",
    "eviction_token_scores",
    "split_qkv",
    "eviction_head",
    "pool_block_scores",
    "top_by_score",
    "select_blocks",
    "swap_lists",
    "place_blocks",
    "recency_bucket",
    "buffer_retrieve",
    "tokens_of_blocks",
    "split_chunks", "share_chunks",
    "attend",
    "merge_partials",
    "softmax_block_mass",
    "alibi_slopes",
    "alibi_bias",
    "rope_inv_freq",
    "rope_rotate",
    "materialise",
    "attend_blocks",
    "decode_step_bh",
    "prefill_attention_bh",
]


# ---------------------------------------------------------------------------
# Input decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64.

    A bfloat16 number is the upper 16 bits of an IEEE-754 binary32 word, so
    widening the pattern into the high half of a 32-bit word and reading it
    as float32 gives the exact value; float32 -> float64 is exact too.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Index-side inputs  [NOSA, NOSI kernel fusion: the eviction head, the QKV
# split and pooling run in one kernel]
# ---------------------------------------------------------------------------

def split_qkv(row: np.ndarray, Hq: int, Hkv: int, D: int):
    """One token's fused QKV projection row, [q heads | k heads | v heads]
    (READING: the usual concatenated layout), into q (Hq, D), k (Hkv, D)
    and v (Hkv, D)."""
    row = np.asarray(row)
    q = row[:Hq * D].reshape(Hq, D)
    k = row[Hq * D:(Hq + Hkv) * D].reshape(Hkv, D)
    v = row[(Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(Hkv, D)
    return q, k, v


def eviction_head(v: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Eviction logits of the query-agnostic selection [NOSA, dual selection:
    a DMA-inspired eviction head scores tokens independently of the query;
    ED-DMA: no exponent before selection].  READING: per KV head a learned
    linear map of the token's value vector, e = w_h . v, evaluated in
    float64 and stored as float32 (one logit per token and KV head).
    v: (..., D) float64; w: (D,).  Returns float32 logits (...)."""
    return (np.asarray(v, dtype=np.float64) @ np.asarray(w, dtype=np.float64)).astype(np.float32)


# ---------------------------------------------------------------------------
# Blocks and sub-blocks  [NOSA, block-wise implementation]
# ---------------------------------------------------------------------------

def num_blocks(T: int, bs: int) -> int:
    """Number of (possibly partial) blocks covering T tokens."""
    return -(-int(T) // int(bs))


def block_token_range(i: int, T: int, bs: int) -> range:
    """Tokens of logical block i that are present: [i*bs, min((i+1)*bs, T))."""
    return range(i * bs, min((i + 1) * bs, T))


def subblock_token_ranges(i: int, T: int, bs: int, ss: int) -> list[range]:
    """Non-empty sub-blocks of block i, each the present tokens of
    [i*bs + j*ss, i*bs + (j+1)*ss).

    READING: a partial sub-block is averaged over the tokens it has; an empty
    one takes no part in the block maximum.
    """
    out = []
    for j in range(bs // ss):
        lo = i * bs + j * ss
        hi = min(i * bs + (j + 1) * ss, T)
        if lo < hi:
            out.append(range(lo, hi))
    return out


# ---------------------------------------------------------------------------
# Scores  [NOSA, dual selection + block-wise implementation + ED-DMA]
# ---------------------------------------------------------------------------

def query_token_scores(q_group: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Query-aware score of every token: the group mean of q_g . k / sqrt(D).

    q_group: (G, D) float64, the query heads that share this KV head.
    K:       (T, D) float64, every key of the sequence for this KV head.
    Returns (T,) float64.
    """
    G, D = q_group.shape
    per_head = np.empty((G, K.shape[0]), dtype=np.float64)
    for g in range(G):
        per_head[g] = (K @ q_group[g]) / math.sqrt(D)
    return per_head.mean(axis=0)


def eviction_token_scores(e: np.ndarray) -> np.ndarray:
    """Query-agnostic score of every token: its eviction-head logit as is.

    ED-DMA keeps the exponent out of selection, so the raw (pre-exp) logit
    is what gets pooled.  READING: logits are unscaled and are never used as
    an attention bias.
    """
    return np.asarray(e, dtype=np.float64)


def pool_block_scores(token_scores: np.ndarray, T: int, bs: int, ss: int) -> np.ndarray:
    """Two-stage pooling: mean inside each sub-block, then max over the
    sub-blocks of a block.  Returns (nb,) float64 for nb = ceil(T / bs)."""
    nb = num_blocks(T, bs)
    out = np.empty(nb, dtype=np.float64)
    for i in range(nb):
        means = [float(np.mean(token_scores[r.start:r.stop]))
                 for r in subblock_token_ranges(i, T, bs, ss)]
        out[i] = max(means)
    return out


# ---------------------------------------------------------------------------
# Selection  [NOSA, dual selection + locality guarantee]
# ---------------------------------------------------------------------------

def top_by_score(scores: np.ndarray, candidates: Iterable[int], k: int) -> list[int]:
    """The k best candidates under the total order (score descending, index
    ascending).  READING: ties are broken towards the lower block index."""
    order = sorted(candidates, key=lambda i: (-float(scores[i]), int(i)))
    return order[:max(0, int(k))]


def select_blocks(S_q: np.ndarray, E: np.ndarray, nb: int, k_e: int, k_q: int,
                  evicted: set[int]):
    """One step of dual selection.

    Eviction part: the candidates are the blocks that have never been
    dropped; the k_e best by eviction score are kept and every other
    candidate is dropped for good (a block left out once never comes back to
    this part).  Query part: the k_q best by query-aware score among the
    blocks the eviction part did not take.

    READINGS: the two parts are disjoint, so the union has min(k_e+k_q, nb)
    blocks; the never-return rule binds only the eviction part (the query
    part may still fetch a dropped block); a block created this step starts
    as a candidate.

    Returns (gamma_e, gamma_q, gamma, evicted_after), the first three as
    ascending lists, the last as a new set.
    """
    cand = [i for i in range(nb) if i not in evicted]
    gamma_e = set(top_by_score(E, cand, min(k_e, len(cand))))
    evicted_after = set(evicted) | (set(cand) - gamma_e)
    rest = [i for i in range(nb) if i not in gamma_e]
    gamma_q = set(top_by_score(S_q, rest, min(k_q, len(rest))))
    gamma = sorted(gamma_e | gamma_q)
    return sorted(gamma_e), sorted(gamma_q), gamma, evicted_after


def swap_lists(prev: Iterable[int], cur: Iterable[int]):
    """Set differences for block swapping [NOSA, NOSI memory layout]:
    blocks to bring in (cur minus prev) and blocks to drop (prev minus cur),
    both ascending."""
    p, c = set(int(x) for x in prev), set(int(x) for x in cur)
    return sorted(c - p), sorted(p - c)


def place_blocks(owner: list[int], drop: Iterable[int], load: Iterable[int]):
    """Resident slots of one (b, h) pair after a block swap, for the host
    tier where HBM holds a fixed number of page slots per pair [NOSA, NOSI
    memory layout: set differences drive block swapping; SPIN 2.A: Offload
    and Retrieve move pages between host memory and the GPU].

    owner: owner[s] is the block held by slot s, or -1 for a free slot.
    Every slot holding a dropped block is freed; then the blocks to load
    take free slots.

    READING: the pages fix which blocks move, not where they land.  Here
    the j-th block of the load list takes the j-th free slot in ascending
    slot order (counted after the drops), so placement is deterministic.

    Returns (new_owner, placed): loads past the last free slot are not
    placed (placed < len(load) is a capacity error for the caller).
    """
    dropped = set(int(x) for x in drop)
    new = [-1 if int(x) in dropped else int(x) for x in owner]
    free = [s for s, x in enumerate(new) if x < 0]
    load = [int(x) for x in load]
    for s, x in zip(free, load):
        new[s] = x
    return new, min(len(free), len(load))


RECENCY_BUCKETS = 64


def recency_bucket(age: int, width: int) -> int:
    """Recency bucket of a buffered page last selected `age` >= 1 steps ago:
    buckets of `width` steps, the last one open-ended [SPIN 2.B, bucketed
    LRU over recency timestamps, e.g. 64 buckets].  READING: the timestamp
    is the step at which the page was last selected; bucket 0 holds the
    most recent pages."""
    return min((max(int(age), 1) - 1) // int(width), RECENCY_BUCKETS - 1)


def buffer_retrieve(owner: list[int], last_use: list[int], sel: Iterable[int], t: int, width: int):
    """One step of the host tier with a locality-aware buffer [SPIN 2.B:
    the per-request GPU buffer holds the pages this step needs and buffered
    pages kept for temporal locality; buffered pages are evicted by a
    bucketed LRU instead of a global LRU].

    owner[s]: block in slot s or -1; last_use[s]: step at which that block
    was last selected.  sel: this step's selection (ascending).  Steps:
      1. a selected block already in a slot is a hit: its slot's timestamp
         becomes t;
      2. the selected blocks not in any slot are the misses (in selection
         order);
      3. if the free slots are too few, buffered pages (resident, not
         selected) are dropped oldest bucket first; READING: inside the
         bucket where dropping stops, lowest slot first;
      4. the misses take the free slots as in place_blocks (the j-th miss
         the j-th free slot in ascending order), timestamp t.

    Returns (owner, last_use, misses, dropped, placed): new lists, the
    missed blocks, the blocks dropped from the buffer, and how many misses
    found a slot.
    """
    owner = [int(x) for x in owner]
    last_use = [int(x) for x in last_use]
    sel = [int(x) for x in sel]
    slot_of = {x: s for s, x in enumerate(owner) if x >= 0}
    for x in sel:
        if x in slot_of:
            last_use[slot_of[x]] = int(t)
    misses = [x for x in sel if x not in slot_of]
    n_free = sum(1 for x in owner if x < 0)
    chosen = set(sel)
    buffered = [s for s, x in enumerate(owner) if x >= 0 and x not in chosen]
    order = sorted(buffered, key=lambda s: (-recency_bucket(t - last_use[s], width), s))
    dropped = [owner[s] for s in order[:max(0, len(misses) - n_free)]]
    owner, placed = place_blocks(owner, dropped, misses)
    for s, x in enumerate(owner):
        if x in set(misses[:placed]):
            last_use[s] = int(t)
    return owner, last_use, misses, dropped, placed


# ---------------------------------------------------------------------------
# Attention  [NOVITA, attention modifications; split-K merge]
# ---------------------------------------------------------------------------

def tokens_of_blocks(blocks: Iterable[int], T: int, bs: int) -> np.ndarray:
    """Present token indices of the given logical blocks, in block order."""
    toks: list[int] = []
    for i in blocks:
        toks.extend(block_token_range(int(i), T, bs))
    return np.asarray(toks, dtype=np.int64)


def split_chunks(sel: list[int], P: int) -> list[list[int]]:
    """Cut a selected-block list into P contiguous chunks of ceil(n/P)
    blocks (trailing chunks may be empty).  READING: the split layout is
    not on the pages; any contiguous partition merges to the same result."""
    n = len(sel)
    c = -(-n // P) if n else 0
    return [list(sel[p * c:(p + 1) * c]) if c else [] for p in range(P)]


def share_chunks(gamma_e: list[int], gamma_q: list[int], P: int) -> list[list[int]]:
    """Another split layout: chunk p holds the p-th of P equal shares, in
    whole blocks, of each part of the selection, eviction blocks
    gamma_e[p n_e / P : (p+1) n_e / P] then query blocks
    gamma_q[p n_q / P : (p+1) n_q / P] (integer division).  READING: as for
    split_chunks, the pages fix no layout; the fused select + decode uses
    this one on steps where the eviction part keeps every block it has not
    dropped, so that each split can start on its eviction share before the
    query part is known."""
    ne, nq = len(gamma_e), len(gamma_q)
    return [list(gamma_e[p * ne // P:(p + 1) * ne // P]) + list(gamma_q[p * nq // P:(p + 1) * nq // P])
            for p in range(P)]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, bias: np.ndarray | None = None):
    """Softmax attention of each query row over the given keys/values.

    s = scale * q . k (+ bias); m = max s; l = sum exp(s - m);
    O = sum exp(s - m) v / l.  q: (G, D); K, V: (n, D); bias: (G, n) or
    None.  Returns O (G, D), m (G,), l (G,).  With no tokens: O = 0,
    m = -inf, l = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    G, D = q.shape
    n = K.shape[0]
    if n == 0:
        return np.zeros((G, D)), np.full(G, -np.inf), np.zeros(G)
    s = (q @ np.asarray(K, dtype=np.float64).T) * scale
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    O = (p @ np.asarray(V, dtype=np.float64)) / l[:, None]
    return O, m, l


def merge_partials(o_parts: np.ndarray, m_parts: np.ndarray, l_parts: np.ndarray):
    """Merge per-split (o, m, l) triples, o already divided by its own l.

    m = max over splits with l > 0; w_p = l_p exp(m_p - m); l = sum w_p;
    O = sum w_p o_p / l.  o_parts (P, D), m_parts (P,), l_parts (P,).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m_parts = np.asarray(m_parts, dtype=np.float64)
    l_parts = np.asarray(l_parts, dtype=np.float64)
    live = l_parts > 0
    if not live.any():
        return np.zeros(o_parts.shape[1]), -np.inf, 0.0
    m = m_parts[live].max()
    w = l_parts[live] * np.exp(m_parts[live] - m)
    l = w.sum()
    O = (w[:, None] * o_parts[live]).sum(axis=0) / l
    return O, float(m), float(l)


def softmax_block_mass(q: np.ndarray, K: np.ndarray, blocks: list[int], T: int, bs: int, scale: float):
    """The online-softmax score step [NOVITA, 2. Attention modifications:
    with the returned row max and l, p = exp(q.k - rowmax) / l is each key's
    softmax score, and a row-wise sum turns it into a sparsification score].

    Softmax over the tokens of the given blocks, computed by its definition
    (max, exponentials, sum, divide); then, for every query row and block,
    the sum of that row's probabilities over the block's tokens.  READING:
    in a decode step the rows are the group's query heads, the sum runs over
    each selected block's present tokens, and the result stays per head.

    q: (G, D); K: (>=T, D) keys in logical order.  Returns (G, len(blocks)).
    """
    q = np.asarray(q, dtype=np.float64)
    G = q.shape[0]
    out = np.zeros((G, len(blocks)))
    toks = tokens_of_blocks(blocks, T, bs)
    if len(toks) == 0:
        return out
    s = (q @ np.asarray(K, dtype=np.float64)[toks].T) * scale      # (G, n)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    start = 0
    for j, i in enumerate(blocks):
        n = len(block_token_range(int(i), T, bs))
        out[:, j] = p[:, start:start + n].sum(axis=1)
        start += n
    return out


# ---------------------------------------------------------------------------
# ALiBi  [LAZY, generalisation: the deferred treatment of positions carries
# over to other relative schemes, ALiBi among them]
# ---------------------------------------------------------------------------

def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes.  READING (the pages name ALiBi, not its
    slopes): the usual geometric sequence, slope_j = 2^(-8 (j + 1) / H) for
    H a power of two."""
    return np.power(2.0, -8.0 * (np.arange(H, dtype=np.float64) + 1.0) / H)


def alibi_bias(slopes: np.ndarray, n: int, positions: np.ndarray) -> np.ndarray:
    """Additive attention bias of a query at position n over keys at the
    given positions: -slope * (n - position), one row per head.  Nothing is
    stored with the keys, so the bias is applied at attention time."""
    slopes = np.asarray(slopes, dtype=np.float64)
    d = float(n) - np.asarray(positions, dtype=np.float64)
    return -slopes[:, None] * d[None, :]


# ---------------------------------------------------------------------------
# Rotary position embedding  [LAZY, decoding + mathematical equivalence]
# ---------------------------------------------------------------------------

def rope_inv_freq(D: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i < D/2 (rotate-half convention; READING)."""
    return np.power(float(base), -(2.0 * np.arange(D // 2, dtype=np.float64)) / D)


def rope_rotate(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of x by position pos (scalar or broadcastable
    over the leading axes): pairs (i, i + D/2) turn by angle pos * theta_i."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------------------
# One decode step for one (b, h) pair
# ---------------------------------------------------------------------------

def materialise(q_group, K, T, bs, rope=None):
    """Queries and keys as attention sees them.  Without deferred RoPE they
    are the inputs (the first T keys).  With it (rope = dict(q_pos=n,
    block_start=(nb,) absolute start of the document holding each block,
    base=...)) every key is materialised as Rot(doc start) k_stored and the
    queries as Rot(n) q [LAZY, mathematical equivalence; READING: stored
    keys carry their in-document rotation].  Returns (q, K), float64."""
    if rope is None:
        return q_group, K[:T]
    nb = num_blocks(T, bs)
    Kt = np.empty((T, K.shape[1]))
    starts = np.asarray(rope["block_start"], dtype=np.float64)
    for i in range(nb):
        r = block_token_range(i, T, bs)
        Kt[r.start:r.stop] = rope_rotate(K[r.start:r.stop], starts[i], rope["base"])
    return rope_rotate(q_group, rope["q_pos"], rope["base"]), Kt


def attend_blocks(qt, Kt, V, T, bs, blocks, num_splits, scale, alibi=None, chunks=None):
    """Attention of the group's query rows over the tokens of the given
    blocks, split into contiguous chunks of the block list (or the given
    partition `chunks` of it: num_splits lists) and unsplit [NOVITA,
    attention modifications]: per-split (o, m, l) partials, the merged
    (O, m, l) over every listed token, and, without ALiBi, each block's
    softmax mass per query row.  qt, Kt as materialise() returns them;
    alibi: None or the group's (G,) slopes, biasing by the distance from the
    query at position T - 1."""
    def bias(toks):
        return None if alibi is None else alibi_bias(alibi, T - 1, toks)

    if chunks is None:
        chunks = split_chunks(list(blocks), num_splits)
    assert len(chunks) == num_splits and sorted(b for c in chunks for b in c) == sorted(blocks), \
        "chunks must partition the block list"
    parts = []
    for chunk in chunks:
        toks = tokens_of_blocks(chunk, T, bs)
        parts.append(attend(qt, Kt[toks], V[toks], scale, bias(toks)))
    out = {"part_o": np.stack([p[0] for p in parts], axis=1),   # (G, P, D)
           "part_m": np.stack([p[1] for p in parts], axis=1),   # (G, P)
           "part_l": np.stack([p[2] for p in parts], axis=1)}
    toks = tokens_of_blocks(blocks, T, bs)
    out["O"], out["m"], out["l"] = attend(qt, Kt[toks], V[toks], scale, bias(toks))
    if alibi is None:
        out["mass"] = softmax_block_mass(qt, Kt, list(blocks), T, bs, scale)
    return out


def decode_step_bh(q_group, K, V, e, T, bs, ss, k_e, k_q, evicted, prev_sel,
                   num_splits, scale, select_all=False, rope=None, alibi=None):
    """The whole step for one (sequence, KV head), from already-appended
    inputs, in the order the pages give: score, select, set differences,
    attention.

    q_group: (G, D) float64 query heads of this group.
    K, V:    (>=T, D) float64 keys/values in logical token order; for the
             deferred-RoPE case these are the *stored* keys.
    e:       (>=T,) float64 eviction logits.
    rope:    None, or dict(q_pos=n, block_start=(nb,) absolute start
             position of the document holding each block, base=...).  Keys
             are then materialised as Rot(doc start) k_stored and queries as
             Rot(n) q (READING: stored keys carry their in-document
             rotation), for the query-aware scores as for attention.
    select_all: skip scoring and take every block (deferred-RoPE workload).
    alibi:   None, or the group's (G,) slopes: attention adds
             alibi_bias(slopes, T - 1, token positions) (READING: the query
             sits at the newest token's position T - 1, and selection scores
             stay as without ALiBi).

    Returns a dict with block scores, the selection, swap lists, per-split
    partials, the merged (O, m, l) and each selected block's softmax mass
    per query head.
    """
    nb = num_blocks(T, bs)
    out: dict = {"nb": nb}
    qt, Kt = materialise(q_group, K, T, bs, rope)
    if select_all:
        gamma_e, gamma_q, gamma = [], list(range(nb)), list(range(nb))
        evicted_after = set(evicted)
    else:
        s_q = query_token_scores(qt, Kt)  # with RoPE: the rotated query and keys
        s_e = eviction_token_scores(e[:T])
        S_q = pool_block_scores(s_q, T, bs, ss)
        E = pool_block_scores(s_e, T, bs, ss)
        out["S_q"], out["E"] = S_q, E
        gamma_e, gamma_q, gamma, evicted_after = select_blocks(S_q, E, nb, k_e, k_q, evicted)
    load, drop = swap_lists(prev_sel, gamma)
    out.update(gamma_e=gamma_e, gamma_q=gamma_q, sel=gamma, evicted=evicted_after,
               load=load, evict=drop)

    out.update(attend_blocks(qt, Kt, V, T, bs, gamma, num_splits, scale, alibi))
    return out


# ---------------------------------------------------------------------------
# Prefill over reused documents  [LAZY, 1. Prefilling + mathematical
# equivalence]
# ---------------------------------------------------------------------------

def prefill_attention_bh(q, K, V, T, q_pos0, block_start, bs, base, scale):
    """Causal attention of a prompt over a context of reused documents, for
    one (sequence, KV head).

    q:  (M, G, D) float64 prompt queries (unrotated), query m at position
        n = q_pos0 + m.
    K, V: (>=T, D) float64 stored keys / values in logical order; the keys
        carry only their in-document rotation.
    block_start: (nb,) absolute start position of the document holding
        each block.

    Keys are materialised as Rot(doc start) k_stored, queries as Rot(n) q;
    query m attends the keys at positions t <= n (t < T), by the softmax
    definition.  READING: the prompt is itself the last document of the
    context (its keys present in the cache), positions are logical token
    indices.  Returns O (M, G, D), m (M, G), l (M, G).
    """
    q = np.asarray(q, dtype=np.float64)
    M, G, D = q.shape
    nb = num_blocks(T, bs)
    Kt = np.empty((T, D))
    for i in range(nb):
        r = block_token_range(i, T, bs)
        Kt[r.start:r.stop] = rope_rotate(K[r.start:r.stop], float(block_start[i]), base)
    O = np.zeros((M, G, D))
    m = np.full((M, G), -np.inf)
    l = np.zeros((M, G))
    for mi in range(M):
        n = q_pos0 + mi
        qt = rope_rotate(q[mi], n, base)
        hi = min(n + 1, T)
        O[mi], m[mi], l[mi] = attend(qt, Kt[:hi], V[:hi], scale)
    return O, m, l

