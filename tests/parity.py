"""Helpers for GPU-vs-oracle parity: run the float64 oracle for one
(b, h) pair of a workload step on the same generated inputs and compare it
with what the HIP library produced.

Acceptance (per pair and step):
* selection, eviction set (recovered from the bitmap) and swap lists are
  bit-exact, except where every mismatched pair of blocks is a near-tie:
  |S[a] - S[b]| <= 1e-6 * max(|S[a]|, |S[b]|) on the oracle's float64
  scores of the stage that chose them.  After such a near-tie the swap
  lists and the attention are compared with the oracle's over the GPU's
  own selection, so no pair-step goes without an attention check, and a
  run fails if near-ties exceed MAX_NEAR_TIE_FRAC of its compared
  pair-steps;
* O within 1e-2 max-abs, LSE = m + ln l within 1e-3, m within 1e-3, and the
  same for every non-empty split partial; empty splits are exactly
  (m, l, O) = (-inf, 0, 0);
* block scores within a bound derived from the arithmetic (one fp32
  rounding of each summary element and of the result);
* softmax block masses (when the session computes them) within 2e-3
  relative + 1e-6 absolute of the oracle's, and exactly 0 past the
  selection.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle
from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.workloads import TABLE_PACKED_ROPE, Workload

O_TOL = 1e-2
LSE_TOL = 1e-3
TIE_REL = 1e-6
# near-tie events allowed per run: this fraction of the compared pair-steps
# (at least one); fp32 scores agree with the float64 ones to ~2^-22
# relative, so a tie inside 1e-6 is rare on Gaussian inputs, and more than
# a few would point at a scoring error, not at ties
MAX_NEAR_TIE_FRAC = 0.01
# softmax block mass: p = exp(s - LSE), so an LSE error within LSE_TOL moves
# every probability by that relative amount, and a block's mass (a sum of
# them) by no more; twice that, plus an absolute floor for fp32 rounding
MASS_REL = 2e-3
MASS_ABS = 1e-6


@dataclass
class PairState:
    evicted: set = field(default_factory=set)
    prev: list = field(default_factory=list)


@dataclass
class Logical:
    """float64 logical view of one (b, h) pair's token stream."""
    K: np.ndarray
    V: np.ndarray
    e: np.ndarray


def logical_pair(inp: synth.Inputs, b: int, h: int) -> Logical:
    return Logical(oracle.bf16_to_f64(inp.K[b, h]), oracle.bf16_to_f64(inp.V[b, h]),
                   inp.e[b, h].astype(np.float64))


def oracle_step(w: Workload, inp: synth.Inputs, lg: Logical, b: int, h: int, t: int,
                st: PairState, P: int, alibi: bool = False) -> dict:
    T = w.seq_len(t)
    q = oracle.bf16_to_f64(inp.q(t)[b, h * w.G:(h + 1) * w.G])
    rope = None
    if w.table == TABLE_PACKED_ROPE:
        rope = dict(q_pos=int(inp.q_pos[b]), block_start=synth.block_doc_start(w) * w.bs, base=w.rope_base)
    slopes = None
    if alibi:  # the group's slopes, as the HIP path receives them (float32)
        slopes = synth.alibi_slopes(w.Hq)[h * w.G:(h + 1) * w.G].astype(np.float64)
    return oracle.decode_step_bh(q, lg.K, lg.V, lg.e, T, w.bs, w.ss, w.k_e, w.k_q, st.evicted, st.prev,
                                 P, 1.0 / math.sqrt(w.D), select_all=w.select_all, rope=rope, alibi=slopes)


def bitmap_set(words: np.ndarray, nb: int) -> set:
    bits = np.unpackbits(words.astype("<u4").view(np.uint8), bitorder="little")
    return {i for i in range(nb) if bits[i]}


def near_tie_ok(scores: np.ndarray, want: set, got: set) -> tuple[bool, str]:
    """All blocks the oracle chose and the GPU did not (and vice versa) are
    within the relative near-tie window of each other."""
    miss, extra = sorted(want - got), sorted(got - want)
    if len(miss) != len(extra):
        return False, f"size differs: missing {miss}, extra {extra}"
    for a in miss:
        for c in extra:
            sa, sc = float(scores[a]), float(scores[c])
            if abs(sa - sc) > TIE_REL * max(abs(sa), abs(sc)):
                return False, f"block {a} ({sa!r}) vs {c} ({sc!r}) is not a near-tie"
    return True, f"near-tie swap {miss} <-> {extra}"


def check_attention(r: dict, O: np.ndarray, m: np.ndarray, l: np.ndarray,
                    part_o: np.ndarray, part_m: np.ndarray, part_l: np.ndarray, where: str):
    """GPU (O, m, l) for the G heads of one pair against the oracle result."""
    Ow, mw, lw = r["O"], r["m"], r["l"]
    empty = ~np.isfinite(mw)
    assert np.all(np.isneginf(m[empty])) and np.all(l[empty] == 0) and np.all(O[empty] == 0), where
    ok = ~empty
    if ok.any():
        assert np.abs(O[ok] - Ow[ok]).max() <= O_TOL, (where, "O", np.abs(O[ok] - Ow[ok]).max())
        lse_g = m[ok] + np.log(l[ok])
        lse_w = mw[ok] + np.log(lw[ok])
        assert np.abs(lse_g - lse_w).max() <= LSE_TOL, (where, "LSE", np.abs(lse_g - lse_w).max())
        assert np.abs(m[ok] - mw[ok]).max() <= LSE_TOL, (where, "m")
    # partials, split by split
    po, pm, pl = r["part_o"], r["part_m"], r["part_l"]
    pe = ~np.isfinite(pm)
    assert np.all(np.isneginf(part_m[pe])) and np.all(part_l[pe] == 0) and np.all(part_o[pe] == 0), \
        (where, "empty split")
    pk = ~pe
    if pk.any():
        assert np.abs(part_o[pk] - po[pk]).max() <= O_TOL, (where, "part_o")
        assert np.abs(part_m[pk] + np.log(part_l[pk]) - pm[pk] - np.log(pl[pk])).max() <= LSE_TOL, \
            (where, "part LSE")


def score_bound(w: Workload, lg: Logical, q: np.ndarray, T: int) -> np.ndarray:
    """Per-block bound on |GPU score_q - oracle S_q|: the sub-block mean keys
    are rounded once to fp32 (relative 2^-24 each) and the block score once
    more; 2^-22 covers both with margin.  Computed per sub-block from
    |qbar| . |kbar| (with deferred RoPE, where the query is rotated, from
    ||qbar|| ||kbar||: the rotation keeps norms)."""
    qbar = np.abs(q.mean(axis=0))
    nb = -(-T // w.bs)
    n_sub = -(-T // w.ss)  # non-empty sub-blocks, in token order
    full = T // w.ss
    sums = np.zeros((n_sub, lg.K.shape[1]))
    sums[:full] = lg.K[:full * w.ss].reshape(full, w.ss, lg.K.shape[1]).mean(axis=1)
    if n_sub > full:
        sums[full] = lg.K[full * w.ss:T].mean(axis=0)
    kbar = np.abs(sums)
    if w.table == TABLE_PACKED_ROPE:
        x = np.linalg.norm(qbar) * np.linalg.norm(kbar, axis=1)
    else:
        x = kbar @ qbar
    x = x / math.sqrt(w.D)
    blk = np.arange(n_sub) * w.ss // w.bs
    out = np.zeros(nb)
    np.maximum.at(out, blk, x)
    return out * 2.0 ** -22


class Gpu:
    """Host copies of one session's step outputs."""

    def __init__(self, sess):
        s = sess
        self.seq_lens = s.seq_lens.cpu().numpy()
        self.sel = s.sel.cpu().numpy()
        self.sel_count = s.sel_count.cpu().numpy()
        self.evicted = s.evicted.cpu().numpy().view(np.uint32)
        self.load = s.load.cpu().numpy()
        self.load_count = s.load_count.cpu().numpy()
        self.evict = s.evict.cpu().numpy()
        self.evict_count = s.evict_count.cpu().numpy()
        self.score_q = s.score_q.cpu().numpy()
        self.score_e = s.score_e.cpu().numpy()
        self.o = s.o.cpu().numpy()
        self.m = s.m.cpu().numpy()
        self.l = s.l.cpu().numpy()
        self.part_o = s.part_o.cpu().numpy()
        self.part_m = s.part_m.cpu().numpy()
        self.part_l = s.part_l.cpu().numpy()
        self.err = int(s.err.cpu().numpy()[0])
        self.mass = s.mass.cpu().numpy() if getattr(s, "mass_on", False) else None


def oracle_over(w: Workload, inp, lg: Logical, b: int, h: int, t: int, prev: list, blocks: list, P: int,
                alibi: bool = False, chunks: list | None = None) -> dict:
    """The oracle's swap lists and attention for a given selection (the
    GPU's, after a near-tie) and split layout (chunks: None for contiguous
    chunks): the same stages as oracle_step after the selection, over
    `blocks`."""
    T = w.seq_len(t)
    q = oracle.bf16_to_f64(inp.q(t)[b, h * w.G:(h + 1) * w.G])
    rope = None
    if w.table == TABLE_PACKED_ROPE:
        rope = dict(q_pos=int(inp.q_pos[b]), block_start=synth.block_doc_start(w) * w.bs, base=w.rope_base)
    slopes = synth.alibi_slopes(w.Hq)[h * w.G:(h + 1) * w.G].astype(np.float64) if alibi else None
    qt, Kt = oracle.materialise(q, lg.K, T, w.bs, rope)
    r = oracle.attend_blocks(qt, Kt, lg.V, T, w.bs, list(blocks), P, 1.0 / math.sqrt(w.D), slopes, chunks)
    r["load"], r["evict"] = oracle.swap_lists(prev, blocks)
    return r


def compare_pair(w: Workload, inp, lg: Logical, g: Gpu, b: int, h: int, t: int, st: PairState,
                 P: int, log: list, check_scores: bool = True, alibi: bool = False, shares: bool = False) -> dict:
    """Compare one pair at step t; returns the oracle result.  Selection
    mismatches must be near-ties (logged); the swap lists and attention are
    then compared with the oracle's over the GPU's selection (the two sides
    attend over different blocks, each correctly).  shares: the step ran
    the fused select + decode, whose splits take equal shares of the
    eviction and query parts (oracle.share_chunks) on steps where the
    eviction part keeps every block it has not dropped."""
    r = oracle_step(w, inp, lg, b, h, t, st, P, alibi)
    where = f"{w.name} t={t} b={b} h={h}"
    nb = r["nb"]
    G = w.G
    n = int(g.sel_count[b, h])
    sel = g.sel[b, h, :n].tolist()
    same_sel = sel == r["sel"]
    if not w.select_all:
        if check_scores:
            q = oracle.bf16_to_f64(inp.q(t)[b, h * G:(h + 1) * G])
            bound = score_bound(w, lg, q, w.seq_len(t))
            dq = np.abs(g.score_q[b, h, :nb].astype(np.float64) - r["S_q"])
            assert np.all(dq <= bound), (where, "score_q", float(dq.max()), float(bound.min()))
            de = np.abs(g.score_e[b, h, :nb].astype(np.float64) - r["E"])
            assert np.all(de <= 2.0 ** -23 * np.abs(r["E"])), (where, "score_e", float(de.max()))
        ge_gpu = set(range(nb)) - bitmap_set(g.evicted[b, h], nb)
        gq_gpu = set(sel) - ge_gpu
        ok_e = ge_gpu == set(r["gamma_e"])
        ok_q = gq_gpu == set(r["gamma_q"])
        if not ok_e:
            good, msg = near_tie_ok(r["E"], set(r["gamma_e"]), ge_gpu)
            assert good, (where, "eviction set", msg)
            log.append(f"{where}: eviction {msg}")
        if ok_e and not ok_q:
            good, msg = near_tie_ok(r["S_q"], set(r["gamma_q"]), gq_gpu)
            assert good, (where, "query set", msg)
            log.append(f"{where}: query {msg}")
        assert sel == sorted(sel) and len(sel) == len(set(sel)), (where, "sel not ascending/unique")
        if ok_e and ok_q:
            assert same_sel, (where, "union", sel, r["sel"])
    else:
        assert same_sel, (where, "select_all", sel[:5], r["sel"][:5])
    chunks = None
    if shares and P > 1 and not w.select_all:
        cand = [i for i in range(nb) if i not in st.evicted]
        if len(cand) <= w.k_e:  # the fast path: every candidate stays, in ascending order
            chunks = oracle.share_chunks(cand, sorted(set(sel) - set(cand)), P)
    ra = r if same_sel and chunks is None else oracle_over(w, inp, lg, b, h, t, st.prev, sel, P, alibi, chunks)
    nl, ne = int(g.load_count[b, h]), int(g.evict_count[b, h])
    assert g.load[b, h, :nl].tolist() == ra["load"], (where, "load")
    assert g.evict[b, h, :ne].tolist() == ra["evict"], (where, "evict")
    hs = slice(h * G, (h + 1) * G)
    check_attention(ra, g.o[b, hs], g.m[b, hs], g.l[b, hs], g.part_o[b, hs], g.part_m[b, hs],
                    g.part_l[b, hs], where)
    if g.mass is not None:
        got = g.mass[b, hs, :len(sel)]
        want = ra["mass"]
        err = np.abs(got - want)
        assert np.all(err <= MASS_REL * want + MASS_ABS), (where, "mass", float(err.max()))
        assert np.all(g.mass[b, hs, len(sel):] == 0), (where, "mass past the selection")
    return r
