"""HIP path vs the float64 oracle, through the C-ABI, on the five workloads.

Small variants compare every (b, h) pair at every step; the full-size runs
(in the launch configuration the benchmark uses) compare sampled pairs and
check the invariants on every pair.  Each case prints its name before it
touches the GPU.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.workloads import WORKLOADS

import parity
from parity import (Gpu, PairState, bitmap_set, check_attention, compare_pair, logical_pair)

pytestmark = pytest.mark.gpu


def announce(msg: str):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def session(w, inp, **kw):
    from block_sparse_kv_score_amd.step import DecodeSession
    return DecodeSession(w, inp, **kw)


def force_pair(sess, b: int, h: int, r: dict):
    """After a logged near-tie, hand the oracle's state for this pair to the
    GPU (an input to the HIP path) so later steps stay comparable."""
    w = sess.w
    words = sess.evicted.shape[-1]
    bits = np.zeros(words * 32, dtype=np.uint8)
    for i in r["evicted"]:
        bits[i] = 1
    packed = np.packbits(bits, bitorder="little").view(np.uint32).view(np.int32)
    sess.evicted[b, h] = torch.from_numpy(packed.copy()).to(sess.dev)
    sel = np.full(sess.cap, -1, dtype=np.int32)
    sel[:len(r["sel"])] = r["sel"]
    sess.sel[b, h] = torch.from_numpy(sel).to(sess.dev)
    sess.sel_count[b, h] = len(r["sel"])
    torch.cuda.synchronize()


def gpu_invariants(w, t, g: Gpu, prev: Gpu | None):
    """Checks on the GPU trajectory itself, every pair."""
    T = w.seq_len(t)
    nb = -(-T // w.bs)
    want = min(w.k, nb)
    assert np.all(g.sel_count == want), ("selection size", np.unique(g.sel_count), want)
    assert np.all(g.seq_lens == T)
    if prev is None:
        return
    nb_prev = -(-(T - 1) // w.bs) if w.append else nb
    for b in range(w.B):
        for h in range(w.Hkv):
            ev_now, ev_before = bitmap_set(g.evicted[b, h], nb), bitmap_set(prev.evicted[b, h], nb)
            assert ev_before <= ev_now, "evicted set shrank"
            ge = set(range(nb)) - ev_now
            ge_prev = set(range(nb_prev)) - ev_before
            new = set(range(nb_prev, nb))
            assert ge <= ge_prev | new, "an evicted block returned to the eviction set"
            cur = set(g.sel[b, h, :g.sel_count[b, h]].tolist())
            old = set(prev.sel[b, h, :prev.sel_count[b, h]].tolist())
            gamma = len(cur & old) / len(cur)
            assert gamma >= (w.k_e - len(new & ge)) / w.k - 1e-12, ("locality", gamma)


def force_slots(sess, b: int, h: int, owner: list, last_use: list | None = None):
    """Host tier: after a forced selection, give the pair the oracle's slot
    state (owners, timestamps, resident table and the pages in the slots)."""
    w, inp = sess.w, sess.inp
    bh = b * w.Hkv + h
    res = torch.full((w.max_blocks,), -1, dtype=torch.int32)
    for s, x in enumerate(owner):
        if x >= 0:
            dp, hp = bh * sess.slots + s, host_page(w, inp, b, h, x)
            res[x] = dp
            sess.k_pages[dp] = sess.host_k[hp].to(sess.dev)
            sess.v_pages[dp] = sess.host_v[hp].to(sess.dev)
            sess.e_pages[dp] = sess.host_e[hp].to(sess.dev)
    sess.resident[b, h] = res.to(sess.dev)
    sess.slot_owner[b, h] = torch.tensor(owner, dtype=torch.int32, device=sess.dev)
    if last_use is not None:
        sess.last_use[b, h] = torch.tensor(last_use, dtype=torch.int32, device=sess.dev)
    torch.cuda.synchronize()


def run_trajectory(w, seed=0, pairs=None, steps=None, splits=None, check_scores=True, fused=True, inp=None,
                   offload=False, buffer_slots=None, bucket_width=1, mass=False, alibi=False, qkv=False,
                   all_pairs_at=(), sess_kw=None):
    """Steps 1..steps of workload w on the GPU, each compared with the
    oracle for `pairs` (all by default) and, at the steps in all_pairs_at,
    for every pair.  A pair compared at step t without having been compared
    at t - 1 starts from the GPU's own state after t - 1 (eviction bitmap
    and previous selection): the teacher-forced check of every step."""
    n_steps = steps or w.steps
    announce(f"trajectory {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T0={w.T0} k={w.k_e}/{w.k_q} "
             f"steps={n_steps} P={splits or w.splits} pairs={'all' if pairs is None else pairs} "
             f"all pairs at {tuple(all_pairs_at)} seed={seed} fused={fused} offload={offload} "
             f"buffer={buffer_slots}/{bucket_width} mass={mass} alibi={alibi} qkv={qkv} {sess_kw or ''}")
    inp = inp if inp is not None else synth.generate(w, seed)
    sess = session(w, inp, splits=splits, fused=fused, offload=offload, buffer_slots=buffer_slots,
                   bucket_width=bucket_width, mass=mass, alibi=alibi, qkv=qkv, **(sess_kw or {}))
    every = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    pairs = pairs or every
    if offload:
        assert not all_pairs_at, "the host tier tracks the oracle's slots for the sampled pairs only"
    w_e = synth.eviction_head_weights(w, inp.seed) if qkv else None

    def make_lg(b, h):
        lg = logical_pair(inp, b, h)
        if qkv:  # appended tokens' logits come from the eviction head (the oracle's)
            lg.e = lg.e.copy()
            lg.e[w.T0:] = oracle.eviction_head(lg.V[w.T0:], w_e[h]).astype(np.float64)
        return lg

    lgs = {p: make_lg(*p) for p in pairs}
    states = {p: PairState() for p in pairs}
    owners = {p: [-1] * sess.slots for p in pairs} if offload else None
    stamps = {p: [0] * sess.slots for p in pairs} if offload else None
    total_misses = 0
    log: list[str] = []
    compared = 0
    prev_g = None
    for t in range(1, n_steps + 1):
        sess.step(t)
        torch.cuda.synchronize()
        g = Gpu(sess)
        assert g.err == 0, "device contract flag raised"
        assert not sess.counters.any().item(), "fused combine left a nonzero arrival counter"
        if not w.select_all:
            gpu_invariants(w, t, g, prev_g)
        forced = False
        slot_owner = sess.slot_owner.cpu().numpy() if offload else None
        if offload and sess.buffered:
            last_use = sess.last_use.cpu().numpy()
            miss_count = sess.miss_count.cpu().numpy()
        step_pairs = every if t in all_pairs_at else pairs
        nb_prev = -(-w.seq_len(t - 1) // w.bs) if t > 1 else 0
        for (b, h) in step_pairs:
            lg = lgs.get((b, h)) or make_lg(b, h)
            st = states.get((b, h))
            if st is None:  # not compared at t - 1: the GPU's state after it
                st = PairState() if prev_g is None else PairState(
                    bitmap_set(prev_g.evicted[b, h], nb_prev), prev_g.sel[b, h, :prev_g.sel_count[b, h]].tolist())
            r = compare_pair(w, inp, lg, g, b, h, t, st, sess.P, log, check_scores, alibi,
                             shares=sess.runs_select_decode)
            compared += 1
            n = int(g.sel_count[b, h])
            same = g.sel[b, h, :n].tolist() == r["sel"]
            if offload and sess.buffered:
                # the oracle's selection through the oracle's buffer
                want, lu, misses, _, placed = oracle.buffer_retrieve(owners[(b, h)], stamps[(b, h)], r["sel"],
                                                                     sess.buffer_clock, bucket_width)
                assert placed == len(misses), (t, b, h, "slots overflow")
                if same:
                    assert slot_owner[b, h].tolist() == want, (w.name, t, b, h, "slot owners")
                    live = [s for s in range(sess.slots) if want[s] >= 0]
                    assert [int(last_use[b, h, s]) for s in live] == [lu[s] for s in live], (t, b, h, "stamps")
                    assert int(miss_count[b, h]) == len(misses), (t, b, h, "misses")
                owners[(b, h)], stamps[(b, h)] = want, lu
                total_misses += len(misses)
            elif offload:
                # the oracle's swap lists placed into the oracle's slot state
                want, placed = oracle.place_blocks(owners[(b, h)], r["evict"], r["load"])
                assert placed == len(r["load"]), (t, b, h, "slots overflow")
                if same:
                    assert slot_owner[b, h].tolist() == want, (w.name, t, b, h, "slot owners")
                owners[(b, h)] = want
            if not same or bitmap_set(g.evicted[b, h], r["nb"]) != r["evicted"]:
                force_pair(sess, b, h, r)
                if offload:
                    force_slots(sess, b, h, owners[(b, h)], stamps[(b, h)] if sess.buffered else None)
                forced = True
            if (b, h) in states:
                states[(b, h)] = PairState(set(r["evicted"]), list(r["sel"]))
        prev_g = Gpu(sess) if forced else g
    for line in log:
        print("near-tie:", line)
    assert len(log) <= max(1, int(parity.MAX_NEAR_TIE_FRAC * compared)), \
        (f"{len(log)} near-ties in {compared} compared pair-steps", log[:5])
    if offload and sess.buffered:
        print(f"buffer misses over the trajectory: {total_misses}")
    return log


# ---------------------------------------------------------------------------
# small variants: every pair, every step
# ---------------------------------------------------------------------------

def test_tiny_nosa_16_steps():
    run_trajectory(WORKLOADS["tiny_nosa"])


def test_8b_shape_small_ragged():
    # T0 not a multiple of the block size: block creation at step 4,
    # partial sub-blocks, 3 splits over 64 selected blocks
    w = WORKLOADS["llama3_8b_32k"].scaled(B=2, Hq=8, Hkv=2, T0=4096 + 61)
    run_trajectory(w, seed=1, splits=3)


def test_70b_shape_small_two_level():
    w = WORKLOADS["llama31_70b_256k"].scaled(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64)
    run_trajectory(w, seed=2)


def test_tiny_nosa_separate_calls():
    # the unfused sequence: nosa_select, nosa_swap_diff, nosa_sparse_decode,
    # nosa_combine as six launches
    run_trajectory(WORKLOADS["tiny_nosa"], seed=10, steps=8, fused=False)


def test_8b_shape_small_separate_calls():
    w = WORKLOADS["llama3_8b_32k"].scaled(B=2, Hq=8, Hkv=2, T0=4096 + 61)
    run_trajectory(w, seed=1, splits=3, steps=6, fused=False)


FUSED_CASES = [
    ("tiny_nosa", {}, 2),
    ("tiny_nosa", {}, 1),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 3),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1),
    ("dense_8b_8k", dict(B=2, Hq=8, Hkv=2, T0=1000), 37),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 16),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 1),
    ("tiny_nosa", dict(B=1, Hq=4, Hkv=1, bs=128, ss=2, T0=1500, k_e=2, k_q=3), 1),
    ("tiny_nosa", dict(B=2, Hq=8, Hkv=2, bs=256, ss=32, T0=3000, k_e=5, k_q=3), 1),
    ("lazy_rope_32k", dict(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512), 9),
    ("lazy_rope_sparse_32k", dict(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512), 2),
    ("lazy_rope_sparse_32k", dict(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512), 1),
    ("tiny_nosa", dict(B=1, Hq=4, Hkv=1, T0=64 * 1100 + 5, k_e=40, k_q=24), 2),  # past 1024 blocks
]


@pytest.mark.parametrize("name,scale,splits", FUSED_CASES,
                         ids=[f"{c[0]}-bs{c[1].get('bs', 'def')}-P{c[2]}" for c in FUSED_CASES])
def test_fused_equals_separate(name, scale, splits):
    """The fused launches against the separate calls they fuse, step after
    step: selections, swap lists, lengths, summaries, block scores, pages
    and the row max bit for bit.  nosa_select_decode visits the selected
    tiles in another order (wave 0 makes the query part while the others
    decode the eviction part), so o and l are held to the parity bar; with
    several splits, on steps where the eviction part keeps every block it
    has not dropped, each split covers its share of the eviction and query
    parts instead of a contiguous chunk, so the partials are not compared
    here (the trajectory tests hold them to the oracle's share layout)."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    announce(f"fused vs separate {name} {scale} P={splits}")
    inp = synth.generate(w, 11)
    a = session(w, inp, splits=splits, fused=True, select_decode=True)
    s = session(w, inp, splits=splits, fused=False)
    names = ["sel", "sel_count", "evicted", "load", "load_count", "evict", "evict_count",
             "part_o", "part_m", "part_l", "o", "m", "l", "seq_lens", "k_summary", "e_summary",
             "score_q", "score_e", "k_pages", "v_pages", "e_pages"]
    for t in range(1, min(w.steps, 6) + 1):
        a.step(t)
        s.step(t)
        torch.cuda.synchronize()
        for n in names:
            x, y = getattr(a, n), getattr(s, n)
            if n in ("load", "evict"):  # compare the listed prefix only
                cnt = getattr(a, n + "_count")
                assert torch.equal(cnt, getattr(s, n + "_count"))
                for b in range(w.B):
                    for h in range(w.Hkv):
                        k = int(cnt[b, h])
                        assert torch.equal(x[b, h, :k], y[b, h, :k]), (n, t, b, h)
                continue
            if n == "sel":
                cnt = a.sel_count
                for b in range(w.B):
                    for h in range(w.Hkv):
                        k = int(cnt[b, h])
                        assert torch.equal(x[b, h, :k], y[b, h, :k]), (n, t, b, h)
                continue
            if splits > 1 and n in ("part_o", "part_m", "part_l"):
                continue
            if n in ("part_o", "o"):
                assert (x - y).abs().max().item() <= parity.O_TOL, (n, t)
                continue
            if n in ("part_l", "l"):
                lx, ly = torch.log(x.double()), torch.log(y.double())
                assert torch.equal(x > 0, y > 0), (n, t)
                assert not (x > 0).any() or (lx - ly)[x > 0].abs().max().item() <= parity.LSE_TOL, (n, t)
                continue
            assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                               y.view(torch.int32) if y.dtype == torch.float32 else y), (n, t)
        assert not a.counters.any().item()


@pytest.mark.parametrize("splits,fused", [(16, True), (18, True), (16, False)])
def test_dense_two_splits_per_workgroup(splits, fused):
    # short splits on enough pairs that a workgroup takes two adjacent
    # splits (two waves on each); at 18 splits over 32 blocks the last two
    # are empty, and the context ends in a partial block.  Unfused: the
    # split-only decode and the separate combine.
    w = WORKLOADS["dense_8b_8k"].scaled(B=8, Hq=16, Hkv=4, T0=2000)
    run_trajectory(w, seed=5, splits=splits, fused=fused)


def test_lazy_rope_two_splits_per_workgroup():
    # the deferred-RoPE decode with two splits per workgroup: each wave
    # rotates the query for its own split's documents
    w = WORKLOADS["lazy_rope_32k"].scaled(B=8, Hq=16, Hkv=4, T0=8 * 256, doc_len=256)
    run_trajectory(w, seed=6, splits=16)


def test_dense_small_many_splits():
    # k = every block, more splits than blocks per split: empty splits
    w = WORKLOADS["dense_8b_8k"].scaled(B=2, Hq=8, Hkv=2, T0=1000)
    run_trajectory(w, seed=3, splits=37)


def test_lazy_rope_small():
    w = WORKLOADS["lazy_rope_32k"].scaled(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512)
    run_trajectory(w, seed=4)


def test_lazy_rope_sparse_small():
    """NOSA selection over a deferred-RoPE cache: query-aware scores with the
    per-document rotated query, then the rotated decode over the selection."""
    w = WORKLOADS["lazy_rope_sparse_32k"].scaled(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512)
    run_trajectory(w, seed=39)


def test_lazy_rope_sparse_g8_split():
    w = WORKLOADS["lazy_rope_sparse_32k"].scaled(B=1, Hq=16, Hkv=2, T0=4 * 1024, doc_len=1024, n_docs=4,
                                                   k_e=8, k_q=24, splits=3)
    run_trajectory(w, seed=40)


@pytest.mark.parametrize("doc_len", [64, 128])
def test_lazy_rope_sparse_short_docs(doc_len):
    # documents of one or two blocks: a scoring workgroup's 16 blocks span 16
    # or 8 documents, so its waves turn the mean query for several each
    n_docs = 2048 // doc_len
    w = WORKLOADS["lazy_rope_sparse_32k"].scaled(B=2, Hq=8, Hkv=2, T0=2048, doc_len=doc_len, n_docs=n_docs,
                                                   k_e=4, k_q=8)
    run_trajectory(w, seed=41)


def test_lazy_rope_g8_and_g1():
    for hq in (16, 2):
        w = WORKLOADS["lazy_rope_32k"].scaled(B=1, Hq=hq, Hkv=2, T0=4 * 256, doc_len=256, n_docs=4)
        run_trajectory(w, seed=5)


def test_group_sizes_and_head_dim_64():
    base = WORKLOADS["tiny_nosa"]
    for hq, hkv, d in [(2, 2, 64), (4, 2, 64), (16, 2, 64), (8, 1, 128), (16, 1, 128), (1, 1, 128)]:
        w = base.scaled(B=2, Hq=hq, Hkv=hkv, D=d, T0=700, k_e=3, k_q=5)
        run_trajectory(w, seed=6, steps=3, splits=2)


@pytest.mark.parametrize("splits", [2, 1])
def test_block_128_sub_1_and_256(splits):
    # at one split the fused select + decode loads each wave's first tile
    # during the selection: with 2 and 4 tiles per block the other waves
    # skip the block's first tile and keep its later ones
    base = WORKLOADS["tiny_nosa"]
    run_trajectory(base.scaled(B=1, Hq=4, Hkv=1, bs=128, ss=2, T0=1500, k_e=2, k_q=3), seed=7, steps=3,
                   splits=splits)
    run_trajectory(base.scaled(B=1, Hq=4, Hkv=1, bs=256, ss=64, T0=1500, k_e=1, k_q=2), seed=8, steps=3,
                   splits=splits)
    run_trajectory(base.scaled(B=2, Hq=8, Hkv=2, bs=256, ss=32, T0=3000, k_e=5, k_q=3, steps=6), seed=12,
                   splits=splits)


def test_70b_shape_small_two_level_one_split():
    # 128-token blocks (2 tiles each), G = 8, two-level table, one split:
    # the speculative first tile of the fused select + decode
    w = WORKLOADS["llama31_70b_256k"].scaled(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64)
    assert w.max_blocks <= 1024
    run_trajectory(w, seed=13, splits=1)


def test_fewer_blocks_than_budget():
    # nb < k_e: every block kept, no eviction
    w = WORKLOADS["tiny_nosa"].scaled(B=1, T0=100, k_e=4, k_q=4)
    run_trajectory(w, seed=9, steps=4)


# ---------------------------------------------------------------------------
# edge cases: exact ties, empty context, zero budgets, maximum capacity,
# out-of-range appends
# ---------------------------------------------------------------------------

def tie_inputs(w, seed, n_distinct):
    """Every whole block's tokens share one of n_distinct key vectors and
    logits (by block index), so those blocks' scores tie exactly in float32
    and in float64.  Blocks from the first partial one on (T0 // bs: the
    tail while tokens are appended) get their own vector and logit: the
    oracle averages per-token float64 scores, which rounds differently for a
    partial sub-block than for a whole one, so a tail block would only
    near-tie."""
    inp = synth.generate(w, seed)
    rng = np.random.default_rng(1000 + n_distinct)
    n_blk = -(-inp.K.shape[2] // w.bs)
    first_tail = w.T0 // w.bs
    keys = synth.f32_to_bf16_bits(rng.standard_normal((n_distinct + n_blk, w.D)).astype(np.float32))
    logits = rng.standard_normal(n_distinct + n_blk).astype(np.float32)
    blk = np.arange(inp.K.shape[2]) // w.bs
    vec = np.where(blk < first_tail, blk % n_distinct, n_distinct + blk)
    inp.K[...] = keys[vec][None, None]
    inp.e[...] = logits[vec][None, None]
    return inp


@pytest.mark.parametrize("n_distinct", [1, 3])
def test_exact_ties_lowest_index_wins(n_distinct):
    # ties must resolve exactly as the oracle's (score desc, index asc): no
    # near-tie allowance is used
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=8, Hkv=2, T0=1500, k_e=3, k_q=5)
    log = run_trajectory(w, seed=20, steps=6, inp=tie_inputs(w, 20, n_distinct))
    assert not log, log
    w = WORKLOADS["llama3_8b_32k"].scaled(B=1, Hq=8, Hkv=2, T0=4096 + 7)
    log = run_trajectory(w, seed=21, steps=3, inp=tie_inputs(w, 21, n_distinct))
    assert not log, log
    # the sixteen-wave selection (above 2048 blocks of capacity)
    w = WORKLOADS["tiny_nosa"].scaled(B=1, Hq=4, Hkv=2, T0=2600 * 64 - 256 - 5, k_e=20, k_q=12)
    assert w.max_blocks > 2048
    log = run_trajectory(w, seed=27, steps=2, inp=tie_inputs(w, 27, n_distinct))
    assert not log, log


def test_empty_context():
    # no prefill: the first step appends token 0 and attends to it alone
    run_trajectory(WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=0), seed=22, steps=8)


@pytest.mark.parametrize("k_e,k_q", [(0, 6), (6, 0)])
def test_zero_budgets(k_e, k_q):
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=8, Hkv=2, T0=1500, k_e=k_e, k_q=k_q)
    run_trajectory(w, seed=23, steps=5)


def test_maximum_capacity():
    # 8192 blocks of capacity (the widest selection form; the fused select +
    # decode falls back to the two calls above 1024 blocks)
    w = WORKLOADS["tiny_nosa"].scaled(B=1, Hq=4, Hkv=1, T0=8192 * 64 - 256 - 10, k_e=6, k_q=10)
    assert w.max_blocks == 8192
    run_trajectory(w, seed=24, steps=3, splits=3)


@pytest.mark.parametrize("blocks", [2049, 3500])
def test_wide_selection_workgroups(blocks):
    # above 2048 blocks of capacity the selection runs on sixteen waves
    # (3 and 4 keys per thread here); ties in the eviction logits are likely
    # at this many blocks, so the budgets are uneven
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=blocks * 64 - 256 - 30, k_e=40, k_q=9)
    assert w.max_blocks == blocks
    run_trajectory(w, seed=26, steps=3, splits=2)


SELECT_DECODE_EDGES = [
    # (name, scaling, steps) for the fused select + decode, which takes its
    # fast path (eviction part fixed, one wave selects while the others
    # decode) on every step where no new block competes
    ("zero-k_e", dict(B=2, Hq=8, Hkv=2, T0=1500, k_e=0, k_q=6), 5),
    ("zero-k_q", dict(B=2, Hq=8, Hkv=2, T0=1500, k_e=6, k_q=0), 5),
    ("empty-context", dict(B=2, Hq=4, Hkv=2, T0=0), 8),
    ("fewer-blocks-than-k_e", dict(B=1, T0=100, k_e=4, k_q=4), 4),
    ("block-creation", dict(B=2, Hq=8, Hkv=2, T0=64 * 20 - 3, k_e=5, k_q=3), 8),
    ("G16-D64", dict(B=2, Hq=32, Hkv=2, T0=900, k_e=3, k_q=5), 4),
]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("name,scale,steps", SELECT_DECODE_EDGES, ids=[c[0] for c in SELECT_DECODE_EDGES])
def test_select_decode_edges(name, scale, steps, splits):
    # with three splits each split takes its share of both parts (or, on a
    # block-creation step, a contiguous chunk), checked against the oracle's
    # layout of the same kind
    w = WORKLOADS["tiny_nosa"].scaled(**scale)
    run_trajectory(w, seed=28, steps=steps, splits=splits, sess_kw=dict(select_decode=True))


@pytest.mark.parametrize("n_blocks", [1100, 2200])
def test_select_decode_past_1024_blocks(n_blocks):
    # the nine-element-per-thread selection: more than 1024 blocks (past
    # 2048, bitmap words 64 and up), shares over three splits, block creation
    # at step 4
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=8, Hkv=2, T0=64 * n_blocks - 3, k_e=40, k_q=24)
    assert 1024 < w.max_blocks <= 2304
    run_trajectory(w, seed=44, steps=6, splits=3, sess_kw=dict(select_decode=True))


@pytest.mark.parametrize("n_distinct", [1, 3])
def test_exact_ties_one_split(n_distinct):
    # exact ties in the one-wave query selection: lowest index first
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=8, Hkv=2, T0=1500, k_e=3, k_q=5)
    log = run_trajectory(w, seed=29, steps=6, splits=1, inp=tie_inputs(w, 29, n_distinct))
    assert not log, log


def test_append_past_capacity_flags_and_keeps_length():
    from block_sparse_kv_score_amd import nosa
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=100)
    announce("append past capacity: error flag, lengths unchanged")
    inp = synth.generate(w, 25)
    sess = session(w, inp)
    cap = w.max_blocks * w.bs
    full = torch.full((w.B,), cap, dtype=torch.int32, device="cuda")
    nosa.nosa_append(sess.dims, sess.kv, sess.k_new[0], sess.v_new[0], sess.e_new[0], full, sess.k_summary,
                     sess.e_summary)
    torch.cuda.synchronize()
    assert int(sess.err.item()) == 1 and full.tolist() == [cap] * w.B
    sess.err.zero_()
    out = torch.zeros_like(full)
    nosa.nosa_append_score(sess.dims, sess.kv, sess.k_new[0], sess.v_new[0], sess.e_new[0], full, out,
                           sess.k_summary, sess.e_summary, sess.q(1), sess.score_q, sess.score_e)
    torch.cuda.synchronize()
    assert int(sess.err.item()) == 1 and out.tolist() == [cap] * w.B


# ---------------------------------------------------------------------------
# host tier: pages in pinned host memory, resident slots in HBM
# ---------------------------------------------------------------------------

def host_page(w, inp, b, h, i):
    """Page of logical block i of pair (b, h) in the session's page pools."""
    if inp.directory is None:
        return int(inp.pages[b, h, i])
    key = ((b * w.Hkv + h) << w.blocks_log2) | i
    seg = int(inp.directory[key >> w.seg_log2])
    return int(inp.segments.reshape(-1)[(seg << w.seg_log2) | (key & ((1 << w.seg_log2) - 1))])


OFFLOAD_CASES = [
    ("tiny_nosa", {}, 2),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 3),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 4),
]


@pytest.mark.parametrize("name,scale,splits", OFFLOAD_CASES, ids=[c[0] for c in OFFLOAD_CASES])
def test_offload_equals_resident(name, scale, splits):
    """The host-tier step gives the same bits as the all-in-HBM step, the
    resident set is exactly the selection, and every resident slot holds
    its block's pages."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    announce(f"host tier vs resident {name} {scale} P={splits}")
    inp = synth.generate(w, 30)
    a = session(w, inp, splits=splits, offload=True)
    s = session(w, inp, splits=splits, select_decode=False)  # the host tier's call sequence
    for t in range(1, min(w.steps, 6) + 1):
        a.step(t)
        s.step(t)
        torch.cuda.synchronize()
        assert int(a.err.item()) == 0 and int(s.err.item()) == 0
        for n in ["sel_count", "evicted", "load_count", "evict_count", "part_o", "part_m", "part_l", "o", "m", "l",
                  "seq_lens", "k_summary", "e_summary", "score_q", "score_e"]:
            x, y = getattr(a, n), getattr(s, n)
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), (n, t)
        res = a.resident.cpu().numpy()
        own = a.slot_owner.cpu().numpy()
        sel = a.sel.cpu().numpy()
        cnt = a.sel_count.cpu().numpy()
        dk, dv = a.k_pages.cpu(), a.v_pages.cpu()
        sk, sv = s.k_pages.cpu(), s.v_pages.cpu()
        assert torch.equal(a.host_k, sk) and torch.equal(a.host_v, sv)  # the host pools took every append
        for b in range(w.B):
            for h in range(w.Hkv):
                bh = b * w.Hkv + h
                chosen = sel[b, h, :cnt[b, h]].tolist()
                assert set(np.nonzero(res[b, h] >= 0)[0].tolist()) == set(chosen), (t, b, h)
                for x in chosen:
                    dp = int(res[b, h, x])
                    assert bh * a.slots <= dp < (bh + 1) * a.slots and own[b, h, dp - bh * a.slots] == x
                    hp = host_page(w, inp, b, h, x)
                    assert torch.equal(dk[dp], sk[hp]) and torch.equal(dv[dp], sv[hp]), (t, b, h, x)
                assert int((own[b, h] >= 0).sum()) == len(chosen)


@pytest.mark.parametrize("name,scale,splits", OFFLOAD_CASES, ids=[c[0] for c in OFFLOAD_CASES])
def test_offload_trajectory_vs_oracle(name, scale, splits):
    """Host tier against the oracle: selections, swap lists and attention
    as in the resident trajectories, plus the slot of every resident block
    (the oracle's placement of its own swap lists), bit-exact."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    run_trajectory(w, seed=32, splits=splits, steps=min(w.steps, 6), offload=True)


BUFFER_CASES = [
    # (workload, scaling, splits, buffer slots, bucket width): few spare
    # slots and fresh query picks, so the LRU evicts most steps
    ("tiny_nosa", dict(steps=24, T0=2048 + 50, k_e=2, k_q=6), 2, 11, 1),
    ("tiny_nosa", dict(steps=24, T0=2048 + 50, k_e=2, k_q=6), 1, 10, 3),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=8192 + 61, steps=8), 3, 80, 1),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64, steps=6), 4, 150, 2),
]


@pytest.mark.parametrize("name,scale,splits,slots,width", BUFFER_CASES,
                         ids=[f"{c[0]}-{c[3]}x{c[4]}" for c in BUFFER_CASES])
def test_buffered_trajectory_vs_oracle(name, scale, splits, slots, width):
    """Host tier with a buffer against the oracle: selections, swap lists
    and attention, plus every slot's block and timestamp and the misses
    per pair (the oracle's bucketed LRU over its own selections)."""
    w = WORKLOADS[name].scaled(**scale)
    run_trajectory(w, seed=33, splits=splits, offload=True, buffer_slots=slots, bucket_width=width)


@pytest.mark.parametrize("name,scale,splits,slots,width", BUFFER_CASES[::2],
                         ids=[f"{c[0]}-{c[3]}x{c[4]}" for c in BUFFER_CASES[::2]])
def test_buffered_equals_resident(name, scale, splits, slots, width):
    """The buffered host-tier step gives the resident step's bits, and
    every resident slot (selected or buffered) holds its block's pages as
    they are in host memory."""
    w = WORKLOADS[name].scaled(**scale)
    announce(f"buffered host tier vs resident {name} {scale} P={splits} slots={slots} width={width}")
    inp = synth.generate(w, 34)
    a = session(w, inp, splits=splits, offload=True, buffer_slots=slots, bucket_width=width)
    s = session(w, inp, splits=splits, select_decode=False)  # the host tier's call sequence
    for t in range(1, w.steps + 1):
        a.step(t)
        s.step(t)
        torch.cuda.synchronize()
        assert int(a.err.item()) == 0 and int(s.err.item()) == 0
        for n in ["sel_count", "evicted", "o", "m", "l", "part_o", "part_m", "part_l", "seq_lens", "score_q"]:
            x, y = getattr(a, n), getattr(s, n)
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), (n, t)
        res, own = a.resident.cpu().numpy(), a.slot_owner.cpu().numpy()
        sel, cnt = a.sel.cpu().numpy(), a.sel_count.cpu().numpy()
        dk, dv, de = a.k_pages.cpu(), a.v_pages.cpu(), a.e_pages.cpu()
        for b in range(w.B):
            for h in range(w.Hkv):
                bh = b * w.Hkv + h
                assert set(sel[b, h, :cnt[b, h]].tolist()) <= set(np.nonzero(res[b, h] >= 0)[0].tolist())
                for x in np.nonzero(res[b, h] >= 0)[0].tolist():
                    dp = int(res[b, h, x])
                    assert bh * a.slots <= dp < (bh + 1) * a.slots and own[b, h, dp - bh * a.slots] == x
                    hp = host_page(w, inp, b, h, x)
                    assert torch.equal(dk[dp], a.host_k[hp]) and torch.equal(dv[dp], a.host_v[hp]), (t, b, h, x)
                    assert torch.equal(de[dp].view(torch.int32), a.host_e[hp].view(torch.int32)), (t, b, h, x)
                assert int((own[b, h] >= 0).sum()) == int((res[b, h] >= 0).sum())


MASS_CASES = [
    ("tiny_nosa", {}, 2),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 3),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 4),
    ("dense_8b_8k", dict(B=2, Hq=8, Hkv=2, T0=2048 + 40), 5),
]


@pytest.mark.parametrize("name,scale,splits", MASS_CASES, ids=[f"{c[0]}-P{c[2]}" for c in MASS_CASES])
def test_softmax_mass_trajectory(name, scale, splits):
    """The softmax score step against the oracle along a trajectory (every
    pair, every step), with selections, swap lists and attention checked as
    in the other trajectories."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    run_trajectory(w, seed=35, splits=splits, steps=min(w.steps, 6), mass=True)


@pytest.mark.parametrize("name,scale,splits", MASS_CASES[1:3], ids=[f"{c[0]}-P{c[2]}" for c in MASS_CASES[1:3]])
def test_softmax_mass_keeps_attention_bits(name, scale, splits):
    """With the score step the attention outputs are the same bits as the
    plain decode's (the separate calls, which visit the tiles in the same
    order), and every head's masses sum to 1."""
    w = WORKLOADS[name].scaled(**scale)
    announce(f"mass vs plain decode bits {name} {scale} P={splits}")
    inp = synth.generate(w, 36)
    a = session(w, inp, splits=splits, mass=True)
    s = session(w, inp, splits=splits, fused=False)
    for t in range(1, 5):
        a.step(t)
        s.step(t)
        torch.cuda.synchronize()
        for n in ["sel_count", "o", "m", "l", "part_o", "part_m", "part_l"]:
            x, y = getattr(a, n), getattr(s, n)
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), (n, t)
        assert torch.allclose(a.mass.sum(dim=2), torch.ones_like(a.m), rtol=0, atol=1e-5)
        assert not a.counters.any().item()


ALIBI_CASES = [
    ("tiny_nosa", {}, 2),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 4),
    ("dense_8b_8k", dict(B=2, Hq=8, Hkv=2, T0=2048 + 40), 5),
]


@pytest.mark.parametrize("name,scale,splits", ALIBI_CASES, ids=[f"{c[0]}-P{c[2]}" for c in ALIBI_CASES])
def test_alibi_trajectory(name, scale, splits):
    """ALiBi decode against the oracle (bias -slope (n - t) at attention
    time) along a trajectory, every pair and step."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    run_trajectory(w, seed=37, splits=splits, steps=min(w.steps, 6), alibi=True)


def test_alibi_full_size_sampled():
    """ALiBi at the 8B shape @32K in the benchmark's launch configuration,
    sampled pairs against the oracle."""
    w = WORKLOADS["llama3_8b_32k"]
    run_trajectory(w, seed=38, steps=2, alibi=True, pairs=[(0, 0), (9, 4), (31, 7)])


QKV_CASES = [
    ("tiny_nosa", {}, 2),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1),
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 4),
]


@pytest.mark.parametrize("name,scale,splits", QKV_CASES, ids=[f"{c[0]}-P{c[2]}" for c in QKV_CASES])
def test_qkv_append_trajectory(name, scale, splits):
    """The append from fused projection rows (QKV split + eviction head +
    pooling in one launch) against the oracle along a trajectory."""
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    run_trajectory(w, seed=41, splits=splits, steps=min(w.steps, 6), qkv=True)


def test_qkv_append_pages_and_split_query():
    """The split query is the row's query bit for bit, the appended K and V
    land exactly as with separate inputs, and each appended logit is the
    oracle's eviction head of the token's value vector."""
    w = WORKLOADS["llama3_8b_32k"].scaled(B=2, Hq=8, Hkv=2, T0=4096 + 61)
    announce("qkv append: split query, pages, eviction logits")
    inp = synth.generate(w, 42)
    a = session(w, inp, splits=1, qkv=True)
    s = session(w, inp, splits=1)
    w_e = synth.eviction_head_weights(w, inp.seed)
    for t in range(1, 4):
        a.step(t)
        s.step(t)
        torch.cuda.synchronize()
        assert int(a.err.item()) == 0
        assert np.array_equal(a.q_out.cpu().numpy().view(np.uint16), inp.q(t))
        assert torch.equal(a.k_pages, s.k_pages) and torch.equal(a.v_pages, s.v_pages)
        assert torch.equal(a.seq_lens, s.seq_lens)
        pos = w.T0 + t - 1
        ep = a.e_pages.cpu().numpy()
        for b in range(w.B):
            for h in range(w.Hkv):
                page = host_page(w, inp, b, h, pos // w.bs)
                want = oracle.eviction_head(oracle.bf16_to_f64(inp.V[b, h, pos]), w_e[h])
                assert ep[page, pos % w.bs] == want, (t, b, h)


def run_prefill(w, seed, rows=None, pairs=None):
    """nosa_prefill_attention against the oracle's prefill for the given
    prompt rows (all by default) of the given pairs (all by default)."""
    announce(f"prefill {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} T0={w.T0} prompt={w.prompt} "
             f"docs={w.n_docs}x{w.doc_len} seed={seed} rows={'all' if rows is None else rows}")
    inp = synth.generate(w, seed)
    sess = session(w, inp)
    sess.prefill_attention()
    torch.cuda.synchronize()
    assert int(sess.err.item()) == 0
    O, m, l = sess.pf_o.cpu().numpy(), sess.pf_m.cpu().numpy(), sess.pf_l.cpu().numpy()
    qp = synth.prefill_queries(w, inp.seed)
    starts = synth.block_doc_start(w) * w.bs
    rows = list(range(w.prompt)) if rows is None else rows
    for (b, h) in pairs or [(b, h) for b in range(w.B) for h in range(w.Hkv)]:
        lg = logical_pair(inp, b, h)
        hs = slice(h * w.G, (h + 1) * w.G)
        q = oracle.bf16_to_f64(qp[b, rows][:, hs])
        # only the requested rows: the oracle's prefill over a row subset
        Ow, mw, lw = oracle.prefill_attention_bh(q, lg.K, lg.V, w.T0, w.T0 - w.prompt, starts, w.bs,
                                                  w.rope_base, w.sm_scale) if rows == list(range(w.prompt)) else \
            _prefill_rows(q, lg, w, rows, starts)
        where = f"{w.name} b={b} h={h}"
        got_o, got_m, got_l = O[b, rows][:, hs], m[b, rows][:, hs], l[b, rows][:, hs]
        assert np.abs(got_o - Ow).max() <= 1e-2, (where, "O", float(np.abs(got_o - Ow).max()))
        assert np.abs(got_m + np.log(got_l) - mw - np.log(lw)).max() <= 1e-3, (where, "LSE")
        assert np.abs(got_m - mw).max() <= 1e-3, (where, "m")


def _prefill_rows(q, lg, w, rows, starts):
    """The oracle's prefill for a subset of prompt rows: each row on its own
    (a prompt of one query at its position)."""
    outs = [oracle.prefill_attention_bh(q[j:j + 1], lg.K, lg.V, w.T0, w.T0 - w.prompt + r, starts, w.bs,
                                        w.rope_base, w.sm_scale) for j, r in enumerate(rows)]
    return tuple(np.concatenate([o[k] for o in outs]) for k in range(3))


PREFILL_CASES = [
    ("G4", dict(B=2, Hq=8, Hkv=2, T0=9 * 128, n_docs=9, doc_len=128, prompt=128)),
    ("G4-ragged", dict(B=1, Hq=8, Hkv=2, T0=8 * 128 + 100, n_docs=9, doc_len=128, prompt=100)),
    ("G8", dict(B=1, Hq=16, Hkv=2, T0=5 * 256, n_docs=5, doc_len=256, prompt=256)),
    ("G1", dict(B=1, Hq=2, Hkv=2, T0=9 * 128, n_docs=9, doc_len=128, prompt=128)),
    ("D64-bs128", dict(B=1, Hq=8, Hkv=2, D=64, bs=128, ss=32, T0=5 * 256, n_docs=5, doc_len=256, prompt=200)),
    ("G2", dict(B=1, Hq=4, Hkv=2, T0=9 * 128, n_docs=9, doc_len=128, prompt=128)),
    ("G16-bs256", dict(B=1, Hq=32, Hkv=2, bs=256, ss=64, T0=5 * 256, n_docs=5, doc_len=256, prompt=256)),
]


@pytest.mark.parametrize("name,scale", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_small(name, scale):
    run_prefill(WORKLOADS["lazy_prefill_33k"].scaled(**scale), seed=43)


def test_prefill_full_size_sampled():
    """The full prefill workload (64 documents of 512 tokens + a 512-token
    prompt), sampled rows and pairs against the oracle."""
    w = WORKLOADS["lazy_prefill_33k"]
    run_prefill(w, seed=0, rows=[0, 1, 63, 64, 255, 511], pairs=[(0, 0), (3, 7)])


def test_prefill_three_runs_of_tiles():
    """A context of 1,300 tiles: the kernel looks the pages up in runs of
    512 tiles, so this crosses two run boundaries (two reloads of the run
    table), with documents of 640 tokens starting mid-run."""
    w = WORKLOADS["lazy_prefill_33k"].scaled(B=1, Hq=8, Hkv=2, T0=130 * 640, n_docs=130, doc_len=640, prompt=640)
    run_prefill(w, seed=50, rows=[0, 1, 300, 639], pairs=[(0, 1)])


# ---------------------------------------------------------------------------
# edge cases of the extensions: empty context, zero budgets, the widest
# capacity, one-token prompts, appends past capacity
# ---------------------------------------------------------------------------

EXT_MODES = [
    ("mass", dict(mass=True)),
    ("alibi", dict(alibi=True)),
    ("qkv", dict(qkv=True)),
    ("offload", dict(offload=True)),
    ("buffer", dict(offload=True, buffer_slots=10, bucket_width=1)),
]


@pytest.mark.parametrize("mode,kw", EXT_MODES, ids=[m[0] for m in EXT_MODES])
def test_extensions_empty_context(mode, kw):
    # the first step appends token 0 and attends to it alone
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=0)
    run_trajectory(w, seed=44, steps=6, **kw)


@pytest.mark.parametrize("mode,kw", EXT_MODES, ids=[m[0] for m in EXT_MODES])
@pytest.mark.parametrize("k_e,k_q", [(0, 6), (6, 0)])
def test_extensions_zero_budgets(mode, kw, k_e, k_q):
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=8, Hkv=2, T0=1500, k_e=k_e, k_q=k_q)
    run_trajectory(w, seed=45, steps=4, **kw)


@pytest.mark.parametrize("mode,kw", [m for m in EXT_MODES if m[0] in ("mass", "buffer")],
                         ids=["mass", "buffer"])
def test_extensions_maximum_capacity(mode, kw):
    # 8192 blocks of capacity
    w = WORKLOADS["tiny_nosa"].scaled(B=1, Hq=4, Hkv=1, T0=8192 * 64 - 256 - 10, k_e=6, k_q=10)
    kw = dict(kw, buffer_slots=24) if mode == "buffer" else kw
    run_trajectory(w, seed=46, steps=3, splits=3, **kw)


def test_prefill_one_token_prompt():
    # a prompt of one token (the last document holds just it), 128-token blocks
    w = WORKLOADS["lazy_prefill_33k"].scaled(B=1, Hq=8, Hkv=2, bs=128, ss=32, T0=4 * 128 + 1, n_docs=5,
                                              doc_len=128, prompt=1)
    run_prefill(w, seed=47)


def test_prefill_unresolvable_page_flags_and_stays_finite():
    # one context block's packed word names a page past the pool: the kernel
    # flags the error, loads nothing from it (its tile is zero-filled and
    # masked), and every other pair still matches the oracle
    w = WORKLOADS["lazy_prefill_33k"].scaled(B=1, Hq=8, Hkv=2, T0=9 * 128, n_docs=9, doc_len=128, prompt=128)
    announce("prefill with an unresolvable page: error flag, finite outputs")
    inp = synth.generate(w, 49)
    sess = session(w, inp)
    bad_pair, bad_block = 1, 3  # (b, KV head) pair 1 = (0, 1)
    packed = sess.packed.view(w.B * w.Hkv, w.max_blocks)
    packed[bad_pair, bad_block] = (1 << 20) - 1  # page id 2^20 - 1 >= num_pages, document start 0
    assert (1 << 20) - 1 >= w.num_pages
    sess.prefill_attention()
    torch.cuda.synchronize()
    assert int(sess.err.item()) == 1
    O, m, l = sess.pf_o.cpu().numpy(), sess.pf_m.cpu().numpy(), sess.pf_l.cpu().numpy()
    assert np.isfinite(O).all() and np.isfinite(m).all() and np.isfinite(l).all()
    # pair 0 never reads the bad entry: it matches the oracle as usual
    qp = synth.prefill_queries(w, inp.seed)
    starts = synth.block_doc_start(w) * w.bs
    lg = logical_pair(inp, 0, 0)
    q = oracle.bf16_to_f64(qp[0][:, 0:w.G])
    Ow, mw, lw = oracle.prefill_attention_bh(q, lg.K, lg.V, w.T0, w.T0 - w.prompt, starts, w.bs,
                                              w.rope_base, w.sm_scale)
    assert np.abs(O[0][:, 0:w.G] - Ow).max() <= 1e-2
    assert np.abs(m[0][:, 0:w.G] - mw).max() <= 1e-3


def test_qkv_append_past_capacity_flags_and_keeps_length():
    from block_sparse_kv_score_amd import nosa
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=100)
    announce("qkv append past capacity: error flag, lengths unchanged")
    inp = synth.generate(w, 48)
    sess = session(w, inp, qkv=True)
    cap = w.max_blocks * w.bs
    full = torch.full((w.B,), cap, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(full)
    nosa.nosa_append_score_qkv(sess.dims, sess.kv, sess.qkv_all[0], sess.w_evict, full, out, sess.k_summary,
                               sess.e_summary, sess.q_out, sess.score_q, sess.score_e)
    torch.cuda.synchronize()
    assert int(sess.err.item()) == 1 and out.tolist() == [cap] * w.B


def test_offload_more_loads_than_slots_flags():
    from block_sparse_kv_score_amd import nosa
    w = WORKLOADS["tiny_nosa"].scaled(B=1, Hq=4, Hkv=1, T0=1500)
    announce("host tier: more loads than free slots sets the error flag")
    inp = synth.generate(w, 31)
    a = session(w, inp, offload=True)
    t = 1
    a.use_buffers(t)
    a.append_score(t)
    a.select_swap()
    torch.cuda.synchronize()
    n_load = int(a.load_count.item())
    small = torch.full((1, 1, max(n_load - 2, 1)), -1, dtype=torch.int32, device="cuda")
    nosa.nosa_retrieve(a.dims, a.host_kv, a.k_pages, a.v_pages, a.e_pages, max(n_load - 2, 1), a.resident,
                       small, a.load, a.load_count, a.evict, a.evict_count, a.seq_lens)
    torch.cuda.synchronize()
    assert n_load > 2 and int(a.err.item()) == 1
    assert int((a.resident >= 0).sum().item()) == max(n_load - 2, 1)


# ---------------------------------------------------------------------------
# full sizes, launch configuration of the benchmark
# ---------------------------------------------------------------------------

def test_dense_8b_8k_full():
    # every pair (k = all 128 blocks, 16 splits)
    run_trajectory(WORKLOADS["dense_8b_8k"], seed=0, check_scores=False)


def test_8b_32k_full_sampled():
    """The headline workload in the benchmark's launch configuration: every
    one of the 256 pairs against the oracle at the first and the last of
    its 8 steps, four sampled pairs at every step, invariants on every pair
    at every step."""
    w = WORKLOADS["llama3_8b_32k"]
    run_trajectory(w, seed=0, pairs=[(0, 0), (5, 3), (17, 7), (31, 2)], all_pairs_at=(1, w.steps))


def test_70b_256k_full_sampled():
    # every one of the 64 pairs at the last of the 4 steps
    w = WORKLOADS["llama31_70b_256k"]
    run_trajectory(w, seed=0, pairs=[(0, 0), (3, 5), (7, 7)], all_pairs_at=(w.steps,))


def test_lazy_rope_sparse_32k_full_sampled():
    w = WORKLOADS["lazy_rope_sparse_32k"]
    run_trajectory(w, seed=0, steps=2, pairs=[(0, 0), (33, 5), (63, 7)])


def test_lazy_rope_32k_full_sampled():
    w = WORKLOADS["lazy_rope_32k"]
    run_trajectory(w, seed=0, pairs=[(0, 0), (21, 4), (63, 7)])
