"""Pins for the float64 oracle: checks against things other than the oracle
itself (a library routine, closed forms worked by hand, brute force over all
subsets, invariants the pages state).

Each ``check_*`` takes the oracle module ``O`` and raises AssertionError on a
violation, so the same checks can be run against planted mistakes
(``test_oracle_mutations.py``) to show that they catch them.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import torch


def _sdpa(q, K, V, scale):
    """torch's CPU scaled-dot-product attention in float64 (library route)."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(K), t(V), scale=scale)[0, 0].numpy()


# ---------------------------------------------------------------------------
# attention + split merge
# ---------------------------------------------------------------------------

def check_attend_vs_sdpa(O, seed=0):
    rng = np.random.default_rng(seed)
    for G, n, D in [(1, 1, 4), (4, 7, 16), (8, 130, 64), (4, 257, 128)]:
        q = rng.standard_normal((G, D))
        K = rng.standard_normal((n, D)) * 2.0
        V = rng.standard_normal((n, D))
        scale = 1.0 / math.sqrt(D)
        out, m, l = O.attend(q, K, V, scale)
        ref = _sdpa(q, K, V, scale)
        assert np.abs(out - ref).max() <= 1e-12, "O differs from SDPA"
        s = torch.tensor(q) @ torch.tensor(K).T * scale
        lse = torch.logsumexp(s, dim=1).numpy()
        assert np.abs(m + np.log(l) - lse).max() <= 1e-12, "m + ln l differs from logsumexp"
        smax = torch.max(s, dim=1).values.numpy()
        assert np.abs(m - smax).max() <= 1e-12 * max(1.0, np.abs(smax).max()), "m is not the row max"
    out, m, l = O.attend(np.ones((3, 8)), np.zeros((0, 8)), np.zeros((0, 8)), 0.5)
    assert np.all(out == 0) and np.all(np.isneginf(m)) and np.all(l == 0), "empty token set"


def check_merge_vs_sdpa(O, seed=1):
    rng = np.random.default_rng(seed)
    D = 32
    for trial in range(20):
        n = int(rng.integers(1, 90))
        P = int(rng.integers(1, 9))
        cuts = np.sort(rng.integers(0, n + 1, size=P - 1))
        bounds = [0, *cuts.tolist(), n]
        q = rng.standard_normal((1, D))
        K = rng.standard_normal((n, D)) * 3.0
        V = rng.standard_normal((n, D))
        parts = [O.attend(q, K[a:b], V[a:b], 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
        o_p = np.stack([p[0][0] for p in parts])
        m_p = np.array([p[1][0] for p in parts])
        l_p = np.array([p[2][0] for p in parts])
        Om, mm, lm = O.merge_partials(o_p, m_p, l_p)
        ref = _sdpa(q, K, V, 0.25)[0]
        assert np.abs(Om - ref).max() <= 1e-12, "merged O differs from SDPA"
        s = torch.tensor(q[0]) @ torch.tensor(K).T * 0.25
        assert abs(mm + math.log(lm) - float(torch.logsumexp(s, 0))) <= 1e-12, "merged LSE"
        assert abs(mm - float(s.max())) <= 1e-12, "merged m is not the global max"
    Om, mm, lm = O.merge_partials(np.zeros((3, D)), np.full(3, -np.inf), np.zeros(3))
    assert np.all(Om == 0) and mm == -np.inf and lm == 0, "all-empty merge"


def check_split_chunks(O):
    for n in range(0, 40):
        sel = list(range(100, 100 + n))
        for P in range(1, 12):
            ch = O.split_chunks(sel, P)
            assert len(ch) == P
            assert [x for c in ch for x in c] == sel, "chunks must tile the list in order"
            c = -(-n // P) if n else 0
            assert all(len(x) <= c for x in ch)


# ---------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------

# token scores worked by hand: bs = 8, ss = 4 (two sub-blocks per block)
_F = [3, 1, 2, 2, 0, 0, 9, 3,      # block 0: sub means 2 and 3        -> 3
      5, 5, 5, 5, 1, 1, 1, 1,      # block 1: sub means 5 and 1        -> 5
      -2, -2, -2, -2, 7]           # block 2: sub means -2 and 7 (1 token) -> 7


def _keys_for_scores(f, g_noise):
    """D = 4, G = 2 keys/queries whose group-mean score q.k/sqrt(4) is f[t]:
    heads (3, 5) and (1, -5) average to (2, 0); keys (f, noise)."""
    T = len(f)
    K = np.zeros((T, 4))
    K[:, 0] = f
    K[:, 1] = g_noise
    q = np.array([[3.0, 5.0, 0.0, 0.0], [1.0, -5.0, 0.0, 0.0]])
    return q, K


def check_pool_closed_form(O, seed=2):
    rng = np.random.default_rng(seed)
    q, K = _keys_for_scores(_F, rng.standard_normal(len(_F)))
    s = O.query_token_scores(q, K)
    assert np.abs(s - np.array(_F, dtype=float)).max() <= 1e-12, "group-mean token score"
    S = O.pool_block_scores(s, len(_F), 8, 4)
    assert np.array_equal(S, [3.0, 5.0, 7.0]), S
    # T = 17: block 2 is one token (-2); its empty second sub-block is ignored
    S17 = O.pool_block_scores(s[:17], 17, 8, 4)
    assert np.array_equal(S17, [3.0, 5.0, -2.0]), S17
    # ss = 1 reduces to the per-token max, ss = bs to the block mean
    f = rng.standard_normal(45)
    S1 = O.pool_block_scores(f, 45, 8, 1)
    Sb = O.pool_block_scores(f, 45, 8, 8)
    for i in range(6):
        seg = f[i * 8:min(i * 8 + 8, 45)]
        assert S1[i] == seg.max(), "ss = 1 must be the max over tokens"
        assert abs(Sb[i] - seg.sum() / len(seg)) <= 1e-15, "ss = bs must be the block mean"
    assert len(S1) == 6 and len(Sb) == 6


def check_pool_linearity(O, seed=3):
    """Pooling the per-token scores equals scoring the sub-block mean keys
    with the group-mean query (mean and dot product are both linear)."""
    rng = np.random.default_rng(seed)
    for G, D, T, bs, ss in [(4, 16, 200, 16, 4), (8, 32, 131, 32, 8), (1, 8, 64, 64, 16)]:
        q = rng.standard_normal((G, D))
        K = rng.standard_normal((T, D))
        S = O.pool_block_scores(O.query_token_scores(q, K), T, bs, ss)
        qbar = q.sum(axis=0) / G
        nb = -(-T // bs)
        ref = np.full(nb, -np.inf)
        for t0 in range(0, T, ss):
            kbar = K[t0:min(t0 + ss, T)].sum(axis=0) / (min(t0 + ss, T) - t0)
            ref[t0 // bs] = max(ref[t0 // bs], float(kbar @ qbar) / math.sqrt(D))
        assert np.abs(S - ref).max() <= 1e-12


def check_eviction_pre_exp(O):
    """ED-DMA: the block order comes from pooled raw logits.  Block 0 has
    sub-block logits (10, -10) -> mean 0, block 1 has (1, 1) -> mean 1; mean
    of exponentials would rank block 0 first instead."""
    e = O.eviction_token_scores(np.array([10.0, -10.0, 1.0, 1.0]))
    E = O.pool_block_scores(e, 4, 2, 2)
    assert np.array_equal(E, [0.0, 1.0]), E
    ge, gq, g, ev = O.select_blocks(np.zeros(2), E, 2, 1, 0, set())
    assert ge == [1] and ev == {0}


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

def _best_subset(scores, cand, k):
    """Brute force: among the k-subsets with the largest score sum, the
    lexicographically first (== lowest indices among ties)."""
    combos = list(itertools.combinations(sorted(cand), k))
    best = max(sum(float(scores[i]) for i in c) for c in combos)
    return set(min(c for c in combos if sum(float(scores[i]) for i in c) == best))


def check_select_bruteforce(O, seed=4, trials=300, ties=False):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        nb = int(rng.integers(1, 9))
        k_e = int(rng.integers(0, nb + 2))
        k_q = int(rng.integers(0, nb + 2))
        if ties:
            E = rng.integers(0, 3, nb).astype(float)
            S = rng.integers(-1, 2, nb).astype(float)
        else:
            E = rng.standard_normal(nb)
            S = rng.standard_normal(nb)
        evicted = {i for i in range(nb) if rng.random() < 0.3}
        ge, gq, g, ev = O.select_blocks(S, E, nb, k_e, k_q, set(evicted))
        C = [i for i in range(nb) if i not in evicted]
        ne = min(k_e, len(C))
        assert set(ge) == _best_subset(E, C, ne), ("eviction part", nb, k_e, evicted)
        assert len(ge) == ne
        rest = [i for i in range(nb) if i not in ge]
        nq = min(k_q, len(rest))
        assert set(gq) == _best_subset(S, rest, nq), ("query part", nb, k_q)
        assert g == sorted(set(ge) | set(gq))
        assert len(g) == min(len(ge) + k_q, nb)
        assert g == sorted(g) and len(set(g)) == len(g)
        assert ev == set(evicted) | (set(C) - set(ge)), "every unkept candidate is evicted"


def check_select_sizes(O, seed=5):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        nb = int(rng.integers(1, 60))
        k_e, k_q = int(rng.integers(0, 20)), int(rng.integers(0, 20))
        ge, gq, g, ev = O.select_blocks(rng.standard_normal(nb), rng.standard_normal(nb), nb, k_e, k_q, set())
        assert len(ge) == min(k_e, nb), "|Gamma_e| = min(k_e, nb) from a fresh state"
        assert len(g) == min(k_e + k_q, nb), "|Gamma| = min(k, nb): the parts are disjoint"
        assert not set(ge) & set(gq)
        if k_e + k_q >= nb:
            assert g == list(range(nb)), "k >= nb selects every block"


def check_trajectory_invariants(O, seed=6, steps=40):
    """Monotone eviction and the locality bound over a synthetic trajectory:
    blocks are created as tokens arrive; scores are redrawn every step."""
    rng = np.random.default_rng(seed)
    for k_e, k_q, bs, T0 in [(4, 4, 4, 64), (3, 5, 2, 20), (6, 2, 8, 200), (1, 1, 1, 5)]:
        k = k_e + k_q
        evicted, prev_e, prev = set(), None, None
        for t in range(1, steps + 1):
            T = T0 + t
            nb = -(-T // bs)
            nb_prev = -(-(T - 1) // bs)
            new = set(range(nb_prev, nb)) if t > 1 else set(range(nb))
            ge, gq, g, ev = O.select_blocks(rng.standard_normal(nb), rng.standard_normal(nb), nb, k_e, k_q, evicted)
            assert evicted <= ev, "the evicted set never shrinks"
            assert not set(ge) & evicted, "an evicted block never returns to the eviction part"
            if prev_e is not None:
                assert set(ge) <= set(prev_e) | new, "Gamma_e(t) within Gamma_e(t-1) and new blocks"
                gamma = len(set(g) & set(prev)) / len(g)
                bound = (k_e - len(new & set(ge))) / k
                assert gamma >= bound - 1e-15, ("locality", gamma, bound)
                if not new:
                    assert gamma >= k_e / k - 1e-15
            evicted, prev_e, prev = ev, ge, g


def check_swap_lists(O, seed=7):
    load, drop = O.swap_lists([1, 3, 5, 7], [3, 4, 5, 8])
    assert load == [4, 8] and drop == [1, 7], (load, drop)
    assert O.swap_lists([], [2, 0]) == ([0, 2], [])
    rng = np.random.default_rng(seed)
    for _ in range(200):
        prev = sorted(set(rng.integers(0, 30, rng.integers(0, 12)).tolist()))
        cur = sorted(set(rng.integers(0, 30, rng.integers(0, 12)).tolist()))
        load, drop = O.swap_lists(prev, cur)
        both = set(prev) & set(cur)
        assert set(load) | both == set(cur) and not set(load) & both
        assert set(drop) | both == set(prev) and not set(drop) & both
        assert not set(load) & set(drop)
        assert load == sorted(load) and drop == sorted(drop)


def check_place_blocks(O, seed=8):
    """Host-tier slot placement: a worked example by hand, brute-force
    checks of the placement rule on random slot states, and a selection
    trajectory in which the resident set always equals the selection."""
    # slots [5, -, 2, 7]; drop 2; load 1 then 9 -> free slots 1, 2
    assert O.place_blocks([5, -1, 2, 7], [2], [1, 9]) == ([5, 1, 9, 7], 2)
    # dropping a block that is not resident changes nothing
    assert O.place_blocks([4, -1], [6], [3]) == ([4, 3], 1)
    # more loads than free slots: the extra ones are not placed
    assert O.place_blocks([0, -1, -1], [], [3, 4, 5]) == ([0, 3, 4], 2)
    rng = np.random.default_rng(seed)
    for _ in range(300):
        RS = int(rng.integers(1, 12))
        pool = rng.permutation(40)
        n_res = int(rng.integers(0, RS + 1))
        owner = [-1] * RS
        for s, x in zip(rng.permutation(RS)[:n_res], pool[:n_res]):
            owner[int(s)] = int(x)
        resident = [x for x in owner if x >= 0]
        drop = [x for x in resident if rng.random() < 0.4] + [int(x) for x in pool[30:32]]
        load = [int(x) for x in pool[n_res:n_res + int(rng.integers(0, RS + 2))]]
        new, placed = O.place_blocks(owner, drop, load)
        kept = set(resident) - set(drop)
        free_after_drop = sorted(s for s in range(RS) if owner[s] < 0 or owner[s] in set(drop))
        assert placed == min(len(load), len(free_after_drop))
        for s in range(RS):  # kept blocks never move
            if owner[s] in kept:
                assert new[s] == owner[s]
        assert set(x for x in new if x >= 0) == kept | set(load[:placed])
        assert len([x for x in new if x >= 0]) == len(kept) + placed
        # brute force over the slots: every free slot below a loaded one is
        # taken by an earlier load, and loads land in list order
        slot_of = {x: s for s, x in enumerate(new) if x >= 0}
        used = [slot_of[x] for x in load[:placed]]
        assert used == sorted(used)
        for s in free_after_drop:
            if used and s < used[-1]:
                assert s in used
    # along a dual-selection trajectory with as many slots as the budget,
    # the swap lists keep the resident set equal to the selection
    nb, k_e, k_q = 40, 6, 4
    owner, evicted, prev = [-1] * (k_e + k_q), set(), []
    for t in range(25):
        nbt = nb + t // 3
        S_q = rng.standard_normal(nbt)
        E = rng.standard_normal(nbt)
        _, _, g, evicted = O.select_blocks(S_q, E, nbt, k_e, k_q, evicted)
        load, drop = O.swap_lists(prev, g)
        owner, placed = O.place_blocks(owner, drop, load)
        assert placed == len(load)
        assert sorted(x for x in owner if x >= 0) == g
        prev = g


def check_buffer_retrieve(O, seed=9):
    """Host tier with a buffer: a worked example by hand, the bucket's
    closed form, agreement with the plain swap placement when the buffer
    holds exactly the selection, agreement with an exact LRU while every
    page is younger than the last bucket, and the eviction-order invariants
    on random states."""
    # slots [5, -, 2, 7], stamps [3, 0, 1, 2]; step 4 selects {1, 5, 9}:
    # 5 is a hit; misses 1, 9; one free slot, so the oldest buffered page
    # (block 2, last used at step 1) goes; 1 -> slot 1, 9 -> slot 2
    assert O.buffer_retrieve([5, -1, 2, 7], [3, 0, 1, 2], [1, 5, 9], 4, 1) == \
        ([5, 1, 9, 7], [4, 4, 4, 2], [1, 9], [2], 2)
    assert [O.recency_bucket(a, 1) for a in (1, 2, 64, 65, 10 ** 6)] == [0, 1, 63, 63, 63]
    assert [O.recency_bucket(a, 4) for a in (1, 4, 5, 8, 9, 256, 257)] == [0, 0, 1, 1, 2, 63, 63]
    rng = np.random.default_rng(seed)
    # (1) a buffer of exactly k slots with k-block selections is the plain
    # swap placement, step by step
    nb, k_e, k_q = 48, 5, 3
    k = k_e + k_q
    plain, buf, stamps, evicted, prev = [-1] * k, [-1] * k, [0] * k, set(), []
    for t in range(1, 30):
        _, _, g, evicted = O.select_blocks(rng.standard_normal(nb + t), rng.standard_normal(nb + t), nb + t,
                                           k_e, k_q, evicted)
        load, drop = O.swap_lists(prev, g)
        plain, _ = O.place_blocks(plain, drop, load)
        buf, stamps, misses, dropped, placed = O.buffer_retrieve(buf, stamps, g, t, 3)
        assert buf == plain and misses == load and sorted(dropped) == drop and placed == len(load)
        prev = g
    # (2) with one-step buckets and fewer than 64 steps, the bucketed LRU
    # is the exact LRU
    for trial in range(20):
        RS = int(rng.integers(4, 12))
        owner, lu, ref_owner, ref_lu = [-1] * RS, [0] * RS, [-1] * RS, [0] * RS
        for t in range(1, 50):
            n = int(rng.integers(1, RS + 1))
            sel = sorted(rng.choice(20, n, replace=False).tolist())
            owner, lu, misses, dropped, placed = O.buffer_retrieve(owner, lu, sel, t, 1)
            assert placed == len(misses)
            # reference: exact LRU victims, then the same slot rule
            where = {x: s for s, x in enumerate(ref_owner) if x >= 0}
            for x in sel:
                if x in where:
                    ref_lu[where[x]] = t
            ref_miss = [x for x in sel if x not in where]
            free = [s for s in range(RS) if ref_owner[s] < 0]
            victims = sorted((s for s in range(RS) if ref_owner[s] >= 0 and ref_owner[s] not in sel),
                             key=lambda s: (ref_lu[s], s))[:max(0, len(ref_miss) - len(free))]
            assert sorted(ref_owner[s] for s in victims) == sorted(dropped), (trial, t)
            for s in victims:
                ref_owner[s] = -1
            for s, x in zip([s for s in range(RS) if ref_owner[s] < 0], ref_miss):
                ref_owner[s], ref_lu[s] = x, t
            assert ref_owner == owner and ref_lu == lu, (trial, t)
    # (3) invariants on random states and wider buckets
    for _ in range(300):
        RS = int(rng.integers(2, 16))
        width = int(rng.integers(1, 5))
        t = int(rng.integers(2, 400))
        blocks = rng.permutation(60)
        owner = [int(blocks[s]) if rng.random() < 0.8 else -1 for s in range(RS)]
        lu = [int(rng.integers(max(0, t - 300), t)) for _ in range(RS)]
        n = int(rng.integers(0, RS + 1))
        pool = [x for x in owner if x >= 0][:n // 2] + [int(x) for x in blocks[RS:RS + n - n // 2]]
        sel = sorted(set(pool))
        new, nlu, misses, dropped, placed = O.buffer_retrieve(owner, lu, sel, t, width)
        was = {x: s for s, x in enumerate(owner) if x >= 0}
        assert misses == [x for x in sel if x not in was]
        assert placed == len(misses) and set(sel) <= set(new)
        n_free = owner.count(-1)
        assert len(dropped) == max(0, len(misses) - n_free)
        assert not set(dropped) & set(sel)
        for x in sel:
            if x in was:  # hits keep their slot and take the new timestamp
                assert new[was[x]] == x and nlu[was[x]] == t
        kept = [s for s, x in enumerate(owner) if x >= 0 and x not in sel and x not in dropped]
        for d in dropped:
            sd = was[d]
            bd = O.recency_bucket(t - lu[sd], width)
            for sk in kept:
                bk = O.recency_bucket(t - lu[sk], width)
                assert bd > bk or (bd == bk and sd < sk), (bd, bk, sd, sk)
        for s in kept:
            assert new[s] == owner[s] and nlu[s] == lu[s]


def check_softmax_block_mass(O, seed=10):
    """The softmax score step: a hand-worked example, torch's softmax summed
    per block, the uniform closed form (mass = share of tokens), and the
    route through attend's returned row max and l, p = exp(s - m) / l."""
    # one dim, q = 1, keys 0, ln 2, ln 3: p = 1/6, 2/6, 3/6; blocks of 2
    K = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])
    got = O.softmax_block_mass(np.array([[1.0]]), K, [0, 1], 3, 2, 1.0)
    assert np.allclose(got, [[0.5, 0.5]], rtol=0, atol=1e-15), got
    got = O.softmax_block_mass(np.array([[1.0]]), K, [1], 3, 2, 1.0)
    assert np.allclose(got, [[1.0]], rtol=0, atol=1e-15)
    assert O.softmax_block_mass(np.ones((2, 1)), K, [], 3, 2, 1.0).shape == (2, 0)
    rng = np.random.default_rng(seed)
    for _ in range(20):
        G, D, bs = int(rng.integers(1, 5)), 8, int(rng.choice([2, 4, 8]))
        T = int(rng.integers(1, 60))
        nb = -(-T // bs)
        blocks = sorted(rng.choice(nb, int(rng.integers(1, nb + 1)), replace=False).tolist())
        q = rng.standard_normal((G, D))
        K = rng.standard_normal((T, D)) * 2
        scale = 1 / math.sqrt(D)
        got = O.softmax_block_mass(q, K, blocks, T, bs, scale)
        toks = O.tokens_of_blocks(blocks, T, bs)
        p = torch.softmax(torch.from_numpy(q @ K[toks].T * scale), dim=1).numpy()
        ref = np.zeros_like(got)
        pos = 0
        for j, i in enumerate(blocks):
            n = min(T, (i + 1) * bs) - i * bs
            ref[:, j] = p[:, pos:pos + n].sum(axis=1)
            pos += n
        assert np.abs(got - ref).max() <= 1e-12
        assert np.abs(got.sum(axis=1) - 1).max() <= 1e-12
        # the returned (m, l) route
        _, m, l = O.attend(q, K[toks], K[toks], scale)
        pos = 0
        for j, i in enumerate(blocks):
            n = min(T, (i + 1) * bs) - i * bs
            s = q @ K[toks[pos:pos + n]].T * scale
            assert np.abs(np.exp(s - m[:, None]).sum(axis=1) / l - got[:, j]).max() <= 1e-12
            pos += n
        # identical keys: mass is the share of present tokens
        flat = O.softmax_block_mass(q, np.ones((T, D)), blocks, T, bs, scale)
        counts = np.array([min(T, (i + 1) * bs) - i * bs for i in blocks], dtype=np.float64)
        assert np.abs(flat - counts / counts.sum()).max() <= 1e-12


def check_alibi(O, seed=11):
    """ALiBi: the slopes' values, a hand-worked softmax over bias alone,
    attention with the bias against torch's float64 SDPA with the same
    additive mask (and its log-sum-exp against torch.logsumexp), zero
    slopes = plain attention, and a whole dense step against SDPA."""
    assert O.alibi_slopes(8).tolist() == [2.0 ** -k for k in range(1, 9)]
    assert np.allclose(O.alibi_slopes(4), [2.0 ** -2, 2.0 ** -4, 2.0 ** -6, 2.0 ** -8], rtol=0, atol=0)
    # zero query: weights exp(-ln2 (2 - j)) = 1/4, 1/2, 1 over positions 0, 1, 2
    b = O.alibi_bias(np.array([math.log(2.0)]), 2, np.arange(3))
    Ob, mb, lb = O.attend(np.zeros((1, 1)), np.ones((3, 1)), np.arange(3, dtype=np.float64)[:, None], 1.0, b)
    assert abs(Ob[0, 0] - 10.0 / 7.0) <= 1e-15 and mb[0] == 0.0 and abs(lb[0] - 7.0 / 4.0) <= 1e-15
    rng = np.random.default_rng(seed)
    for G, n, D in [(2, 5, 8), (4, 70, 32), (8, 130, 64)]:
        q = rng.standard_normal((G, D))
        K = rng.standard_normal((n, D))
        V = rng.standard_normal((n, D))
        pos = np.sort(rng.choice(4 * n, n, replace=False))
        slopes = O.alibi_slopes(G)
        qpos = int(pos[-1]) + int(rng.integers(0, 5))
        bias = O.alibi_bias(slopes, qpos, pos)
        scale = 1 / math.sqrt(D)
        Ow, m, l = O.attend(q, K, V, scale, bias)
        t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q)[:, None], t(K)[None].expand(G, n, D), t(V)[None].expand(G, n, D), attn_mask=t(bias)[:, None],
            scale=scale)[:, 0].numpy()
        assert np.abs(Ow - ref).max() <= 1e-12
        lse = torch.logsumexp(t(q) @ t(K).T * scale + t(bias), dim=1).numpy()
        assert np.abs(m + np.log(l) - lse).max() <= 1e-12
        O0 = O.attend(q, K, V, scale, O.alibi_bias(np.zeros(G), qpos, pos))
        assert np.abs(O0[0] - _sdpa(q, K, V, scale)).max() <= 1e-12
    # the whole step, every block selected, against SDPA over all tokens
    G, D, T, bs = 4, 16, 150, 16
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    slopes = O.alibi_slopes(G)
    r = O.decode_step_bh(q, K, V, np.zeros(T), T, bs, bs, 0, 64, set(), [], 3, 1 / math.sqrt(D),
                         select_all=True, alibi=slopes)
    bias = O.alibi_bias(slopes, T - 1, np.arange(T))
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q)[:, None], t(K)[None].expand(G, T, D), t(V)[None].expand(G, T, D), attn_mask=t(bias)[:, None],
        scale=1 / math.sqrt(D))[:, 0].numpy()
    assert np.abs(r["O"] - ref).max() <= 1e-12


def check_rope_scores(O, seed=12):
    """Query-aware block scores with deferred RoPE against the complex-number
    form of the rotated dot product (q and k as D/2 complex numbers turned by
    e^(i n theta) and e^(i start theta); the real part of q conj(k)), pooled
    by explicit loops; and with every document starting at the query
    position they reduce to the unrotated scores of the stored keys."""
    rng = np.random.default_rng(seed)
    G, D, bs, ss, base = 2, 16, 8, 4, 500.0
    T = 45
    nb = -(-T // bs)
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    starts = np.repeat([0.0, 16.0, 24.0, 40.0], 2)[:nb]  # documents of 2 blocks
    n = 77
    r = O.decode_step_bh(q, K, V, np.zeros(T), T, bs, ss, 2, 2, set(), [], 1, 1 / math.sqrt(D),
                         rope=dict(q_pos=n, block_start=starts, base=base))
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    qc = (q[:, :D // 2] + 1j * q[:, D // 2:]) * np.exp(1j * n * theta)
    want = np.full(nb, -np.inf)
    for i in range(nb):
        for lo in range(i * bs, min(T, (i + 1) * bs), ss):
            hi = min(lo + ss, T, (i + 1) * bs)
            vals = []
            for t in range(lo, hi):
                kc = (K[t, :D // 2] + 1j * K[t, D // 2:]) * np.exp(1j * starts[i] * theta)
                vals.append(np.mean(np.real(qc @ np.conj(kc))) / math.sqrt(D))
            want[i] = max(want[i], float(np.mean(vals)))
    assert np.abs(r["S_q"] - want).max() <= 1e-12, np.abs(r["S_q"] - want).max()
    r0 = O.decode_step_bh(q, K, V, np.zeros(T), T, bs, ss, 2, 2, set(), [], 1, 1 / math.sqrt(D),
                          rope=dict(q_pos=n, block_start=np.full(nb, float(n)), base=base))
    plain = O.pool_block_scores(O.query_token_scores(q, K), T, bs, ss)
    assert np.abs(r0["S_q"] - plain).max() <= 1e-12


def check_index_inputs(O, seed=13):
    """QKV split and eviction head: a hand-built row splits into the blocks
    it was made of; a one-hot weight reads one value dim exactly; the head is
    linear in the weights; and it matches an explicit float64 loop over dims,
    rounded once to float32."""
    Hq, Hkv, D = 4, 2, 3
    row = np.arange((Hq + 2 * Hkv) * D)
    q, k, v = O.split_qkv(row, Hq, Hkv, D)
    assert q[1, 2] == 5 and k[0, 0] == 12 and k[1, 2] == 17 and v[0, 0] == 18 and v[1, 2] == 23
    assert q.shape == (4, 3) and k.shape == (2, 3) and v.shape == (2, 3)
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((50, 8))
    onehot = np.zeros(8)
    onehot[5] = 1.0
    assert np.array_equal(O.eviction_head(V, onehot), V[:, 5].astype(np.float32))
    w1, w2 = rng.standard_normal(8), rng.standard_normal(8)
    e = O.eviction_head(V, w1 + w2).astype(np.float64)
    assert np.abs(e - (O.eviction_head(V, w1).astype(np.float64) + O.eviction_head(V, w2))).max() <= 1e-5
    for t in range(50):
        acc = 0.0
        for d in range(8):
            acc += float(V[t, d]) * float(w1[d])
        assert O.eviction_head(V[t], w1) == np.float32(acc)


def check_prefill(O, seed=14):
    """Prefill over reused documents: against torch's float64 SDPA with an
    explicit causal mask on rotated queries and keys built from the
    complex-number form, and the last prompt query against the decode
    step's dense attention at the same position."""
    rng = np.random.default_rng(seed)
    G, D, bs, base = 2, 16, 4, 1000.0
    T, M = 40, 9
    q_pos0 = T - M
    q = rng.standard_normal((M, G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    nb = -(-T // bs)
    starts = (np.arange(nb) // 2) * 2 * bs * 1.0  # documents of two blocks
    Ow, mw, lw = O.prefill_attention_bh(q, K, V, T, q_pos0, starts, bs, base, 1 / math.sqrt(D))
    theta = base ** (-2.0 * np.arange(D // 2) / D)
    def rot(x, pos):
        c = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos * theta)
        return np.concatenate([c.real, c.imag], axis=-1)
    Kr = np.stack([rot(K[t], starts[t // bs]) for t in range(T)])
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    for g in range(G):
        Qr = np.stack([rot(q[mi, g], q_pos0 + mi) for mi in range(M)])
        mask = np.arange(T)[None, :] <= (q_pos0 + np.arange(M))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(Qr)[None], t(Kr)[None], t(V)[None], attn_mask=torch.tensor(mask)[None], scale=1 / math.sqrt(D))[0]
        assert np.abs(Ow[:, g] - ref.numpy()).max() <= 1e-12
        s = t(Qr) @ t(Kr).T / math.sqrt(D)
        lse = torch.logsumexp(s.masked_fill(~torch.tensor(mask), -math.inf), dim=1).numpy()
        assert np.abs(mw[:, g] + np.log(lw[:, g]) - lse).max() <= 1e-12
    r = O.decode_step_bh(q[M - 1], K, V, np.zeros(T), T, bs, bs, 0, nb, set(), [], 1, 1 / math.sqrt(D),
                         select_all=True, rope=dict(q_pos=T - 1, block_start=starts, base=base))
    assert np.abs(r["O"] - Ow[M - 1]).max() <= 1e-12 and np.abs(r["m"] - mw[M - 1]).max() <= 1e-12


# ---------------------------------------------------------------------------
# rotary embedding and the deferred (lazy) rotation
# ---------------------------------------------------------------------------

def check_rope_complex(O, seed=8):
    """Rotate-half RoPE is multiplication of z_i = x_i + i x_{i+D/2} by
    exp(i pos theta_i); theta_0 = 1 and consecutive thetas have the constant
    ratio base^(-2/D)."""
    rng = np.random.default_rng(seed)
    for D, base in [(8, 10000.0), (64, 500000.0), (128, 500000.0)]:
        th = O.rope_inv_freq(D, base)
        assert th[0] == 1.0 and len(th) == D // 2
        assert np.abs(th[1:] / th[:-1] - base ** (-2.0 / D)).max() <= 1e-14
        for pos in [0, 1, 7, 4096, 32768]:
            x = rng.standard_normal(D)
            z = (x[: D // 2] + 1j * x[D // 2:]) * np.exp(1j * pos * th)
            ref = np.concatenate([z.real, z.imag])
            assert np.abs(O.rope_rotate(x, pos, base) - ref).max() <= 1e-12


def check_rope_identities(O, seed=9):
    rng = np.random.default_rng(seed)
    D, base = 128, 500000.0
    x = rng.standard_normal((5, D))
    assert np.array_equal(O.rope_rotate(x, 0, base), x), "Rot(0) = I"
    for a, b in [(3, 4), (4096, 28672), (12345, 20423)]:
        lhs = O.rope_rotate(O.rope_rotate(x, b, base), a, base)
        assert np.abs(lhs - O.rope_rotate(x, a + b, base)).max() <= 1e-10, "Rot(a) Rot(b) = Rot(a+b)"
        assert np.abs(np.linalg.norm(O.rope_rotate(x, a, base), axis=1) - np.linalg.norm(x, axis=1)).max() <= 1e-12
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        lhs = O.rope_rotate(q, a + b, base) @ O.rope_rotate(k, b, base)
        rhs = O.rope_rotate(q, a, base) @ k
        assert abs(lhs - rhs) <= 1e-10, "score depends on the offset only"


# ---------------------------------------------------------------------------
# whole step (one (b, h)), special cases
# ---------------------------------------------------------------------------

def check_step_dense_equivalence(O, seed=10):
    """With k >= nb the step is plain softmax attention over every token."""
    rng = np.random.default_rng(seed)
    G, D, T, bs, ss = 4, 32, 301, 16, 4
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    e = rng.standard_normal(T)
    nb = -(-T // bs)
    for k_e, k_q in [(nb, 0), (0, nb), (7, nb - 7), (nb, nb)]:
        r = O.decode_step_bh(q, K, V, e, T, bs, ss, k_e, k_q, set(), [], 5, 1 / math.sqrt(D))
        assert r["sel"] == list(range(nb))
        assert np.abs(r["O"] - _sdpa(q, K, V, 1 / math.sqrt(D))).max() <= 1e-12
        Om, mm, lm = O.merge_partials(r["part_o"][0], r["part_m"][0], r["part_l"][0])
        assert np.abs(Om - r["O"][0]).max() <= 1e-12


def check_step_sparse_subset(O, seed=11):
    """With k < nb the output is exactly SDPA over the selected blocks'
    tokens, and the swap lists are the differences to the previous set."""
    rng = np.random.default_rng(seed)
    G, D, T, bs, ss = 2, 16, 150, 16, 4
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    e = rng.standard_normal(T)
    r = O.decode_step_bh(q, K, V, e, T, bs, ss, 2, 3, set(), [0, 9], 3, 0.25)
    assert len(r["sel"]) == 5
    toks = np.concatenate([np.arange(i * bs, min(i * bs + bs, T)) for i in r["sel"]])
    assert np.abs(r["O"] - _sdpa(q, K[toks], V[toks], 0.25)).max() <= 1e-12
    assert set(r["load"]) == set(r["sel"]) - {0, 9} and set(r["evict"]) == {0, 9} - set(r["sel"])


def check_step_lazy_rope(O, seed=12):
    """Deferred RoPE: materialised rotated keys and the lazy relative
    rotation of the query (once per document) give the same attention."""
    rng = np.random.default_rng(seed)
    G, D, bs, base = 4, 64, 8, 500000.0
    doc_blocks = 3
    T = bs * doc_blocks * 4
    nb = T // bs
    starts = (np.arange(nb) // doc_blocks) * doc_blocks * bs
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    n = T
    r = O.decode_step_bh(q, K, V, np.zeros(T), T, bs, bs, 0, nb, set(), [], 4, 1 / math.sqrt(D),
                         select_all=True, rope=dict(q_pos=n, block_start=starts, base=base))
    # lazy route: scores of block i use Rot(n - start_i) q against stored keys
    s = np.empty((G, T))
    for i in range(nb):
        qr = O.rope_rotate(q, n - starts[i], base)
        s[:, i * bs:(i + 1) * bs] = qr @ K[i * bs:(i + 1) * bs].T / math.sqrt(D)
    lse = torch.logsumexp(torch.tensor(s), dim=1).numpy()
    p = np.exp(s - lse[:, None])
    assert np.abs(r["O"] - p @ V).max() <= 1e-10
    assert np.abs(r["m"] + np.log(r["l"]) - lse).max() <= 1e-10
    # no rotation (position 0, documents at 0) reduces to plain attention
    r0 = O.decode_step_bh(q, K, V, np.zeros(T), T, bs, bs, 0, nb, set(), [], 4, 1 / math.sqrt(D),
                          select_all=True, rope=dict(q_pos=0, block_start=np.zeros(nb), base=base))
    assert np.abs(r0["O"] - _sdpa(q, K, V, 1 / math.sqrt(D))).max() <= 1e-12


def check_bf16_decode(O):
    """bf16 bit patterns decode to their exact values."""
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4000, 0x3F00, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [0.0, 1.0, -1.0, 2.0, 0.5, 3.3895313892515355e38, 2.0 ** -133, 3.140625]
    assert O.bf16_to_f64(bits).tolist() == want


def check_attend_blocks(O, seed=15):
    """Attention over an arbitrary block list (not a selection: any order,
    the ragged tail block included, more splits than blocks) is SDPA over
    those blocks' tokens, each split partial is SDPA over its chunk's
    tokens (empty chunks exactly (0, -inf, 0)), and each query row's block
    masses sum to 1."""
    rng = np.random.default_rng(seed)
    G, D, T, bs = 4, 16, 181, 16
    q, K, V = rng.standard_normal((G, D)), rng.standard_normal((T, D)), rng.standard_normal((T, D))
    blocks = [11, 3, 0, 7]  # block 11 holds the 5 tokens 176..180
    P = 6
    r = O.attend_blocks(q, K, V, T, bs, blocks, P, 0.3)
    toks = np.concatenate([np.arange(i * bs, min(i * bs + bs, T)) for i in blocks])
    assert len(toks) == 3 * bs + 5
    assert np.abs(r["O"] - _sdpa(q, K[toks], V[toks], 0.3)).max() <= 1e-12
    ref_lse = torch.logsumexp(torch.tensor(q @ K[toks].T * 0.3), dim=1).numpy()
    assert np.abs(r["m"] + np.log(r["l"]) - ref_lse).max() <= 1e-12
    for p_, i in enumerate(blocks):  # one block per chunk, then empty chunks
        t_ = np.arange(i * bs, min(i * bs + bs, T))
        assert np.abs(r["part_o"][:, p_] - _sdpa(q, K[t_], V[t_], 0.3)).max() <= 1e-12
    assert np.all(r["part_o"][:, len(blocks):] == 0) and np.all(np.isneginf(r["part_m"][:, len(blocks):]))
    assert np.all(r["part_l"][:, len(blocks):] == 0)
    assert np.abs(r["mass"].sum(axis=1) - 1).max() <= 1e-12
    # materialise without RoPE hands back the inputs (first T keys)
    qt, Kt = O.materialise(q, np.vstack([K, K[:3]]), T, bs)
    assert qt is q and Kt.shape == (T, D) and np.array_equal(Kt, K)


def check_share_chunks(O, seed=16):
    """The share layout, worked by hand: 5 eviction and 3 query blocks over
    2 splits give eviction blocks [0, 2) and [2, 5) of the eviction list
    and query blocks [0, 1) and [1, 3) of the query list; one block over 4
    splits lands in the last.  attend_blocks over an explicit partition:
    each partial is SDPA over its chunk's tokens, the merged result is the
    unsplit one, and a list that is not a partition is refused."""
    assert O.share_chunks([1, 4, 6, 9, 12], [2, 3, 20], 2) == [[1, 4, 2], [6, 9, 12, 3, 20]]
    assert O.share_chunks([5], [], 4) == [[], [], [], [5]]
    assert O.share_chunks([], [7, 8, 9], 3) == [[7], [8], [9]]
    rng = np.random.default_rng(seed)
    G, D, T, bs = 2, 8, 150, 16
    q, K, V = rng.standard_normal((G, D)), rng.standard_normal((T, D)), rng.standard_normal((T, D))
    e, qq = [0, 2, 5, 9], [1, 7]  # block 9 holds the 6 tokens 144..149
    blocks = sorted(e + qq)
    chunks = O.share_chunks(e, qq, 3)
    assert chunks == [[0], [2, 1], [5, 9, 7]]
    r = O.attend_blocks(q, K, V, T, bs, blocks, 3, 0.4, chunks=chunks)
    for p_, c in enumerate(chunks):
        t_ = np.concatenate([np.arange(i * bs, min(i * bs + bs, T)) for i in c])
        assert np.abs(r["part_o"][:, p_] - _sdpa(q, K[t_], V[t_], 0.4)).max() <= 1e-12
    toks = np.concatenate([np.arange(i * bs, min(i * bs + bs, T)) for i in blocks])
    for g in range(G):  # the share partials merge to attention over every listed token
        Om, mm, lm = O.merge_partials(r["part_o"][g], r["part_m"][g], r["part_l"][g])
        assert np.abs(Om - _sdpa(q[g:g + 1], K[toks], V[toks], 0.4)[0]).max() <= 1e-12
    try:
        O.attend_blocks(q, K, V, T, bs, blocks, 2, 0.4, chunks=[[0, 1], [2, 5]])
    except AssertionError:
        pass
    else:
        raise AssertionError("a partial cover was accepted")


ALL_CHECKS = [
    check_attend_vs_sdpa, check_merge_vs_sdpa, check_split_chunks,
    check_pool_closed_form, check_pool_linearity, check_eviction_pre_exp,
    check_select_bruteforce, check_select_sizes, check_trajectory_invariants,
    check_swap_lists, check_place_blocks, check_buffer_retrieve, check_rope_complex, check_rope_identities,
    check_softmax_block_mass, check_alibi, check_rope_scores, check_index_inputs, check_prefill, check_step_dense_equivalence, check_step_sparse_subset, check_step_lazy_rope,
    check_attend_blocks, check_share_chunks, check_bf16_decode,
]
