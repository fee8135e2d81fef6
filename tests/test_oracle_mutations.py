"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Every mutant below is a plausible slip -- a dropped term, a wrong sign or
index, a transposed operand, a wrong pooling, a missing state update -- and
is patched into the oracle module for the duration of one check only.
"""

import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

import oracle.nosa_oracle as O  # noqa: E402
import oracle_pins as P  # noqa: E402

_attend = O.attend
_merge = O.merge_partials
_pool = O.pool_block_scores
_select = O.select_blocks
_rotate = O.rope_rotate
_top = O.top_by_score
_swap = O.swap_lists
_place = O.place_blocks
_bucket = O.recency_bucket
_buffer = O.buffer_retrieve
_mass = O.softmax_block_mass
_abias = O.alibi_bias
_aslopes = O.alibi_slopes
_split = O.split_qkv
_ehead = O.eviction_head
_prefill = O.prefill_attention_bh
_qscore = O.query_token_scores
_freq = O.rope_inv_freq


def _attend_no_scale(q, K, V, scale):
    return _attend(q, K, V, 1.0)


def _attend_kv_swapped(q, K, V, scale):
    return _attend(q, V, K, scale)


def _attend_no_max_shift(q, K, V, scale):
    O_, m, l = _attend(q, K, V, scale)
    return O_, np.zeros_like(m), l


def _merge_unweighted(o, m, l):
    return _merge(o, m, np.where(np.asarray(l) > 0, 1.0, 0.0))


def _pool_mean_of_blocks(ts, T, bs, ss):
    return _pool(ts, T, bs, bs)


def _pool_full_subblock_divisor(ts, T, bs, ss):
    nb = O.num_blocks(T, bs)
    out = np.empty(nb)
    for i in range(nb):
        out[i] = max(float(np.sum(ts[r.start:r.stop])) / ss for r in O.subblock_token_ranges(i, T, bs, ss))
    return out


def _qscore_head_max(q, K):
    return np.max(np.stack([(K @ qg) / math.sqrt(q.shape[1]) for qg in q]), axis=0)


def _qscore_no_sqrt(q, K):
    return _qscore(q, K) * math.sqrt(q.shape[1])


def _evict_with_exp(e):
    return np.exp(np.asarray(e, dtype=np.float64))


def _top_ties_high_index(scores, cand, k):
    order = sorted(cand, key=lambda i: (-float(scores[i]), -int(i)))
    return order[:max(0, int(k))]


def _top_ascending(scores, cand, k):
    order = sorted(cand, key=lambda i: (float(scores[i]), int(i)))
    return order[:max(0, int(k))]


def _select_never_evicts(S_q, E, nb, k_e, k_q, evicted):
    ge, gq, g, ev = _select(S_q, E, nb, k_e, k_q, evicted)
    return ge, gq, g, set(evicted)


def _select_overlapping(S_q, E, nb, k_e, k_q, evicted):
    ge, _, _, ev = _select(S_q, E, nb, k_e, k_q, evicted)
    gq = sorted(_top(S_q, range(nb), min(k_q, nb)))
    return ge, gq, sorted(set(ge) | set(gq)), ev


def _select_swapped_scores(S_q, E, nb, k_e, k_q, evicted):
    return _select(E, S_q, nb, k_e, k_q, evicted)


def _swap_reversed(prev, cur):
    a, b = _swap(prev, cur)
    return b, a


def _place_no_drop(owner, drop, load):
    return _place(owner, [], load)


def _place_from_top(owner, drop, load):
    new, placed = _place(list(reversed(owner)), drop, load)
    return list(reversed(new)), placed


def _place_reversed_loads(owner, drop, load):
    return _place(owner, drop, list(reversed(list(load))))


def _bucket_reversed(age, width):
    return O.RECENCY_BUCKETS - 1 - _bucket(age, width)


def _bucket_off_by_one(age, width):
    return min(int(age) // int(width), O.RECENCY_BUCKETS - 1)


def _buffer_no_hit_refresh(owner, last_use, sel, t, width):
    new, lu, misses, dropped, placed = _buffer(owner, last_use, sel, t, width)
    for s, x in enumerate(owner):
        if x >= 0 and x in set(sel):
            lu[s] = last_use[s]
    return new, lu, misses, dropped, placed


def _buffer_high_slot_first(owner, last_use, sel, t, width):
    new, lu, misses, dropped, placed = _buffer(owner[::-1], last_use[::-1], sel, t, width)
    return new[::-1], lu[::-1], misses, dropped, placed


def _mass_unnormalised(q, K, blocks, T, bs, scale):
    toks = O.tokens_of_blocks(blocks, T, bs)
    out = _mass(q, K, blocks, T, bs, scale)
    if len(toks):
        s = (np.asarray(q) @ np.asarray(K)[toks].T) * scale
        out = out * np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)
    return out


def _mass_blocks_reversed(q, K, blocks, T, bs, scale):
    return _mass(q, K, blocks, T, bs, scale)[:, ::-1]


def _mass_no_scale(q, K, blocks, T, bs, scale):
    return _mass(q, K, blocks, T, bs, 1.0)


def _alibi_sign(slopes, n, positions):
    return -_abias(slopes, n, positions)


def _alibi_from_origin(slopes, n, positions):
    return _abias(slopes, 0, positions)  # slope * position: the same softmax, another row max


def _alibi_slopes_reversed(H):
    return _aslopes(H)[::-1].copy()


def _rotate_none(x, pos, base):
    return np.asarray(x, dtype=np.float64)


def _split_kv_swapped(row, Hq, Hkv, D):
    q, k, v = _split(row, Hq, Hkv, D)
    return q, v, k


def _ehead_on_exp(v, w):
    return _ehead(np.exp(np.asarray(v, dtype=np.float64)), w)


def _prefill_not_causal(q, K, V, T, q_pos0, block_start, bs, base, scale):
    # every prompt query placed at the last position: it sees the whole prompt
    return _prefill(q, K, V, T, T - 1, block_start, bs, base, scale)


def _rotate_sign(x, pos, base):
    return _rotate(x, -np.asarray(pos), base)


def _rotate_pairs_adjacent(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * _freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


def _freq_wrong_exponent(D, base):
    return np.power(float(base), -(np.arange(D // 2, dtype=np.float64)) / D)


MUTANTS = [
    ("attend", _attend_no_scale, P.check_attend_vs_sdpa),
    ("attend", _attend_kv_swapped, P.check_attend_vs_sdpa),
    ("attend", _attend_no_max_shift, P.check_attend_vs_sdpa),
    ("merge_partials", _merge_unweighted, P.check_merge_vs_sdpa),
    ("pool_block_scores", _pool_mean_of_blocks, P.check_pool_closed_form),
    ("pool_block_scores", _pool_full_subblock_divisor, P.check_pool_closed_form),
    ("query_token_scores", _qscore_head_max, P.check_pool_closed_form),
    ("query_token_scores", _qscore_no_sqrt, P.check_pool_linearity),
    ("eviction_token_scores", _evict_with_exp, P.check_eviction_pre_exp),
    ("top_by_score", _top_ascending, P.check_select_bruteforce),
    ("select_blocks", _select_never_evicts, P.check_trajectory_invariants),
    ("select_blocks", _select_overlapping, P.check_select_sizes),
    ("select_blocks", _select_swapped_scores, P.check_select_bruteforce),
    ("swap_lists", _swap_reversed, P.check_swap_lists),
    ("place_blocks", _place_no_drop, P.check_place_blocks),
    ("place_blocks", _place_from_top, P.check_place_blocks),
    ("place_blocks", _place_reversed_loads, P.check_place_blocks),
    ("recency_bucket", _bucket_reversed, P.check_buffer_retrieve),
    ("recency_bucket", _bucket_off_by_one, P.check_buffer_retrieve),
    ("buffer_retrieve", _buffer_no_hit_refresh, P.check_buffer_retrieve),
    ("buffer_retrieve", _buffer_high_slot_first, P.check_buffer_retrieve),
    ("softmax_block_mass", _mass_unnormalised, P.check_softmax_block_mass),
    ("softmax_block_mass", _mass_blocks_reversed, P.check_softmax_block_mass),
    ("softmax_block_mass", _mass_no_scale, P.check_softmax_block_mass),
    ("alibi_bias", _alibi_sign, P.check_alibi),
    ("alibi_bias", _alibi_from_origin, P.check_alibi),
    ("alibi_slopes", _alibi_slopes_reversed, P.check_alibi),
    ("rope_rotate", _rotate_none, P.check_rope_scores),
    ("split_qkv", _split_kv_swapped, P.check_index_inputs),
    ("eviction_head", _ehead_on_exp, P.check_index_inputs),
    ("prefill_attention_bh", _prefill_not_causal, P.check_prefill),
    ("rope_rotate", _rotate_sign, P.check_rope_complex),
    ("rope_rotate", _rotate_pairs_adjacent, P.check_rope_complex),
    ("rope_inv_freq", _freq_wrong_exponent, P.check_rope_complex),
]


@pytest.mark.parametrize("attr,mutant,check", MUTANTS, ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, check):
    monkeypatch.setattr(O, attr, mutant)
    with pytest.raises(AssertionError):
        check(O)


def test_tie_order_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(O, "top_by_score", _top_ties_high_index)
    with pytest.raises(AssertionError):
        P.check_select_bruteforce(O, seed=40, ties=True)
