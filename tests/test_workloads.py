"""Workload presets and the input generator (host logic, no GPU)."""

import json
import os

import numpy as np
import pytest

from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.workloads import WORKLOADS, TABLE_TWO_LEVEL

HERE = os.path.dirname(__file__)


def test_workload_shapes_match_their_descriptions():
    w1 = WORKLOADS["tiny_nosa"]
    assert (w1.T0 // w1.bs, w1.G, w1.k) == (32, 4, 8)
    w2 = WORKLOADS["llama3_8b_32k"]
    assert (w2.T0 // w2.bs, w2.G, w2.nsub, w2.k) == (512, 4, 4, 64)
    w3 = WORKLOADS["dense_8b_8k"]
    assert w3.T0 // w3.bs == 128 and w3.k >= w3.T0 // w3.bs and w3.splits == 16
    w4 = WORKLOADS["llama31_70b_256k"]
    assert (w4.T0 // w4.bs, w4.G, w4.nsub, w4.dir_entries) == (2048, 8, 4, 256)
    assert (w4.B * w4.Hkv << w4.blocks_log2) >> w4.seg_log2 <= w4.dir_entries
    w5 = WORKLOADS["lazy_rope_32k"]
    assert w5.n_docs * w5.doc_len == w5.T0 == 32768 and w5.select_all


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], dtype=np.float32)
    got = synth.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6); 1+2^-9 rounds down
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x0000]


def test_generator_is_seeded_and_per_pair():
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hkv=2, Hq=8)
    a, b = synth.generate(w, 0), synth.generate(w, 0)
    assert np.array_equal(a.K, b.K) and np.array_equal(a.e, b.e) and np.array_equal(a.pages, b.pages)
    K11, V11, e11 = synth.tokens_bh(w, 0, 1, 1)
    assert np.array_equal(K11, a.K[1, 1]) and np.array_equal(e11, a.e[1, 1])
    assert not np.array_equal(synth.generate(w, 1).K, a.K)
    assert sorted(a.pages.ravel().tolist()) == list(range(w.num_pages))


def test_heavy_hitter_rows():
    w = WORKLOADS["llama3_8b_32k"].scaled(B=1, Hkv=1, Hq=4, T0=4096)
    K, _, e = synth.tokens_bh(w, 0, 0, 0)
    from oracle import bf16_to_f64
    norms = np.linalg.norm(bf16_to_f64(K), axis=1)
    frac = float(np.mean(norms > 5 * np.sqrt(w.D)))
    assert 0.005 < frac < 0.02, frac
    assert 1.3 < float(np.std(e)) < 1.5  # sigma = sqrt(2)


def test_two_level_and_packed_tables():
    w4 = WORKLOADS["llama31_70b_256k"].scaled(B=2, T0=4096)
    assert w4.table == TABLE_TWO_LEVEL
    directory, segments = synth.two_level_tables(w4, 0)
    pages = synth.logical_pages(w4, 0)
    for b in range(w4.B):
        for h in range(w4.Hkv):
            for i in [0, 5, w4.max_blocks - 1]:
                key = ((b * w4.Hkv + h) << w4.blocks_log2) | i
                seg = directory[key >> w4.seg_log2]
                assert segments[seg, key & ((1 << w4.seg_log2) - 1)] == pages[b, h, i]
    w5 = WORKLOADS["lazy_rope_32k"].scaled(B=2)
    packed = synth.packed_table(w5, 0)
    lp = synth.logical_pages(w5, 0)
    assert np.array_equal(packed & synth.PACK_PAGE_MASK, lp)
    assert np.array_equal((packed >> 20)[0, 0], (np.arange(512) // 64) * 64)
    # each document's blocks stay contiguous in storage, documents move as a whole
    base = synth.page_ids(w5, 0)
    order = synth.doc_order(w5, 0, 1)
    assert np.array_equal(lp[1, 3, 64:128], base[1, 3, order[1] * 64:order[1] * 64 + 64])


def test_golden_rotation_overhead_figure():
    g = json.load(open(os.path.join(HERE, "golden", "lazyattention_rotation_overhead.json")))
    assert round(100 * 3 / (4 * g["M"]), 2) == g["printed_percent"]
