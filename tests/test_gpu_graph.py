"""The decode step replayed from HIP graphs gives the eager step's bits.

Each graph is replayed several times, with eager work (input staging,
synchronisations, comparisons, and eager steps of the same session) between
the replays, and every step is checked against an eager session over the
same inputs: selections, bitmaps, outputs, lengths, summaries, scores and
pages."""

from __future__ import annotations

import pytest
import torch

from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.step import DecodeSession
from block_sparse_kv_score_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny_nosa", {}, None, 1),                                                     # select+decode, 2 splits
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1, 1),                  # speculative first tile
    ("dense_8b_8k", dict(B=2, Hq=8, Hkv=2, T0=1000), 16, 1),                        # select+swap, decode+combine
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), None, 1),  # two-level
    ("lazy_rope_32k", dict(B=2, Hq=8, Hkv=2, T0=8 * 512, doc_len=512), None, 2),    # every block, deferred RoPE
]

STATE = ["sel", "sel_count", "evicted", "o", "m", "l", "seq_lens", "k_summary", "e_summary", "score_q",
         "score_e", "k_pages", "v_pages", "e_pages", "part_m", "part_l"]


@pytest.mark.parametrize("name,scale,splits,eager_first", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, scale, splits, eager_first):
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    print(f"\n[case] graph replays vs eager {name} {scale} P={splits}", flush=True)
    inp = synth.generate(w, 21)
    a = DecodeSession(w, inp, splits=splits)
    g = DecodeSession(w, inp, splits=splits)
    steps = 8
    for t in range(1, eager_first + 1):
        tt = t if w.append else 1
        a.step(tt)
        g.step(tt)
    g.capture_graphs()
    for i, t in enumerate(range(eager_first + 1, eager_first + 1 + steps)):
        tt = t if w.append else 1
        a.step(tt)
        if i in (2, 4, 5):  # eager steps between replays: the graphs stay in step with the buffers
            g.step(tt)
        else:
            g.graph_step(tt)
        torch.cuda.synchronize()
        for n in STATE:
            x, y = getattr(a, n), getattr(g, n)
            if n == "sel":
                for b in range(w.B):
                    for h in range(w.Hkv):
                        k = int(a.sel_count[b, h])
                        assert torch.equal(x[b, h, :k], y[b, h, :k]), (n, t, b, h)
                continue
            assert torch.equal(x, y) or (x.is_floating_point() and torch.equal(x.isnan(), y.isnan())
                                         and torch.equal(x.nan_to_num(), y.nan_to_num())), (n, t)
        assert int(g.err.item()) == 0
