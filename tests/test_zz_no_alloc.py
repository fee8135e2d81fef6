"""nosa_select_decode_noalloc against nosa_select_decode.

The no-allocation entry point runs the same fused select + decode launch
with its split partials and arrival counters in the library's static
scratch.  Through the C-ABI, on the same inputs and state, its selections,
eviction bitmaps, swap lists and outputs must equal those of
nosa_select_decode bit for bit, over two calls in a row (several steps
each), the second with a smaller input.  (That a call whose partials do not
fit the scratch is refused before any launch is a host check, tested in
test_abi.py.)
"""

from __future__ import annotations

import sys

import pytest
import torch

from block_sparse_kv_score_amd import nosa, synth
from block_sparse_kv_score_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu


def _noalloc_step(s, t: int):
    """Step t of session s with the decode launch through the no-allocation
    entry point (the append + score launch as usual)."""
    w = s.w
    s.use_buffers(t)
    s.append_score(t)
    out = s.ev_bufs[1] if s.evicted is s.ev_bufs[0] else s.ev_bufs[0]
    nosa.nosa_select_decode_noalloc(s.dims, s.kv, s.q(t), s.score_q, s.score_e, s.seq_lens, w.k_e, w.k_q, s.evicted,
                                    out, s.sel, s.sel_count, s.prev, s.prev_count, s.load, s.load_count, s.evict,
                                    s.evict_count, s.P, w.sm_scale, s.o, s.m, s.l)
    s.evicted = out
    s.step_index = t
    s.n_steps += 1


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int32) if x.dtype == torch.float32 else x


def _compare(a, b, t: int):
    w = a.w
    for n in ("sel_count", "evicted", "load_count", "evict_count", "o", "m", "l", "seq_lens"):
        assert torch.equal(_bits(getattr(a, n)), _bits(getattr(b, n))), (w.name, n, t)
    for n in ("sel", "load", "evict"):
        cnt = getattr(a, "sel_count" if n == "sel" else n + "_count")
        x, y = getattr(a, n), getattr(b, n)
        for i in range(w.B):
            for j in range(w.Hkv):
                k = int(cnt[i, j])
                assert torch.equal(x[i, j, :k], y[i, j, :k]), (w.name, n, t, i, j)


CALLS = [
    # the larger call first: 2 x 2 pairs, 3 splits (partials and counters in use)
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 3),
    # then a smaller one: 1 pair, 2 splits
    ("tiny_nosa", dict(B=1, Hq=4, Hkv=1, T0=1500), 2),
]


def test_noalloc_equals_select_decode_two_calls():
    from block_sparse_kv_score_amd.step import DecodeSession
    for name, scale, splits in CALLS:
        w = WORKLOADS[name].scaled(**scale)
        print(f"\n[case] noalloc vs select_decode {name} {scale} P={splits}", flush=True)
        sys.stdout.flush()
        inp = synth.generate(w, 60)
        a = DecodeSession(w, inp, splits=splits, select_decode=True)
        b = DecodeSession(w, inp, splits=splits, select_decode=True)
        assert a.select_decode_ok
        for t in range(1, 5):
            a.step(t)
            _noalloc_step(b, t)
            torch.cuda.synchronize()
            assert int(a.err.item()) == 0 and int(b.err.item()) == 0
            _compare(a, b, t)

