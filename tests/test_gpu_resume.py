"""Checkpoint and resume of the cross-step state.

NOSA's eviction part follows a strict policy (NOSA summary, Methodology 1,
dual selection: a block it leaves out never comes back), so the eviction
bitmap is state that every later step depends on, as are the previous
selection (the swap lists are its set differences, Methodology 2), the
lengths, the summaries and the pages holding the appended tokens.  A session
saved after step t and loaded into a fresh session must continue exactly as
the original: the same selections, bitmaps, swap lists, partials, outputs,
summaries and pages, bit for bit, at every later step.
"""

from __future__ import annotations

import sys

import pytest
import torch

from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

OUTPUTS = ["sel_count", "evicted", "load_count", "evict_count", "part_o", "part_m", "part_l", "o", "m", "l",
           "seq_lens", "k_summary", "e_summary", "score_q", "score_e", "k_pages", "v_pages", "e_pages"]

CASES = [
    # (workload, scaling, splits, session options, steps before the save)
    ("tiny_nosa", {}, 2, {}, 5),
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 1, {}, 3),      # fused select + decode
    ("llama3_8b_32k", dict(B=2, Hq=8, Hkv=2, T0=4096 + 61), 3, dict(fused=False), 2),  # six calls
    ("llama31_70b_256k", dict(B=2, Hq=16, Hkv=2, T0=16384 + 100, dir_entries=64), 4, {}, 2),
    ("tiny_nosa", dict(T0=2048 + 50, k_e=2, k_q=6), 2, dict(offload=True), 4),
    ("tiny_nosa", dict(T0=2048 + 50, k_e=2, k_q=6), 1, dict(offload=True, buffer_slots=11, bucket_width=2), 6),
]


def _same(x: torch.Tensor, y: torch.Tensor) -> bool:
    if x.dtype == torch.float32:
        x, y = x.view(torch.int32), y.view(torch.int32)
    return torch.equal(x, y)


def _lists_equal(a, b, name: str) -> bool:
    cnt = getattr(a, name + "_count")
    if not torch.equal(cnt, getattr(b, name + "_count")):
        return False
    x, y = getattr(a, name), getattr(b, name)
    return all(torch.equal(x[i, j, :int(cnt[i, j])], y[i, j, :int(cnt[i, j])])
               for i in range(cnt.shape[0]) for j in range(cnt.shape[1]))


@pytest.mark.parametrize("name,scale,splits,kw,t_save", CASES,
                         ids=[f"{c[0]}-P{c[2]}-{'-'.join(c[3]) or 'fused'}" for c in CASES])
def test_resume_continues_bit_identically(tmp_path, name, scale, splits, kw, t_save):
    from block_sparse_kv_score_amd.step import DecodeSession
    w = WORKLOADS[name].scaled(**scale) if scale else WORKLOADS[name]
    print(f"\n[case] resume {name} {scale} P={splits} {kw} save after step {t_save}", flush=True)
    sys.stdout.flush()
    inp = synth.generate(w, 50)
    a = DecodeSession(w, inp, splits=splits, **kw)
    for t in range(1, t_save + 1):
        a.step(t)
    path = tmp_path / "state.safetensors"
    a.save_state(path)

    b = DecodeSession(w, inp, splits=splits, **kw)
    fresh = DecodeSession(w, inp, splits=splits, **kw)
    b.load_state(path)
    assert b.step_index == t_save and b.seq_lens.tolist() == a.seq_lens.tolist()
    for t in range(t_save + 1, min(w.steps, t_save + 4) + 1):
        a.step(t)
        b.step(t)
        torch.cuda.synchronize()
        assert int(a.err.item()) == 0 and int(b.err.item()) == 0
        for n in OUTPUTS:
            assert _same(getattr(a, n), getattr(b, n)), (n, t)
        for n in ("sel", "load", "evict"):
            assert _lists_equal(a, b, n), (n, t)
        if a.offload:
            for n in ("resident", "slot_owner") + (("last_use", "miss_count") if a.buffered else ()):
                assert torch.equal(getattr(a, n), getattr(b, n)), (n, t)
        assert not b.counters.any().item()
    # the saved state is what carries the run: a session that did not load
    # it starts from the prefill (nothing evicted, the prefill's lengths)
    fresh.step(t_save + 1)
    torch.cuda.synchronize()
    assert fresh.seq_lens.tolist() != a.seq_lens.tolist()
    assert not _same(fresh.e_pages, a.e_pages)


def test_load_rejects_another_workload(tmp_path):
    from block_sparse_kv_score_amd.step import DecodeSession
    w = WORKLOADS["tiny_nosa"]
    print("\n[case] resume: a state of another workload is refused", flush=True)
    a = DecodeSession(w, synth.generate(w, 51))
    a.step(1)
    path = tmp_path / "state.safetensors"
    a.save_state(path)
    other = w.scaled(T0=1500)
    b = DecodeSession(other, synth.generate(other, 51), splits=3)
    with pytest.raises(ValueError):
        b.load_state(path)
