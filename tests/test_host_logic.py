"""Host-side logic of the step and the benchmark (no GPU): option checks
made before any allocation, the generator's extra inputs, and the
benchmark's counting."""

import math
import os
import subprocess
import sys

import numpy as np
import pytest

from block_sparse_kv_score_amd import synth
from block_sparse_kv_score_amd.workloads import TABLE_PACKED_ROPE, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _session(w, **kw):
    from block_sparse_kv_score_amd.step import DecodeSession
    return DecodeSession(w, None, device="cpu", **kw)


@pytest.mark.parametrize("name,kw", [
    ("lazy_rope_32k", dict(mass=True)),                   # mass: no packed RoPE table
    ("tiny_nosa", dict(mass=True, fused=False)),          # mass: fused decode only
    ("tiny_nosa", dict(alibi=True, mass=True)),           # ALiBi without the mass step
    ("lazy_rope_sparse_32k", dict(alibi=True)),           # ALiBi: no packed RoPE table
    ("dense_8b_8k", dict(qkv=True)),                      # QKV rows need an append
    ("tiny_nosa", dict(qkv=True, offload=True)),          # QKV rows: HBM only
    ("tiny_nosa", dict(buffer_slots=16)),                 # a buffer needs the host tier
    ("lazy_rope_32k", dict(offload=True)),                # host tier: selecting, flat / two-level
])
def test_session_rejects_unsupported_combinations(name, kw):
    with pytest.raises(ValueError):
        _session(WORKLOADS[name], **kw)


def test_qkv_rows_are_q_then_k_then_v():
    w = WORKLOADS["tiny_nosa"].scaled(B=2, Hq=4, Hkv=2, T0=70)
    inp = synth.generate(w, 3)
    rows = synth.qkv_rows(w, inp, 2)
    D, pos = w.D, w.T0 + 1
    assert rows.shape == (w.B, (w.Hq + 2 * w.Hkv) * D) and rows.dtype == np.uint16
    for b in range(w.B):
        assert np.array_equal(rows[b, :w.Hq * D].reshape(w.Hq, D), inp.q(2)[b])
        for h in range(w.Hkv):
            k = rows[b, (w.Hq + h) * D:(w.Hq + h + 1) * D]
            v = rows[b, (w.Hq + w.Hkv + h) * D:(w.Hq + w.Hkv + h + 1) * D]
            assert np.array_equal(k, inp.K[b, h, pos]) and np.array_equal(v, inp.V[b, h, pos])


def test_alibi_slopes_and_eviction_weights():
    assert synth.alibi_slopes(8).tolist() == [2.0 ** -k for k in range(1, 9)]
    w = WORKLOADS["tiny_nosa"]
    a, b = synth.eviction_head_weights(w, 0), synth.eviction_head_weights(w, 0)
    assert a.shape == (w.Hkv, w.D) and a.dtype == np.float32 and np.array_equal(a, b)
    assert abs(float(a.std()) * math.sqrt(w.D) - 1.0) < 0.3  # N(0, 1/D)
    assert not np.array_equal(a, synth.eviction_head_weights(w, 1))


def test_prefill_workload_layout():
    w = WORKLOADS["lazy_prefill_33k"]
    assert w.table == TABLE_PACKED_ROPE and not w.append and w.prompt == w.doc_len
    assert w.n_docs * w.doc_len == w.T0 and w.max_blocks == w.n_docs * (w.doc_len // w.bs)
    starts = synth.block_doc_start(w) * w.bs
    assert starts[-1] == w.T0 - w.prompt  # the prompt is the last document
    q = synth.prefill_queries(w.scaled(B=1, prompt=3), 0)
    assert q.shape == (1, 3, w.Hq, w.D) and q.dtype == np.uint16


def test_prefill_flop_count_is_the_causal_sum():
    sys.path.insert(0, ROOT)
    import bench
    w = WORKLOADS["lazy_prefill_33k"].scaled(B=2, Hq=4, Hkv=2, D=64, T0=10, prompt=4)
    # queries at positions 6..9 see 7..10 keys
    assert bench.prefill_flops(w) == 4.0 * 64 * (7 + 8 + 9 + 10) * 4 * 2


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
