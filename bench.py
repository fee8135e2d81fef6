"""Benchmark of one NOSA-style block-sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--splits P]

A step is the whole hot path over one batch: append -> score -> select ->
swap_diff -> sparse_decode (split-K) -> combine, for every sequence of the
batch, on synthetic inputs resident in HBM before timing starts.  By default
the step is two launches: append + score (nosa_append_score) and select +
swap_diff + decode + combine (nosa_select_decode); --unfused times the six
separate calls.  The
default workload is the Llama-3-8B-shaped layer at 32K context.

Timing (HIP events on the stream the kernels run on):
  * cold: before every step a 1 GiB buffer is read so L2 and the Infinity
    Cache hold none of the step's data; the step is bracketed by events;
  * per-kernel: a second cold pass with an event between every launch;
  * warm: back-to-back steps, for context.
`value` is B / (cold step time): decode tokens per second.  HBM bandwidth
counts algorithmic bytes: K and V of the tokens present in the selected
blocks plus the block summaries (fp32 mean keys and logits) that scoring
streams.  The CPU baseline times the float64 oracle on a bounded sample of
(b, h) pairs of the same workload and scales it to the whole batch.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0
PEAK_HOST_LINK_GBPS = 64.0  # PCIe 5.0 x16, one direction
PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense bf16 matrix cores
METRIC = "sparse decode attn tokens/s + achieved HBM GB/s (% peak), 8B shape @32K"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_llama3_8b_32k.json")
CSRC = os.path.join(ROOT, "block_sparse_kv_score_amd", "csrc")
# the sources the decode kernel (and its select variant) is built from
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("nosa_decode.hip", "nosa_select_impl.hpp", "nosa_device.hpp")]
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic_lazy_prefill_33k.json")
# the sources the prefill kernel is built from
PREFILL_SRCS = [os.path.join(CSRC, f) for f in ("nosa_prefill.hip", "nosa_device.hpp")]


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 5; 60 with --buffer-slots, so the buffer has filled)")
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the bandwidth probes (practical ceilings)")
    ap.add_argument("--graph", action="store_true",
                    help="time the cold steps as HIP graph replays (the plain HBM-tier step; other passes eager)")
    ap.add_argument("--unfused", action="store_true", help="time the six separate entry points")
    ap.add_argument("--separate-select", action="store_true",
                    help="nosa_select_swap + nosa_sparse_decode_combine where nosa_select_decode would run")
    ap.add_argument("--offload", action="store_true",
                    help="host tier: pages in pinned host memory, resident slots in HBM, nosa_retrieve per step")
    ap.add_argument("--buffer-slots", type=int, default=None,
                    help="host tier with this many HBM slots per (b, h) (>= the selection budget): pages stay "
                         "buffered after leaving the selection, bucketed-LRU eviction (nosa_retrieve_buffered)")
    ap.add_argument("--bucket-width", type=int, default=1, help="steps per recency bucket of the buffer")
    ap.add_argument("--mass", action="store_true",
                    help="decode with the softmax score step (nosa_sparse_decode_mass): block masses per head")
    ap.add_argument("--alibi", action="store_true",
                    help="decode with ALiBi biases (nosa_sparse_decode_alibi), slopes 2^(-8(j+1)/Hq)")
    ap.add_argument("--qkv", action="store_true",
                    help="the step's input is each sequence's fused projection row: nosa_append_score_qkv "
                         "(QKV split + eviction head + pooling + scoring in one launch)")
    ap.add_argument("--probe-matrix", action="store_true",
                    help="after the warm-up, run the page-gather probe matrix over the current selection and "
                         "print it as one JSON line (no step timing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with one plain 1 GiB device copy, a known-size kernel for counter calibration")
    return ap.parse_args(argv)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, sel, sel_count, T):
    """K+V bytes of the tokens present in the selected blocks, and the
    summary bytes scoring streams (valid sub-blocks), for one step."""
    import numpy as np
    nb = -(-T // w.bs)
    tail = T - (nb - 1) * w.bs
    n_tok = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            s = sel[b, h, :sel_count[b, h]]
            n_tok += len(s) * w.bs - int(np.count_nonzero(s == nb - 1)) * (w.bs - tail)
    kv = n_tok * w.D * 2 * 2
    n_sub = (nb - 1) * w.nsub + -(-tail // w.ss)
    summ = 0 if w.select_all else w.B * w.Hkv * n_sub * (w.D * 4 + 4)
    return kv, summ


def host_threads() -> tuple[int, int]:
    """Host cores this process may run on, and the BLAS threads NumPy uses."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    return cores, int(threads)


def cpu_baseline(w, inp, budget_s: float):
    """The oracle as it stands, on (b, h) pairs of decode step 1 until the
    time budget is spent; scaled to the whole batch."""
    import numpy as np
    import oracle
    from block_sparse_kv_score_amd import synth
    cores, threads = host_threads()
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    rng = np.random.default_rng(0)
    rng.shuffle(pairs)
    t = 1
    T = w.seq_len(t)
    q = inp.q(t)
    done, elapsed = 0, 0.0
    stage = {"score": 0.0, "select": 0.0, "swap": 0.0, "attend": 0.0}
    scale = 1.0 / math.sqrt(w.D)
    for (b, h) in pairs:
        t0 = time.perf_counter()
        K = oracle.bf16_to_f64(inp.K[b, h, :T])
        V = oracle.bf16_to_f64(inp.V[b, h, :T])
        e = inp.e[b, h, :T].astype(np.float64)
        qg = oracle.bf16_to_f64(q[b, h * w.G:(h + 1) * w.G])
        rope = None
        if w.select_all and w.rope_base:
            rope = dict(q_pos=int(inp.q_pos[b]), block_start=synth.block_doc_start(w) * w.bs, base=w.rope_base)
        oracle.decode_step_bh(qg, K, V, e, T, w.bs, w.ss, w.k_e, w.k_q, set(), [], w.splits, scale,
                              select_all=w.select_all, rope=rope)
        elapsed += time.perf_counter() - t0
        if not w.select_all:
            # the same pair again, stage by stage through the oracle's own stage functions
            t1 = time.perf_counter()
            S_q = oracle.pool_block_scores(oracle.query_token_scores(qg, K), T, w.bs, w.ss)
            E = oracle.pool_block_scores(oracle.eviction_token_scores(e), T, w.bs, w.ss)
            t2 = time.perf_counter()
            gamma = oracle.select_blocks(S_q, E, oracle.num_blocks(T, w.bs), w.k_e, w.k_q, set())[2]
            t3 = time.perf_counter()
            oracle.swap_lists([], gamma)
            t4 = time.perf_counter()
            for chunk in oracle.split_chunks(gamma, w.splits):
                toks = oracle.tokens_of_blocks(chunk, T, w.bs)
                oracle.attend(qg, K[toks], V[toks], scale)
            toks = oracle.tokens_of_blocks(gamma, T, w.bs)
            oracle.attend(qg, K[toks], V[toks], scale)
            t5 = time.perf_counter()
            for k_, dt in zip(stage, (t2 - t1, t3 - t2, t4 - t3, t5 - t4)):
                stage[k_] += dt
        done += 1
        if elapsed >= budget_s:
            break
    step_s = elapsed / done * len(pairs)
    out = {"value": w.B / step_s, "unit": "tokens/s", "cores": cores, "blas_threads": threads, "kind": "oracle",
           "sample": f"{done} of {len(pairs)} (b,h) pairs of decode step 1 ({elapsed:.1f} s), "
                     f"scaled to the batch; float64 NumPy on {cores} host cores, BLAS threads = {threads}",
           "sec_per_step": step_s}
    if not w.select_all:
        out["stage_sec_per_step"] = {k_: round(v / done * len(pairs), 4) for k_, v in stage.items()}
    return out


def prefill_flops(w) -> float:
    """Algorithmic FLOPs of one prefill launch: every prompt query of every
    head attends its n + 1 visible keys, 2 D for q.k and 2 D for p.v each."""
    M, p0 = w.prompt, w.T0 - w.prompt
    keys = sum(p0 + m + 1 for m in range(M))
    return 4.0 * w.D * keys * w.Hq * w.B


def prefill_cpu_baseline(w, inp, budget_s: float):
    """The oracle's prefill (as it stands) on single prompt rows of random
    (b, h) pairs until the budget is spent; scaled to the launch."""
    import numpy as np
    import oracle
    from block_sparse_kv_score_amd import synth
    cores, threads = host_threads()
    rng = np.random.default_rng(0)
    qp = synth.prefill_queries(w, inp.seed)
    starts = synth.block_doc_start(w) * w.bs
    p0 = w.T0 - w.prompt
    done, elapsed = 0, 0.0
    while elapsed < budget_s:
        b, h, r = int(rng.integers(w.B)), int(rng.integers(w.Hkv)), int(rng.integers(w.prompt))
        t0 = time.perf_counter()
        K = oracle.bf16_to_f64(inp.K[b, h, :w.T0])
        V = oracle.bf16_to_f64(inp.V[b, h, :w.T0])
        q = oracle.bf16_to_f64(qp[b, r:r + 1, h * w.G:(h + 1) * w.G])
        oracle.prefill_attention_bh(q, K, V, w.T0, p0 + r, starts, w.bs, w.rope_base, w.sm_scale)
        elapsed += time.perf_counter() - t0
        done += 1
    launch_s = elapsed / done * w.prompt * w.B * w.Hkv
    return {"value": w.B * w.prompt / launch_s, "unit": "tokens/s", "cores": cores, "blas_threads": threads,
            "kind": "oracle",
            "sample": f"{done} prompt rows of random (b, h) pairs ({elapsed:.1f} s), scaled to the launch "
                      f"({w.B * w.Hkv * w.prompt} rows); float64 NumPy on {cores} host cores, "
                      f"BLAS threads = {threads}",
            "sec_per_launch": launch_s}


def bench_prefill(args, w) -> int:
    """Prefill over reused documents: K cold launches (1 GiB read before
    each), events around each launch on the launch stream."""
    import numpy as np
    import torch
    from block_sparse_kv_score_amd import synth
    from block_sparse_kv_score_amd.step import DecodeSession
    K, W = args.steps, args.warmup
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.generate(w, args.seed)
    sess = DecodeSession(w, inp, poison=False)
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(W):
        flush_buf.sum()
        sess.prefill_attention()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for k in range(K):
        flush_buf.sum()
        ev[k][0].record(stream)
        sess.prefill_attention()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    assert int(sess.err.cpu()[0]) == 0, "device contract flag raised"
    ms = [a.elapsed_time(b) for a, b in ev]
    t = float(np.median(ms)) / 1e3
    flops = prefill_flops(w)
    tflops = flops / t / 1e12
    kv_bytes = w.B * w.Hkv * w.T0 * 4 * w.D  # every cached K and V byte once
    if args.copy_calibration:  # a plain 1 GiB device copy, to scale memory counters by
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w, inp, args.cpu_seconds)
    traffic = None  # counter bytes per launch, while the kernel is the one they were taken on
    if os.path.exists(PREFILL_TRAFFIC_FILE):
        tr = json.load(open(PREFILL_TRAFFIC_FILE))
        if tr.get("prefill_sources_sha256_16") == source_hash(PREFILL_SRCS) and tr.get("workload") == w.name:
            traffic = tr.get("bytes_per_launch")
    out = {
        "metric": f"prefill tokens/s over reused documents, deferred RoPE ({w.name})",
        "value": round(w.B * w.prompt / t, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "context": w.T0, "prompt": w.prompt, "documents": w.n_docs, "doc_len": w.doc_len,
                   "block": w.bs, "parallelism": "single GPU"},
        "step_ms_p10_p90": [round(float(np.percentile(ms, 10)), 4), round(float(np.percentile(ms, 90)), 4)],
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "nosa_prefill_attention (prefill_rope_kernel)",
                     "algorithmic_flops_per_launch": flops, "avg_launch_us": round(float(np.mean(ms)) * 1e3, 2)},
        "hbm_gbps_kv_once": round(kv_bytes / t / 1e9, 1),
        "cpu_baseline": cpu,
        "seed": args.seed,
    }
    print(json.dumps(out))
    return 0


def practical_ceilings(sess, flush, stream, reps: int = 10) -> dict:
    """Live HBM read rates of the step's two access patterns with nothing
    computed on the data (libnosa's bandwidth probes), timed as the step is:
    after the same cache flush, between events on the step's stream, median
    of `reps`.  The stream read covers the whole K page pool; the page gather
    reads the K and V pages of the current selection (flat tables), with the
    decode's grid.  The stream read runs one workgroup per compute unit (the
    grid that streams fastest here) over the block-summary buffer -- the bytes
    the scoring reads -- and over the whole K page pool."""
    import numpy as np
    import torch
    from block_sparse_kv_score_amd import nosa

    def timed(fn) -> float:
        evs = []
        for _ in range(reps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs])) / 1e3

    out = {}
    pool = sess.k_pages
    n_bytes = pool.numel() * pool.element_size()
    sink = torch.zeros(torch.cuda.get_device_properties(pool.device).multi_processor_count, dtype=torch.int32,
                       device=pool.device)
    summ = sess.k_summary
    s_bytes = summ.numel() * summ.element_size()
    t = timed(lambda: nosa.nosa_probe_stream_read(summ, sink, stream))
    out["stream_read_gbps"] = round(s_bytes / t / 1e9, 1)
    out["stream_read_bytes"] = int(s_bytes)
    t = timed(lambda: nosa.nosa_probe_stream_read(pool, sink, stream))
    out["stream_read_large_gbps"] = round(n_bytes / t / 1e9, 1)
    out["stream_read_large_bytes"] = int(n_bytes)
    if sess.table is not None and sess.cap <= 256:
        sel = sess.sel.long()
        slot = torch.arange(sel.shape[-1], device=sel.device)
        pages = torch.gather(sess.table.long(), 2, sel.clamp(min=0))
        pages = torch.where(slot < sess.sel_count.long()[..., None], pages, torch.full_like(pages, -1))
        pages = pages.reshape(-1, sel.shape[-1]).to(torch.int32).contiguous()
        page_bytes = n_bytes // pool.shape[0]
        g_bytes = int((pages >= 0).sum().item()) * 2 * page_bytes
        g_sink = torch.zeros(pages.shape[0], dtype=torch.int32, device=pool.device)
        t = timed(lambda: nosa.nosa_probe_page_gather(sess.k_pages, sess.v_pages, pages, g_sink, stream))
        out["page_gather_gbps"] = round(g_bytes / t / 1e9, 1)
        out["page_gather_bytes"] = g_bytes
    return out


def probe_matrix(sess, flush, stream, reps: int = 10) -> list:
    """The page-gather probe over the current selection's pages (flat
    tables, selections of at most 256 pages) in several arrangements, to
    tell what bounds the decode's gather: the same pages with 4, 8 and 16
    waves per CU (one K and one V page in flight per wave, so 4, 8 or 16
    page pairs in flight per CU: each pair's list cut into 1, 2 or 4
    lists); each list in ascending page order; and a compact pool (the
    selected pages renumbered 0, 1, ... in list order, then in a random
    order), which reads the same number of pages from a region the size of
    the selection instead of the whole pool.  Median of `reps` cold runs."""
    import numpy as np
    import torch
    from block_sparse_kv_score_amd import nosa

    sel = sess.sel.long()
    if sess.table is None or sel.shape[-1] > 256 or not bool((sess.sel_count == sel.shape[-1]).all()):
        raise SystemExit("--probe-matrix needs a flat table and full selections of at most 256 blocks")
    pages = torch.gather(sess.table.long(), 2, sel).reshape(-1, sel.shape[-1])
    K, V = sess.k_pages, sess.v_pages
    page_bytes = K.shape[1] * K.element_size()

    def gather(plist, label):
        plist = plist.to(torch.int32).contiguous()
        assert int(plist.min()) >= 0 and int(plist.max()) < K.shape[0]
        sink = torch.zeros(plist.shape[0], dtype=torch.int32, device=K.device)
        evs = []
        for _ in range(reps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nosa.nosa_probe_page_gather(K, V, plist, sink, stream)
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in evs])) / 1e3
        nbytes = plist.numel() * 2 * page_bytes
        print(f"[bench] probe {label}: {nbytes / t / 1e9:.1f} GB/s", file=sys.stderr, flush=True)
        return {"arrangement": label, "lists": list(plist.shape), "us": round(t * 1e6, 2),
                "gbps": round(nbytes / t / 1e9, 1), "bytes": int(nbytes)}

    n_pairs, n_sel = pages.shape
    out = []
    for cut in (1, 2, 4):
        if n_sel % cut == 0:
            out.append(gather(pages.reshape(n_pairs * cut, n_sel // cut), f"selection, {4 * cut} waves/CU"))
    out.append(gather(pages.sort(dim=1).values, "selection, each list ascending, 4 waves/CU"))
    compact = torch.arange(pages.numel(), device=K.device).reshape(pages.shape)
    out.append(gather(compact, "compact pool, list order, 4 waves/CU"))
    perm = torch.randperm(pages.numel(), device=K.device, generator=torch.Generator(device=K.device).manual_seed(1))
    out.append(gather(perm.reshape(pages.shape), "compact pool, random order, 4 waves/CU"))
    return out


def main(argv=None) -> int:
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU only (asked for --gpus {args.gpus}); "
              "the per-(b, h) work shards without communication, see the design notes.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from block_sparse_kv_score_amd import synth
    from block_sparse_kv_score_amd.step import DecodeSession
    from block_sparse_kv_score_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.warmup is None:
        args.warmup = 60 if args.buffer_slots is not None else 5
    if w.prompt:
        return bench_prefill(args, w)
    K, W = args.steps, args.warmup
    passes = 3
    if w.append and W + passes * K > w.n_append:
        raise SystemExit(f"at most {w.n_append} appended tokens: lower --steps/--warmup")
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = synth.generate(w, args.seed)
    if args.buffer_slots is not None:
        args.offload = True
    sess = DecodeSession(w, inp, splits=args.splits, poison=False, fused=not args.unfused or args.offload,
                         offload=args.offload, buffer_slots=args.buffer_slots, bucket_width=args.bucket_width,
                         mass=args.mass, alibi=args.alibi, qkv=args.qkv,
                         select_decode=False if args.separate_select else None)
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB

    def flush():
        flush_buf.sum()

    def next_t():
        return sess.step_index + 1 if w.append else 1

    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for _ in range(W):
        flush()
        sess.step(next_t())
    torch.cuda.synchronize()
    if args.probe_matrix:
        print(json.dumps({"workload": w.name, "probe_matrix": probe_matrix(sess, flush, stream)}))
        return 0
    if args.graph:
        if W < 2:
            raise SystemExit("--graph needs at least two warm-up steps")
        sess.capture_graphs()
        torch.cuda.synchronize()

    # pass 1: cold steps, events at the ends only (the headline); with
    # --graph each step is one graph replay, its inputs staged before the flush
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    bytes_kv, bytes_sum = [], []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        if args.graph:
            sess.graph_step(next_t(), replay=False)
        flush()
        ev[k][0].record(stream)
        if args.graph:
            sess.next_graph.replay()
        else:
            sess.step(next_t())
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in ev]
    sel = sess.sel.cpu().numpy()
    cnt = sess.sel_count.cpu().numpy()
    kvb, sb = algorithmic_bytes(w, sel, cnt, w.seq_len(sess.step_index))
    print(f"[bench] cold pass done: median {np.median(step_ms)*1e3:.1f} us", file=sys.stderr, flush=True)

    # pass 2: cold steps with an event between every launch
    fused = sess.fused
    if sess.offload:
        names = ["append_score", "select_swap", "retrieve", "decode_combine"]
    elif fused:
        if w.select_all:
            names = (["append"] if w.append else []) + ["swap_diff", "decode_combine"]
        elif sess.runs_select_decode:
            names = ["append_score", "select_decode"]
        else:
            names = ["append_score", "select_swap", "decode_combine"]
    else:
        names = (["append"] if w.append else []) + ([] if w.select_all else ["score", "select"])
        names += ["swap_diff", "decode", "combine"]
    dec_name = "select_decode" if "select_decode" in names else ("decode_combine" if fused else "decode")
    per = {n: [] for n in names}
    page_bytes = 2 * w.bs * w.D * 2 + w.bs * 4  # K + V + E of one page
    retrieved = []  # bytes the retrieve copied, per step
    misses, selected = 0, 0
    for k in range(K):
        flush()
        t = next_t()
        if sess.offload:  # residency of the tail blocks before this step's retrieve
            tail_before = sess.resident[:, :, (w.seq_len(t) - 1) // w.bs].clone()
        sess.use_buffers(t)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        evs[0].record(stream)
        for j, n in enumerate(names):
            if n == "append":
                sess.append(t)
            elif n == "score":
                sess.score(t)
            elif n == "select":
                sess.select()
            elif n == "select_swap":
                sess.select_swap()
            elif n == "append_score":
                sess.append_score(t)
            elif n == "decode_combine":
                sess.decode_combine(t)
            elif n == "select_decode":
                sess.select_decode(t)
            elif n == "retrieve":
                sess.retrieve()
            elif n == "swap_diff":
                sess.swap_diff()
            elif n == "decode":
                sess.decode(t)
            else:
                sess.combine()
            evs[j + 1].record(stream)
        sess.step_index = t
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            per[n].append(evs[j].elapsed_time(evs[j + 1]))
        if sess.offload:  # loaded pages + the appended tokens of tail pages resident before and after
            tail = sess.resident[:, :, (w.seq_len(t) - 1) // w.bs]
            refreshed = int(((tail_before >= 0) & (tail >= 0)).sum().item())
            loaded = int((sess.miss_count if sess.buffered else sess.load_count).sum().item())
            # a refresh copies the appended token's units: D/8 of K, the
            # 8-token row of V (D units), the 4-token unit of E
            refresh_bytes = 16 * (w.D // 8 + w.D + 1) if w.append else page_bytes
            retrieved.append(page_bytes * loaded + refresh_bytes * refreshed)
            misses += loaded
            selected += int(sess.sel_count.sum().item())
    kernels_us = {n: float(np.mean(v) * 1e3) for n, v in per.items()}

    # pass 3: warm, back to back
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(K):
        sess.step(next_t())
    e1.record(stream)
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K
    assert int(sess.err.cpu()[0]) == 0, "device contract flag raised"

    t_step = float(np.median(step_ms)) / 1e3
    total_bytes = kvb + sb
    gbps = total_bytes / t_step / 1e9
    dec_s = kernels_us[dec_name] / 1e6
    dec_gbps = kvb / dec_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("decode_sources_sha256_16") == source_hash(DECODE_SRCS) and tr.get("workload") == w.name \
                and tr.get("splits") == sess.P and tr.get("entry_point") == dec_name and not sess.mass_on \
                and not sess.alibi_on:
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": {"select_decode": "nosa_select_decode",
                           "decode_combine": ("nosa_sparse_decode_mass" if sess.mass_on
                                              else "nosa_sparse_decode_alibi" if sess.alibi_on
                                              else "nosa_sparse_decode_combine"),
                           "decode": "nosa_sparse_decode"}[dec_name] + " (decode_kernel)",
                "algorithmic_bytes_per_launch": int(kvb), "avg_launch_us": round(kernels_us[dec_name], 2)}
    offload = None
    if sess.offload:
        # the dominant launch is the retrieve, bound by the host link
        rb = float(np.mean(retrieved))
        r_gbps = rb / (kernels_us["retrieve"] / 1e6) / 1e9
        kname = ("nosa_retrieve_buffered (retrieve_buffered_kernel)" if sess.buffered
                 else "nosa_retrieve (retrieve_kernel)")
        roofline = {"bound": "host_link", "achieved": round(r_gbps, 2), "peak": PEAK_HOST_LINK_GBPS, "unit": "GB/s",
                    "frac": round(r_gbps / PEAK_HOST_LINK_GBPS, 4), "traffic": None,
                    "kernel": kname, "algorithmic_bytes_per_launch": int(rb),
                    "avg_launch_us": round(kernels_us["retrieve"], 2)}
        offload = {"host_pool_bytes": int(sess.host_k.numel() * 2 * 2 + sess.host_e.numel() * 4),
                   "resident_pool_bytes": int(sess.k_pages.numel() * 2 * 2 + sess.e_pages.numel() * 4),
                   "resident_slots_per_pair": sess.slots, "retrieve_bytes_per_step": int(rb),
                   "pages_per_pair_per_step": round(rb / page_bytes / (w.B * w.Hkv), 2),
                   "host_link_gbps": round(r_gbps, 2),
                   "buffer_slots": sess.buffer_slots, "softmax_mass": sess.mass_on, "alibi": sess.alibi_on, "qkv_rows": sess.qkv_on, "bucket_width": sess.bucket_width if sess.buffered else None,
                   "selected_pages_resident_before_retrieve": round(1.0 - misses / max(selected, 1), 4),
                   "retrieve_bytes_per_step_p10_p90": [int(np.percentile(retrieved, 10)),
                                                       int(np.percentile(retrieved, 90))]}

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ceiling = None
    if not args.no_ceiling and not sess.offload:
        print("[bench] practical ceilings (bandwidth probes)", file=sys.stderr, flush=True)
        ceiling = practical_ceilings(sess, flush, stream)
        score_name = "append_score" if "append_score" in kernels_us else ("score" if "score" in kernels_us else None)
        if score_name is not None:
            ceiling["scoring_launch_gbps"] = round(sb / (kernels_us[score_name] / 1e6) / 1e9, 1)
            ceiling["scoring_frac_of_stream_read"] = round(ceiling["scoring_launch_gbps"] / ceiling["stream_read_gbps"], 4)
        if "page_gather_gbps" in ceiling:
            ceiling["decode_launch_gbps"] = round(dec_gbps, 1)
            ceiling["decode_frac_of_page_gather"] = round(dec_gbps / ceiling["page_gather_gbps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, args.cpu_seconds)

    out = {
        "metric": (METRIC if w.name == "llama3_8b_32k" else f"sparse decode attn tokens/s ({w.name})")
        + (" [host tier: pages in pinned host memory]" if sess.offload and not sess.buffered else "")
        + (f" [host tier: pages in pinned host memory, {sess.slots}-slot HBM buffer per (b, h)]"
           if sess.buffered else "")
        + (" [with the softmax score step]" if sess.mass_on else "")
        + (" [ALiBi]" if sess.alibi_on else "")
        + (" [input: fused QKV rows + eviction head]" if sess.qkv_on else ""),
        "value": round(w.B / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
                   "context": w.T0, "block": w.bs, "sub_block": w.ss, "k_e": w.k_e, "k_q": w.k_q,
                   "splits": sess.P, "table": w.table, "fused": fused, "select_decode": sess.runs_select_decode, "graph": bool(args.graph), "offload": sess.offload,
                   "buffer_slots": sess.buffer_slots,
                   "parallelism": "single GPU"},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": int(total_bytes),
        "bytes_kv": int(kvb), "bytes_summaries": int(sb),
        "step_ms_p10_p90": [round(float(np.percentile(step_ms, 10)), 4), round(float(np.percentile(step_ms, 90)), 4)],
        "ms_per_step_warm": round(warm_ms, 4),
        "wall_ms_per_step_incl_flush": round(wall_cold / K * 1e3, 4),
        "kernels_us": {k: round(v, 2) for k, v in kernels_us.items()},
        "roofline": roofline,
        "practical_ceiling": ceiling,
        "offload": offload,
        "cpu_baseline": cpu,
        "seed": args.seed,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
