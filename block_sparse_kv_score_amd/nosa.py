"""ctypes binding of libnosa (include/nosa.h), one Python function per C
entry point, same names.  Argument marshalling only: every function checks
that tensors live on the GPU with the expected dtype and contiguity, turns
them into device pointers and calls the library on the current (or given)
HIP stream.  There is no fallback: if libnosa.so is missing, every call
raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnosa.so")

NOSA_OK = 0
NOSA_ERR_ARG = -1
NOSA_ERR_UNSUPPORTED = -2
NOSA_ERR_HIP = -3
NOSA_ERR_SCRATCH = -4

NOSA_TABLE_FLAT = 0
NOSA_TABLE_TWO_LEVEL = 1
NOSA_TABLE_PACKED_ROPE = 2
NOSA_PACK_PAGE_BITS = 20

ENTRY_POINTS = [
    "nosa_prefill_pages",
    "nosa_build_summaries",
    "nosa_append",
    "nosa_score_blocks",
    "nosa_select",
    "nosa_select_swap",
    "nosa_append_score",
    "nosa_swap_diff",
    "nosa_sparse_decode",
    "nosa_sparse_decode_combine",
    "nosa_select_decode",
    "nosa_select_decode_noalloc",
    "nosa_append_score_qkv",
    "nosa_prefill_attention",
    "nosa_sparse_decode_mass",
    "nosa_sparse_decode_alibi",
    "nosa_combine",
    "nosa_retrieve",
    "nosa_retrieve_buffered",
    "nosa_host_device_pointer",
    "nosa_probe_stream_read",
    "nosa_probe_page_gather",
    "nosa_status_string",
]


class NosaError(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name} failed: {status_string(status)} ({status})")
        self.status = status


class nosa_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("sub_block", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
    ]


class nosa_kv(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("e_pages", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("kind", ctypes.c_int32),
        ("dir_entries", ctypes.c_int32),
        ("table", ctypes.c_void_p),
        ("directory", ctypes.c_void_p),
        ("segments", ctypes.c_void_p),
        ("num_segments", ctypes.c_int64),
        ("seg_log2", ctypes.c_int32),
        ("blocks_log2", ctypes.c_int32),
        ("packed", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("rope_base", ctypes.c_float),
        ("err_flags", ctypes.c_void_p),
    ]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_DIMS = ctypes.POINTER(nosa_dims)
_KV = ctypes.POINTER(nosa_kv)

_SIGNATURES = {
    "nosa_prefill_pages": [_DIMS, _KV, _P, _P, _P, _I32, _P, _P],
    "nosa_build_summaries": [_DIMS, _KV, _P, _P, _P, _P],
    "nosa_append": [_DIMS, _KV, _P, _P, _P, _P, _P, _P, _P],
    "nosa_score_blocks": [_DIMS, _P, _P, _P, _P, _P, _P, _P],
    "nosa_select": [_DIMS, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _P],
    "nosa_select_swap": [_DIMS, _P, _P, _P, _I32, _I32, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_append_score": [_DIMS, _KV, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_swap_diff": [_DIMS, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_sparse_decode": [_DIMS, _P, _KV, _P, _P, _I32, _P, _I32, _F32, _P, _P, _P, _P],
    "nosa_sparse_decode_combine": [_DIMS, _P, _KV, _P, _P, _I32, _P, _I32, _F32, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_select_decode": [_DIMS, _KV, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P,
                           _I32, _F32, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_select_decode_noalloc": [_DIMS, _KV, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                   _P, _P, _I32, _F32, _P, _P, _P, _P],
    "nosa_sparse_decode_mass": [_DIMS, _P, _KV, _P, _P, _I32, _P, _I32, _F32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P],
    "nosa_sparse_decode_alibi": [_DIMS, _P, _KV, _P, _P, _I32, _P, _I32, _F32, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P],
    "nosa_append_score_qkv": [_DIMS, _KV, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "nosa_prefill_attention": [_DIMS, _KV, _P, _I32, _P, _P, _F32, _P, _P, _P, _P],
    "nosa_combine": [_DIMS, _I32, _P, _P, _P, _P, _P, _P, _P],
    "nosa_retrieve": [_DIMS, _KV, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P],
    "nosa_retrieve_buffered": [_DIMS, _KV, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P],
    "nosa_host_device_pointer": [_P, ctypes.POINTER(ctypes.c_void_p)],
    "nosa_probe_stream_read": [_P, ctypes.c_int64, _P, _I32, _P],
    "nosa_probe_page_gather": [_P, _P, ctypes.c_int64, ctypes.c_int64, _P, _I32, _I32, _P, _P],
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_kv_score_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        L.nosa_status_string.argtypes = [ctypes.c_int32]
        L.nosa_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().nosa_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _dev(t: torch.Tensor | None, name: str, dtypes, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != NOSA_OK:
        raise NosaError(name, st)


def make_dims(B, Hq, Hkv, D, bs, ss, max_blocks) -> nosa_dims:
    return nosa_dims(int(B), int(Hq), int(Hkv), int(D), int(bs), int(ss), int(max_blocks))


def make_kv(k_pages, v_pages, e_pages, kind, *, table=None, directory=None, segments=None,
            seg_log2=0, blocks_log2=0, packed=None, q_pos=None, rope_base=0.0,
            err_flags=None, page_ptrs=None) -> nosa_kv:
    """Build the nosa_kv descriptor.  The tensors must outlive every call
    that receives the descriptor.  page_ptrs: (k, v, e) raw addresses used
    instead of the page tensors' device addresses (host pools: their host
    addresses, or their device mapping from nosa_host_device_pointer)."""
    kv = nosa_kv()
    if page_ptrs is None:
        kv.k_pages = _dev(k_pages, "k_pages", _BF16_LIKE)
        kv.v_pages = _dev(v_pages, "v_pages", _BF16_LIKE)
        kv.e_pages = _dev(e_pages, "e_pages", (torch.float32,))
    else:
        for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages"), (e_pages, "e_pages")):
            if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
                raise ValueError(f"{n}: a host pool must be a contiguous pinned CPU tensor")
        kv.k_pages, kv.v_pages, kv.e_pages = (ctypes.c_void_p(int(x)) for x in page_ptrs)
    kv.num_pages = int(k_pages.shape[0])
    kv.kind = int(kind)
    kv.table = _dev(table, "table", (torch.int32,), optional=True)
    kv.directory = _dev(directory, "directory", (torch.int32,), optional=True)
    kv.dir_entries = int(directory.numel()) if directory is not None else 0
    kv.segments = _dev(segments, "segments", (torch.int32,), optional=True)
    kv.num_segments = int(segments.shape[0]) if segments is not None else 0
    kv.seg_log2 = int(seg_log2)
    kv.blocks_log2 = int(blocks_log2)
    kv.packed = _dev(packed, "packed", (torch.int32, torch.uint32), optional=True)
    kv.q_pos = _dev(q_pos, "q_pos", (torch.int32,), optional=True)
    kv.rope_base = float(rope_base)
    kv.err_flags = _dev(err_flags, "err_flags", (torch.int32,), optional=True)
    return kv


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def nosa_prefill_pages(dims, kv, k_src, v_src, e_src, seq_lens, stream=None):
    src_tokens = int(k_src.shape[-2])
    _call("nosa_prefill_pages", ctypes.byref(dims), ctypes.byref(kv),
          _dev(k_src, "k_src", _BF16_LIKE), _dev(v_src, "v_src", _BF16_LIKE),
          _dev(e_src, "e_src", (torch.float32,)), src_tokens,
          _dev(seq_lens, "seq_lens", (torch.int32,)), _stream(stream))


def nosa_build_summaries(dims, kv, seq_lens, k_summary, e_summary, stream=None):
    _call("nosa_build_summaries", ctypes.byref(dims), ctypes.byref(kv),
          _dev(seq_lens, "seq_lens", (torch.int32,)), _dev(k_summary, "k_summary", (torch.float32,)),
          _dev(e_summary, "e_summary", (torch.float32,)), _stream(stream))


def nosa_append(dims, kv, k_new, v_new, e_new, seq_lens, k_summary, e_summary, stream=None):
    _call("nosa_append", ctypes.byref(dims), ctypes.byref(kv),
          _dev(k_new, "k_new", _BF16_LIKE), _dev(v_new, "v_new", _BF16_LIKE),
          _dev(e_new, "e_new", (torch.float32,)), _dev(seq_lens, "seq_lens", (torch.int32,)),
          _dev(k_summary, "k_summary", (torch.float32,)), _dev(e_summary, "e_summary", (torch.float32,)),
          _stream(stream))


def nosa_score_blocks(dims, q, k_summary, e_summary, seq_lens, score_q, score_e, stream=None):
    _call("nosa_score_blocks", ctypes.byref(dims), _dev(q, "q", _BF16_LIKE),
          _dev(k_summary, "k_summary", (torch.float32,)), _dev(e_summary, "e_summary", (torch.float32,)),
          _dev(seq_lens, "seq_lens", (torch.int32,)), _dev(score_q, "score_q", (torch.float32,)),
          _dev(score_e, "score_e", (torch.float32,)), _stream(stream))


def nosa_select(dims, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_count, stream=None):
    _call("nosa_select", ctypes.byref(dims), _dev(score_q, "score_q", (torch.float32,)),
          _dev(score_e, "score_e", (torch.float32,)), _dev(seq_lens, "seq_lens", (torch.int32,)),
          int(k_e), int(k_q), _dev(evicted, "evicted", (torch.int32, torch.uint32)),
          _dev(sel, "sel", (torch.int32,)), int(sel.shape[-1]),
          _dev(sel_count, "sel_count", (torch.int32,)), _stream(stream))


def nosa_select_swap(dims, score_q, score_e, seq_lens, k_e, k_q, evicted, sel, sel_count,
                     prev, prev_count, load, load_count, evict, evict_count, stream=None):
    cap = int(sel.shape[-1])
    for t, n in ((prev, "prev"), (load, "load"), (evict, "evict")):
        if int(t.shape[-1]) != cap:
            raise ValueError(f"{n} must have the same last dimension as sel ({cap})")
    _call("nosa_select_swap", ctypes.byref(dims), _dev(score_q, "score_q", (torch.float32,)),
          _dev(score_e, "score_e", (torch.float32,)), _dev(seq_lens, "seq_lens", (torch.int32,)),
          int(k_e), int(k_q), _dev(evicted, "evicted", (torch.int32, torch.uint32)),
          _dev(sel, "sel", (torch.int32,)), cap, _dev(sel_count, "sel_count", (torch.int32,)),
          _dev(prev, "prev", (torch.int32,)), _dev(prev_count, "prev_count", (torch.int32,)),
          _dev(load, "load", (torch.int32,)), _dev(load_count, "load_count", (torch.int32,)),
          _dev(evict, "evict", (torch.int32,)), _dev(evict_count, "evict_count", (torch.int32,)),
          _stream(stream))


def nosa_append_score(dims, kv, k_new, v_new, e_new, seq_lens_in, seq_lens_out, k_summary, e_summary, q,
                      score_q, score_e, stream=None):
    """k_new / v_new / e_new / seq_lens_out may all be None (no append)."""
    opt = k_new is None
    _call("nosa_append_score", ctypes.byref(dims), ctypes.byref(kv),
          _dev(k_new, "k_new", _BF16_LIKE, optional=opt), _dev(v_new, "v_new", _BF16_LIKE, optional=opt),
          _dev(e_new, "e_new", (torch.float32,), optional=opt),
          _dev(seq_lens_in, "seq_lens_in", (torch.int32,)),
          _dev(seq_lens_out, "seq_lens_out", (torch.int32,), optional=opt),
          _dev(k_summary, "k_summary", (torch.float32,)), _dev(e_summary, "e_summary", (torch.float32,)),
          _dev(q, "q", _BF16_LIKE), _dev(score_q, "score_q", (torch.float32,)),
          _dev(score_e, "score_e", (torch.float32,)), _stream(stream))


def nosa_swap_diff(dims, prev, prev_count, cur, cur_count, load, load_count, evict, evict_count,
                   stream=None):
    cap = int(prev.shape[-1])
    for t, n in ((cur, "cur"), (load, "load"), (evict, "evict")):
        if int(t.shape[-1]) != cap:
            raise ValueError(f"{n} must have the same last dimension as prev ({cap})")
    _call("nosa_swap_diff", ctypes.byref(dims), cap,
          _dev(prev, "prev", (torch.int32,)), _dev(prev_count, "prev_count", (torch.int32,)),
          _dev(cur, "cur", (torch.int32,)), _dev(cur_count, "cur_count", (torch.int32,)),
          _dev(load, "load", (torch.int32,)), _dev(load_count, "load_count", (torch.int32,)),
          _dev(evict, "evict", (torch.int32,)), _dev(evict_count, "evict_count", (torch.int32,)),
          _stream(stream))


def nosa_sparse_decode(dims, q, kv, sel, sel_count, seq_lens, num_splits, sm_scale,
                       part_o, part_m, part_l, stream=None):
    _call("nosa_sparse_decode", ctypes.byref(dims), _dev(q, "q", _BF16_LIKE), ctypes.byref(kv),
          _dev(sel, "sel", (torch.int32,)), _dev(sel_count, "sel_count", (torch.int32,)),
          int(sel.shape[-1]), _dev(seq_lens, "seq_lens", (torch.int32,)), int(num_splits),
          float(sm_scale), _dev(part_o, "part_o", (torch.float32,)),
          _dev(part_m, "part_m", (torch.float32,)), _dev(part_l, "part_l", (torch.float32,)),
          _stream(stream))


def nosa_sparse_decode_combine(dims, q, kv, sel, sel_count, seq_lens, num_splits, sm_scale,
                               part_o, part_m, part_l, counters, o, m, l, stream=None):
    _call("nosa_sparse_decode_combine", ctypes.byref(dims), _dev(q, "q", _BF16_LIKE), ctypes.byref(kv),
          _dev(sel, "sel", (torch.int32,)), _dev(sel_count, "sel_count", (torch.int32,)),
          int(sel.shape[-1]), _dev(seq_lens, "seq_lens", (torch.int32,)), int(num_splits),
          float(sm_scale), _dev(part_o, "part_o", (torch.float32,)),
          _dev(part_m, "part_m", (torch.float32,)), _dev(part_l, "part_l", (torch.float32,)),
          _dev(counters, "counters", (torch.int32,)), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)), _stream(stream))


def nosa_sparse_decode_mass(dims, q, kv, sel, sel_count, seq_lens, num_splits, sm_scale, part_o, part_m, part_l,
                            counters, o, m, l, tile_stats, mass, stream=None):
    """nosa_sparse_decode_combine plus each selected block's softmax mass
    per query head (mass: fp32 [B, Hq, sel_cap]; tile_stats: fp32 workspace
    of B * Hkv * sel_cap * (block_size // 64) * G * 2 elements)."""
    _call("nosa_sparse_decode_mass", ctypes.byref(dims), _dev(q, "q", _BF16_LIKE), ctypes.byref(kv),
          _dev(sel, "sel", (torch.int32,)), _dev(sel_count, "sel_count", (torch.int32,)),
          int(sel.shape[-1]), _dev(seq_lens, "seq_lens", (torch.int32,)), int(num_splits),
          float(sm_scale), _dev(part_o, "part_o", (torch.float32,)),
          _dev(part_m, "part_m", (torch.float32,)), _dev(part_l, "part_l", (torch.float32,)),
          _dev(counters, "counters", (torch.int32,)), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)),
          _dev(tile_stats, "tile_stats", (torch.float32,)), _dev(mass, "mass", (torch.float32,)), _stream(stream))


def nosa_sparse_decode_alibi(dims, q, kv, sel, sel_count, seq_lens, num_splits, sm_scale, alibi_slopes, part_o,
                             part_m, part_l, counters, o, m, l, stream=None):
    """nosa_sparse_decode_combine with ALiBi biases (alibi_slopes: fp32 [Hq])."""
    _call("nosa_sparse_decode_alibi", ctypes.byref(dims), _dev(q, "q", _BF16_LIKE), ctypes.byref(kv),
          _dev(sel, "sel", (torch.int32,)), _dev(sel_count, "sel_count", (torch.int32,)),
          int(sel.shape[-1]), _dev(seq_lens, "seq_lens", (torch.int32,)), int(num_splits),
          float(sm_scale), _dev(alibi_slopes, "alibi_slopes", (torch.float32,)),
          _dev(part_o, "part_o", (torch.float32,)),
          _dev(part_m, "part_m", (torch.float32,)), _dev(part_l, "part_l", (torch.float32,)),
          _dev(counters, "counters", (torch.int32,)), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)), _stream(stream))


def nosa_append_score_qkv(dims, kv, qkv, w_evict, seq_lens_in, seq_lens_out, k_summary, e_summary, q_out,
                          score_q, score_e, stream=None):
    """Append + score from the fused projection rows (qkv: bf16 [B, (Hq + 2 Hkv) D];
    w_evict: fp32 [Hkv, D]; q_out: bf16 [B, Hq, D])."""
    _call("nosa_append_score_qkv", ctypes.byref(dims), ctypes.byref(kv), _dev(qkv, "qkv", _BF16_LIKE),
          _dev(w_evict, "w_evict", (torch.float32,)), _dev(seq_lens_in, "seq_lens_in", (torch.int32,)),
          _dev(seq_lens_out, "seq_lens_out", (torch.int32,)),
          _dev(k_summary, "k_summary", (torch.float32,)), _dev(e_summary, "e_summary", (torch.float32,)),
          _dev(q_out, "q_out", _BF16_LIKE), _dev(score_q, "score_q", (torch.float32,)),
          _dev(score_e, "score_e", (torch.float32,)), _stream(stream))


def nosa_prefill_attention(dims, kv, q, q_pos0, seq_lens, sm_scale, o, m, l, stream=None):
    """Causal prefill of the prompt over reused documents (q: bf16 [B, M, Hq, D])."""
    _call("nosa_prefill_attention", ctypes.byref(dims), ctypes.byref(kv), _dev(q, "q", _BF16_LIKE),
          int(q.shape[1]), _dev(q_pos0, "q_pos0", (torch.int32,)), _dev(seq_lens, "seq_lens", (torch.int32,)),
          float(sm_scale), _dev(o, "o", (torch.float32,)), _dev(m, "m", (torch.float32,)),
          _dev(l, "l", (torch.float32,)), _stream(stream))


SELECT_DECODE_MAX_BLOCKS = 2304


def nosa_select_decode(dims, kv, q, score_q, score_e, seq_lens, k_e, k_q, evicted_in, evicted_out, sel, sel_count,
                       prev, prev_count, load, load_count, evict, evict_count, num_splits, sm_scale,
                       part_o, part_m, part_l, counters, o, m, l, stream=None):
    cap = int(sel.shape[-1])
    for t, n in ((prev, "prev"), (load, "load"), (evict, "evict")):
        if int(t.shape[-1]) != cap:
            raise ValueError(f"{n} must have the same last dimension as sel ({cap})")
    ev = (torch.int32, torch.uint32)
    _call("nosa_select_decode", ctypes.byref(dims), ctypes.byref(kv), _dev(q, "q", _BF16_LIKE),
          _dev(score_q, "score_q", (torch.float32,)), _dev(score_e, "score_e", (torch.float32,)),
          _dev(seq_lens, "seq_lens", (torch.int32,)), int(k_e), int(k_q),
          _dev(evicted_in, "evicted_in", ev), _dev(evicted_out, "evicted_out", ev),
          _dev(sel, "sel", (torch.int32,)), cap, _dev(sel_count, "sel_count", (torch.int32,)),
          _dev(prev, "prev", (torch.int32,)), _dev(prev_count, "prev_count", (torch.int32,)),
          _dev(load, "load", (torch.int32,)), _dev(load_count, "load_count", (torch.int32,)),
          _dev(evict, "evict", (torch.int32,)), _dev(evict_count, "evict_count", (torch.int32,)),
          int(num_splits), float(sm_scale), _dev(part_o, "part_o", (torch.float32,)),
          _dev(part_m, "part_m", (torch.float32,)), _dev(part_l, "part_l", (torch.float32,)),
          _dev(counters, "counters", (torch.int32,)), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)), _stream(stream))


def nosa_select_decode_noalloc(dims, kv, q, score_q, score_e, seq_lens, k_e, k_q, evicted_in, evicted_out, sel,
                               sel_count, prev, prev_count, load, load_count, evict, evict_count, num_splits,
                               sm_scale, o, m, l, stream=None):
    """nosa_select_decode with its workspaces in the library's static
    scratch: the call allocates nothing."""
    cap = int(sel.shape[-1])
    for t, n in ((prev, "prev"), (load, "load"), (evict, "evict")):
        if int(t.shape[-1]) != cap:
            raise ValueError(f"{n} must have the same last dimension as sel ({cap})")
    ev = (torch.int32, torch.uint32)
    _call("nosa_select_decode_noalloc", ctypes.byref(dims), ctypes.byref(kv), _dev(q, "q", _BF16_LIKE),
          _dev(score_q, "score_q", (torch.float32,)), _dev(score_e, "score_e", (torch.float32,)),
          _dev(seq_lens, "seq_lens", (torch.int32,)), int(k_e), int(k_q),
          _dev(evicted_in, "evicted_in", ev), _dev(evicted_out, "evicted_out", ev),
          _dev(sel, "sel", (torch.int32,)), cap, _dev(sel_count, "sel_count", (torch.int32,)),
          _dev(prev, "prev", (torch.int32,)), _dev(prev_count, "prev_count", (torch.int32,)),
          _dev(load, "load", (torch.int32,)), _dev(load_count, "load_count", (torch.int32,)),
          _dev(evict, "evict", (torch.int32,)), _dev(evict_count, "evict_count", (torch.int32,)),
          int(num_splits), float(sm_scale), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)), _stream(stream))


def nosa_host_device_pointer(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor."""
    if t.is_cuda or not t.is_pinned():
        raise ValueError("a pinned CPU tensor is required")
    out = ctypes.c_void_p()
    _call("nosa_host_device_pointer", ctypes.c_void_p(t.data_ptr()), ctypes.byref(out))
    return int(out.value)


def nosa_retrieve(dims, host_kv, dev_k, dev_v, dev_e, slots, resident, slot_owner, load, load_count, evict,
                  evict_count, seq_lens, seq_lens_prev=None, stream=None):
    """host_kv: descriptor whose page pointers are the host pools' HOST
    addresses (make_kv(..., page_ptrs=(t.data_ptr() ...)))."""
    cap = int(load.shape[-1])
    if int(evict.shape[-1]) != cap:
        raise ValueError("load and evict must have the same last dimension")
    _call("nosa_retrieve", ctypes.byref(dims), ctypes.byref(host_kv), _dev(dev_k, "dev_k", _BF16_LIKE),
          _dev(dev_v, "dev_v", _BF16_LIKE), _dev(dev_e, "dev_e", (torch.float32,)), int(slots),
          _dev(resident, "resident", (torch.int32,)), _dev(slot_owner, "slot_owner", (torch.int32,)),
          _dev(load, "load", (torch.int32,)), _dev(load_count, "load_count", (torch.int32,)),
          _dev(evict, "evict", (torch.int32,)), _dev(evict_count, "evict_count", (torch.int32,)), cap,
          _dev(seq_lens, "seq_lens", (torch.int32,)), _dev(seq_lens_prev, "seq_lens_prev", (torch.int32,), True),
          _stream(stream))


def nosa_retrieve_buffered(dims, host_kv, dev_k, dev_v, dev_e, slots, resident, slot_owner, last_use, sel,
                           sel_count, step, bucket_width, seq_lens, seq_lens_prev=None, miss_count=None,
                           stream=None):
    """As nosa_retrieve, driven by the selection itself, with the slots
    beyond the selection's capacity kept as a buffer (bucketed LRU)."""
    _call("nosa_retrieve_buffered", ctypes.byref(dims), ctypes.byref(host_kv), _dev(dev_k, "dev_k", _BF16_LIKE),
          _dev(dev_v, "dev_v", _BF16_LIKE), _dev(dev_e, "dev_e", (torch.float32,)), int(slots),
          _dev(resident, "resident", (torch.int32,)), _dev(slot_owner, "slot_owner", (torch.int32,)),
          _dev(last_use, "last_use", (torch.int32,)), _dev(sel, "sel", (torch.int32,)),
          _dev(sel_count, "sel_count", (torch.int32,)), int(sel.shape[-1]), int(step), int(bucket_width),
          _dev(seq_lens, "seq_lens", (torch.int32,)), _dev(seq_lens_prev, "seq_lens_prev", (torch.int32,), True),
          _dev(miss_count, "miss_count", (torch.int32,), optional=True), _stream(stream))


def nosa_combine(dims, num_splits, part_o, part_m, part_l, o, m, l, stream=None):
    _call("nosa_combine", ctypes.byref(dims), int(num_splits),
          _dev(part_o, "part_o", (torch.float32,)), _dev(part_m, "part_m", (torch.float32,)),
          _dev(part_l, "part_l", (torch.float32,)), _dev(o, "o", (torch.float32,)),
          _dev(m, "m", (torch.float32,)), _dev(l, "l", (torch.float32,)), _stream(stream))


def nosa_probe_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Read all of `src` (any dtype, contiguous, a multiple of 16 bytes) with
    the streaming-read probe; sink int32 [n_workgroups] receives the xor of
    each workgroup's words (the grid is sink's length)."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    _call("nosa_probe_stream_read", ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
          _dev(sink, "sink", (torch.int32,)), int(sink.numel()), _stream(stream))


def nosa_probe_page_gather(k_pool: torch.Tensor, v_pool: torch.Tensor, pages: torch.Tensor, sink: torch.Tensor,
                           stream=None):
    """Read the K and V pages listed in pages int32 [n_lists][pages_per_list]
    from the pools ([num_pages][...], contiguous, same shape) with the
    page-gather probe; sink int32 [n_lists]."""
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    if pages.dim() != 2:
        raise ValueError("pages must be [n_lists][pages_per_list]")
    num_pages = int(k_pool.shape[0])
    page_bytes = k_pool.numel() * k_pool.element_size() // num_pages
    _call("nosa_probe_page_gather", ctypes.c_void_p(k_pool.data_ptr()), ctypes.c_void_p(v_pool.data_ptr()),
          page_bytes, num_pages, _dev(pages, "pages", (torch.int32,)), int(pages.shape[0]), int(pages.shape[1]),
          _dev(sink, "sink", (torch.int32,)), _stream(stream))
