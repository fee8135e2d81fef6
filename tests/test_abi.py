"""The C-ABI library loads on the CPU host, exports every symbol the header
declares, and rejects bad arguments in its host-side checks (these return
before anything touches HIP, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nosa.h")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.path.join(ROOT, "block_sparse_kv_score_amd", "libnosa.so")),
    reason="libnosa.so not built (run __graft_entry__.build())")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:nosa_status|const char\*)\s+(nosa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_step_calls():
    names = declared_symbols()
    for n in ["nosa_score_blocks", "nosa_select", "nosa_swap_diff", "nosa_sparse_decode", "nosa_combine",
              "nosa_append", "nosa_build_summaries", "nosa_prefill_pages", "nosa_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    from block_sparse_kv_score_amd import nosa
    L = nosa.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert sorted(nosa.ENTRY_POINTS) == declared_symbols()


def test_status_strings():
    from block_sparse_kv_score_amd import nosa
    assert nosa.status_string(0) == "ok"
    assert "invalid" in nosa.status_string(-1)
    assert "unsupported" in nosa.status_string(-2)
    assert nosa.status_string(12345) == "unknown status"


def _good_dims(nosa):
    return nosa.make_dims(2, 8, 2, 128, 64, 16, 40)


def test_host_checks_reject_bad_arguments():
    from block_sparse_kv_score_amd import nosa
    L = nosa.lib()
    P = ctypes.c_void_p
    fake = P(256)  # never dereferenced: every call below fails its checks first
    d = _good_dims(nosa)
    D = ctypes.byref
    # null dims
    assert L.nosa_combine(None, 4, fake, fake, fake, fake, fake, fake, None) == nosa.NOSA_ERR_ARG
    # splits out of range, null outputs
    assert L.nosa_combine(D(d), 0, fake, fake, fake, fake, fake, fake, None) == nosa.NOSA_ERR_ARG
    assert L.nosa_combine(D(d), 257, fake, fake, fake, fake, fake, fake, None) == nosa.NOSA_ERR_ARG
    assert L.nosa_combine(D(d), 4, fake, fake, fake, None, fake, fake, None) == nosa.NOSA_ERR_ARG
    # shapes
    for field, value, want in [("n_q_heads", 7, nosa.NOSA_ERR_ARG),        # Hq % Hkv != 0
                               ("n_q_heads", 12, nosa.NOSA_ERR_UNSUPPORTED),  # G = 6
                               ("head_dim", 96, nosa.NOSA_ERR_UNSUPPORTED),
                               ("block_size", 56, nosa.NOSA_ERR_ARG),       # 56 % 16 != 0
                               ("block_size", 32, nosa.NOSA_ERR_UNSUPPORTED),
                               ("sub_block", 3, nosa.NOSA_ERR_ARG),
                               ("sub_block", 64 // 3 + 1, nosa.NOSA_ERR_ARG),
                               ("max_blocks", 0, nosa.NOSA_ERR_ARG),
                               ("max_blocks", 9000, nosa.NOSA_ERR_UNSUPPORTED),
                               ("batch", 0, nosa.NOSA_ERR_ARG)]:
        bad = _good_dims(nosa)
        setattr(bad, field, value)
        assert L.nosa_combine(D(bad), 4, fake, fake, fake, fake, fake, fake, None) == want, field
    # nsub = 64 / 2 = 32 is fine, 64 / 1 = 64 too; block 128 / sub 1 = 128 is not
    bad = _good_dims(nosa)
    bad.block_size, bad.sub_block = 128, 1
    assert L.nosa_combine(D(bad), 4, fake, fake, fake, fake, fake, fake, None) == nosa.NOSA_ERR_UNSUPPORTED
    # select: negative budgets, selection capacity too small
    assert L.nosa_select(D(d), fake, fake, fake, -1, 4, fake, fake, 8, fake, None) == nosa.NOSA_ERR_ARG
    assert L.nosa_select(D(d), fake, fake, fake, 4, 4, fake, fake, 7, fake, None) == nosa.NOSA_ERR_ARG
    # swap_diff capacity
    assert L.nosa_swap_diff(D(d), 0, fake, fake, fake, fake, fake, fake, fake, fake, None) == nosa.NOSA_ERR_ARG
    # decode: descriptor checks
    kv = nosa.nosa_kv()
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # no pages
    kv.k_pages = kv.v_pages = kv.e_pages = ctypes.c_void_p(4096)
    kv.num_pages = 10
    kv.kind = nosa.NOSA_TABLE_FLAT
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # flat table missing
    kv.kind = 7
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # unknown kind
    kv.kind = nosa.NOSA_TABLE_TWO_LEVEL
    kv.directory = kv.segments = ctypes.c_void_p(4096)
    kv.num_segments, kv.seg_log2, kv.blocks_log2, kv.dir_entries = 4, 10, 12, 15  # needs 16 entries
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG
    kv.kind = nosa.NOSA_TABLE_PACKED_ROPE
    kv.packed = ctypes.c_void_p(4096)
    kv.rope_base = 10000.0
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # q_pos missing
    kv.q_pos = ctypes.c_void_p(4096)
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 0, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # zero splits
    assert L.nosa_sparse_decode(D(d), fake, D(kv), fake, fake, 8, fake, 4, -1.0, fake, fake, fake,
                                None) == nosa.NOSA_ERR_ARG  # bad scale
    g16 = nosa.make_dims(2, 32, 2, 128, 64, 16, 40)
    assert L.nosa_sparse_decode(D(g16), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                None) == nosa.NOSA_ERR_UNSUPPORTED  # deferred RoPE with G = 16
    # misaligned 16-byte operands
    assert L.nosa_score_blocks(D(d), fake, ctypes.c_void_p(4100), fake, fake, fake, fake,
                               None) == nosa.NOSA_ERR_ARG
    # fused selection + swap lists: distinct list buffers, swap lists required
    sel_a, sel_b = P(1024), P(2048)
    assert L.nosa_select_swap(D(d), fake, fake, fake, 4, 4, fake, sel_a, 8, fake, sel_a, fake, fake, fake,
                              sel_b, fake, None) == nosa.NOSA_ERR_ARG  # prev aliases sel
    assert L.nosa_select_swap(D(d), fake, fake, fake, 4, 4, fake, sel_a, 8, fake, None, fake, fake, fake,
                              sel_b, fake, None) == nosa.NOSA_ERR_ARG  # prev missing
    # fused decode + combine: the arrival counters are required
    kv.kind = nosa.NOSA_TABLE_FLAT
    kv.table = ctypes.c_void_p(4096)
    assert L.nosa_sparse_decode_combine(D(d), fake, D(kv), fake, fake, 8, fake, 4, 0.1, fake, fake, fake,
                                        None, fake, fake, fake, None) == nosa.NOSA_ERR_ARG
    # fused select + decode
    def sdec(kvd, dims=d, ev_in=P(256), ev_out=P(512), splits=1, counters=fake):
        return L.nosa_select_decode(D(dims), D(kvd), fake, fake, fake, fake, 4, 4, ev_in, ev_out, sel_a, 8, fake,
                                    P(3072), fake, P(4096), fake, P(8192), fake, splits, 0.1, fake, fake, fake,
                                    counters, fake, fake, fake, None)
    assert sdec(kv, ev_in=P(256), ev_out=P(256), splits=2) == nosa.NOSA_ERR_ARG  # shared bitmap, 2 splits
    assert sdec(kv, counters=None) == nosa.NOSA_ERR_ARG
    big = nosa.make_dims(2, 8, 2, 128, 64, 16, 2305)
    assert sdec(kv, dims=big) == nosa.NOSA_ERR_UNSUPPORTED  # capacity above the fused selection's
    rope = nosa.nosa_kv()
    rope.k_pages = rope.v_pages = rope.e_pages = ctypes.c_void_p(4096)
    rope.num_pages, rope.kind, rope.packed = 10, nosa.NOSA_TABLE_PACKED_ROPE, ctypes.c_void_p(4096)
    assert sdec(rope) == nosa.NOSA_ERR_ARG  # deferred RoPE without query positions
    rope_g16 = nosa.nosa_kv()
    rope_g16.k_pages = rope_g16.v_pages = rope_g16.e_pages = ctypes.c_void_p(4096)
    rope_g16.num_pages, rope_g16.kind, rope_g16.packed = 10, nosa.NOSA_TABLE_PACKED_ROPE, ctypes.c_void_p(4096)
    rope_g16.q_pos, rope_g16.rope_base = ctypes.c_void_p(4096), 10000.0
    assert sdec(rope_g16, dims=nosa.make_dims(2, 32, 2, 128, 64, 16, 40)) == nosa.NOSA_ERR_UNSUPPORTED  # G = 16
    # softmax score step: workspace and output required, no packed RoPE kind
    def mdec(kvd, stats=fake, mass=fake):
        return L.nosa_sparse_decode_mass(D(d), fake, D(kvd), fake, fake, 8, fake, 1, 0.1, fake, fake, fake, fake,
                                         fake, fake, fake, stats, mass, None)
    assert mdec(kv, stats=None) == nosa.NOSA_ERR_ARG
    assert mdec(kv, mass=None) == nosa.NOSA_ERR_ARG
    rope.q_pos, rope.rope_base = ctypes.c_void_p(4096), 10000.0
    assert mdec(rope) == nosa.NOSA_ERR_UNSUPPORTED
    # ALiBi decode: slopes required, no packed RoPE kind
    def adec(kvd, slopes=fake):
        return L.nosa_sparse_decode_alibi(D(d), fake, D(kvd), fake, fake, 8, fake, 1, 0.1, slopes, fake, fake, fake,
                                          fake, fake, fake, fake, None)
    assert adec(kv, slopes=None) == nosa.NOSA_ERR_ARG
    assert adec(rope) == nosa.NOSA_ERR_UNSUPPORTED
    # append from fused projection rows: weights and split-query output required
    def qkv_app(kvd, w_e=fake, q_out=fake, seq_out=P(768)):
        return L.nosa_append_score_qkv(D(d), D(kvd), fake, w_e, P(512), seq_out, fake, fake, q_out, fake, fake,
                                       None)
    assert qkv_app(kv, w_e=None) == nosa.NOSA_ERR_ARG
    assert qkv_app(kv, q_out=None) == nosa.NOSA_ERR_ARG
    assert qkv_app(kv, seq_out=P(512)) == nosa.NOSA_ERR_ARG  # lengths in place
    assert qkv_app(rope) == nosa.NOSA_ERR_UNSUPPORTED
    # prefill: packed RoPE descriptors only, a prompt of at least one token
    def pf(kvd, n_prompt=4, q_pos0=fake):
        return L.nosa_prefill_attention(D(d), D(kvd), fake, n_prompt, q_pos0, fake, 0.1, fake, fake, fake, None)
    assert pf(kv) == nosa.NOSA_ERR_UNSUPPORTED
    assert pf(rope, n_prompt=0) == nosa.NOSA_ERR_ARG
    assert pf(rope, q_pos0=None) == nosa.NOSA_ERR_ARG
    # host-tier retrieve: slot count bounds, required lists
    def retr(slots, load=fake):
        return L.nosa_retrieve(D(d), D(kv), P(4096), P(8192), P(12288), slots, fake, fake, load, fake, fake, fake,
                               8, fake, None, None)
    assert retr(0) == nosa.NOSA_ERR_ARG
    assert retr(1025) == nosa.NOSA_ERR_ARG
    assert retr(8, load=None) == nosa.NOSA_ERR_ARG
    assert L.nosa_host_device_pointer(None, ctypes.byref(ctypes.c_void_p())) == nosa.NOSA_ERR_ARG
    # buffered retrieve: cap <= slots <= 1024, step >= 1, bucket width >= 1
    def buf(slots, cap=8, step=1, width=1, last_use=fake):
        return L.nosa_retrieve_buffered(D(d), D(kv), P(4096), P(8192), P(12288), slots, fake, fake, last_use, fake,
                                        fake, cap, step, width, fake, None, None, None)
    assert buf(7) == nosa.NOSA_ERR_ARG                 # fewer slots than the selection can hold
    assert buf(1025) == nosa.NOSA_ERR_ARG
    assert buf(16, step=0) == nosa.NOSA_ERR_ARG
    assert buf(16, width=0) == nosa.NOSA_ERR_ARG
    assert buf(16, last_use=None) == nosa.NOSA_ERR_ARG
    # fused append + score
    def ascore(k_new, seq_in, seq_out, v_new=None):
        v = v_new if v_new is not None else (fake if k_new else None)
        return L.nosa_append_score(D(d), D(kv), k_new, v, fake if k_new else None, seq_in, seq_out, fake, fake,
                                   fake, fake, fake, None)
    seq_a, seq_b = P(512), P(768)
    assert ascore(fake, seq_a, seq_a) == nosa.NOSA_ERR_ARG      # lengths in place
    assert ascore(fake, seq_a, None) == nosa.NOSA_ERR_ARG       # append without an output length
    assert ascore(P(4100), seq_a, seq_b) == nosa.NOSA_ERR_ARG   # misaligned k_new
    assert ascore(None, seq_a, None, v_new=fake) == nosa.NOSA_ERR_ARG  # v_new without k_new
    assert ascore(None, None, None) == nosa.NOSA_ERR_ARG        # no lengths


def test_binding_refuses_cpu_tensors():
    import torch
    from block_sparse_kv_score_amd import nosa
    d = _good_dims(nosa)
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        nosa.nosa_combine(d, 4, x, x, x, x, x, x)


def test_probe_host_checks():
    """The bandwidth probes refuse bad arguments before any launch."""
    from block_sparse_kv_score_amd import nosa
    L = nosa.lib()
    P = ctypes.c_void_p
    fake, odd = P(256), P(264)  # never dereferenced
    E = nosa.NOSA_ERR_ARG
    assert L.nosa_probe_stream_read(None, 1024, fake, 8, None) == E
    assert L.nosa_probe_stream_read(odd, 1024, fake, 8, None) == E      # src not 16-byte aligned
    assert L.nosa_probe_stream_read(fake, 1000, fake, 8, None) == E     # not a multiple of 16
    assert L.nosa_probe_stream_read(fake, 1024, fake, 0, None) == E
    assert L.nosa_probe_stream_read(fake, 1024, fake, 65537, None) == E
    assert L.nosa_probe_stream_read(fake, 1024, None, 8, None) == E
    assert L.nosa_probe_page_gather(fake, fake, 12288, 10, fake, 4, 16, fake, None) == E  # page size
    assert L.nosa_probe_page_gather(fake, odd, 16384, 10, fake, 4, 16, fake, None) == E
    assert L.nosa_probe_page_gather(fake, fake, 16384, 0, fake, 4, 16, fake, None) == E
    assert L.nosa_probe_page_gather(fake, fake, 16384, 10, fake, 0, 16, fake, None) == E
    assert L.nosa_probe_page_gather(fake, fake, 16384, 10, fake, 4, 257, fake, None) == E
    assert L.nosa_probe_page_gather(fake, fake, 16384, 10, None, 4, 16, fake, None) == E


def test_noalloc_refuses_partials_beyond_the_scratch():
    from block_sparse_kv_score_amd import nosa
    L = nosa.lib()
    fake = ctypes.c_void_p(256)  # never dereferenced: the call is refused before any launch
    d = nosa.make_dims(32, 32, 8, 128, 64, 16, 600)
    kv = nosa.nosa_kv()
    kv.k_pages = kv.v_pages = kv.e_pages = fake
    kv.num_pages = 1 << 16
    kv.kind = nosa.NOSA_TABLE_FLAT
    kv.table = fake
    args = [ctypes.byref(d), ctypes.byref(kv), fake, fake, fake, fake, 32, 32, fake, ctypes.c_void_p(512), fake, 64,
            fake, ctypes.c_void_p(768), fake, ctypes.c_void_p(1024), fake, ctypes.c_void_p(1280), fake]
    tail = [0.088, fake, fake, fake, None]
    assert L.nosa_select_decode_noalloc(*args, 32, *tail) == nosa.NOSA_ERR_SCRATCH
    assert L.nosa_select_decode_noalloc(*args, 256, *tail) == nosa.NOSA_ERR_SCRATCH
    assert "scratch" in nosa.status_string(nosa.NOSA_ERR_SCRATCH)
