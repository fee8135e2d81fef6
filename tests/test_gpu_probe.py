"""The bandwidth probes read every byte they are given: the xor of each
probe's sink equals the xor of the 32-bit words it was to read, computed on
the CPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel()))


def test_stream_read_reads_every_word():
    from block_sparse_kv_score_amd import nosa
    print("\n[case] probe stream read, 3 sizes", flush=True)
    g = np.random.default_rng(5)
    for n16, wgs in [(1, 1), (1000 * 256 + 7, 97), (1 << 20, 2048)]:
        host = g.integers(0, 2**32, size=n16 * 4, dtype=np.uint32)
        src = torch.from_numpy(host.view(np.int32)).cuda()
        sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        nosa.nosa_probe_stream_read(src, sink)
        torch.cuda.synchronize()
        assert _xor_words(sink.cpu().numpy()) == _xor_words(host), (n16, wgs)


@pytest.mark.parametrize("page_bytes", [8192, 16384, 32768])
def test_page_gather_reads_every_listed_page(page_bytes):
    from block_sparse_kv_score_amd import nosa
    print(f"\n[case] probe page gather, pages of {page_bytes} bytes", flush=True)
    g = np.random.default_rng(page_bytes)
    num_pages, n_lists = 300, 6
    words = page_bytes // 4
    k = g.integers(0, 2**32, size=(num_pages, words), dtype=np.uint32)
    v = g.integers(0, 2**32, size=(num_pages, words), dtype=np.uint32)
    for ppl in [1, 5, 64, 256]:
        pages = g.integers(0, num_pages, size=(n_lists, ppl)).astype(np.int32)
        pages[0, 0] = -1               # skipped
        pages[-1, -1] = num_pages      # skipped
        kt = torch.from_numpy(k.view(np.int32)).cuda()
        vt = torch.from_numpy(v.view(np.int32)).cuda()
        sink = torch.zeros(n_lists, dtype=torch.int32, device="cuda")
        nosa.nosa_probe_page_gather(kt, vt, torch.from_numpy(pages).cuda(), sink)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        for li in range(n_lists):
            ids = [p for p in pages[li] if 0 <= p < num_pages]
            want = 0
            for p in ids:
                want ^= _xor_words(k[p]) ^ _xor_words(v[p])
            assert int(got[li]) == want, (ppl, li)
