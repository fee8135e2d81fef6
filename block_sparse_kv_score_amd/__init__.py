"""MI355X-native (gfx950) block-sparse KV scoring and sparse decode.

One decode step of NOSA-style block-sparse attention over a paged KV cache:
block scoring (sub-block mean pool, then block max pool) for a query-aware
score and a pre-exp eviction score, dual selection, the swap set
difference, split-K decode over the selected pages and the (O, rowmax, l)
combine.  The work runs in hand-written HIP kernels behind the C-ABI library
``libnosa.so``; ``nosa`` is its thin ctypes binding.

Importing the package loads nothing native; ``block_sparse_kv_score_amd.nosa``
loads the library on first use and raises if it is missing.
"""

__all__ = ["nosa", "workloads", "synth"]
