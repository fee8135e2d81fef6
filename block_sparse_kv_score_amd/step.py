"""Device buffers for one decode-step workload and the call sequence of a
step.  Marshalling only: every step of the path runs in libnosa's kernels;
this module allocates buffers with PyTorch and calls the C-ABI entry points
in order on one stream.

Call sequence of decode step t (1-based):
  nosa_append            (workloads that append a token per step)
  nosa_score_blocks      (skipped when every block is selected)
  nosa_select            ( "            "              " )
  nosa_swap_diff         against the previous step's selection
  nosa_sparse_decode     split-K over the selected pages
  nosa_combine           -> O, rowmax m, l
With `fused` (the default) the step is two launches with the same results:
  nosa_append_score          append + score
  nosa_select_decode         select + swap_diff + decode + combine
(where nosa_select_decode is not supported -- more than 2304 blocks of
capacity, or deferred RoPE with more than 8 query heads per KV head -- or
by default above four splits, nosa_select_swap then
nosa_sparse_decode_combine; with every block selected: nosa_swap_diff,
then the fused decode).  The fused launches
write the new lengths and the new eviction bitmap to the other of two
buffers, so `seq_lens` and `evicted` name the current ones.

With `offload` the whole paged cache lives in pinned host memory and HBM
keeps `cap` resident pages per (b, h) (the host tier): the step is
nosa_append_score (into the host pages), nosa_select_swap, nosa_retrieve
(the swap lists move pages into the resident slots) and
nosa_sparse_decode_combine over the resident pages.  With `buffer_slots`
(>= the selection's capacity) HBM keeps that many slots per (b, h) and
nosa_retrieve_buffered replaces nosa_retrieve: pages stay resident after
they leave the selection and a bucketed LRU frees slots for misses.

With `mass` the decode is nosa_sparse_decode_mass (after nosa_select_swap):
the softmax score step adds each selected block's softmax mass per query
head (`mass`) to O, m, l.  With `alibi` it is nosa_sparse_decode_alibi,
with the slopes of the synthetic inputs.  With `qkv` the append is
nosa_append_score_qkv: the step's input is each sequence's fused projection
row, the eviction logit comes from the eviction head, and the decode reads
the query that call split out.
"""

from __future__ import annotations

import numpy as np
import torch

from . import nosa, synth
from .synth import Inputs
from .workloads import TABLE_FLAT, TABLE_PACKED_ROPE, TABLE_TWO_LEVEL, Workload

_KIND = {TABLE_FLAT: nosa.NOSA_TABLE_FLAT, TABLE_TWO_LEVEL: nosa.NOSA_TABLE_TWO_LEVEL,
         TABLE_PACKED_ROPE: nosa.NOSA_TABLE_PACKED_ROPE}

BF16_NAN = -1  # 0xFFFF as int16: a NaN bit pattern for never-written slots
SELECT_DECODE_AUTO_MAX_SPLITS = 4  # default: nosa_select_decode up to this many splits


def _i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32))


class DecodeSession:
    """All device state of one workload: page pools, tables, summaries,
    selection state and step outputs."""

    def __init__(self, w: Workload, inp: Inputs, splits: int | None = None, device: str = "cuda",
                 poison: bool = True, stream: torch.cuda.Stream | None = None, fused: bool = True,
                 offload: bool = False, buffer_slots: int | None = None, bucket_width: int = 1,
                 mass: bool = False, alibi: bool = False, qkv: bool = False,
                 select_decode: bool | None = None):
        self.w, self.inp = w, inp
        self.buffered = buffer_slots is not None
        self.buffer_slots, self.bucket_width = buffer_slots, int(bucket_width)
        self.buffer_clock = 0  # the buffer's timestamps: one tick per retrieve
        self.mass_on = mass
        if mass and (w.table == TABLE_PACKED_ROPE or not fused):
            raise ValueError("the softmax score step runs in the fused decode over flat or two-level tables")
        self.qkv_on = qkv
        if qkv and (w.table == TABLE_PACKED_ROPE or not fused or not w.append or offload):
            raise ValueError("the QKV-row append runs in the fused step over flat or two-level tables, in HBM")
        self.alibi_on = alibi
        if alibi and (w.table == TABLE_PACKED_ROPE or not fused or mass):
            raise ValueError("ALiBi runs in the fused decode over flat or two-level tables, without the mass step")
        if self.buffered and not offload:
            raise ValueError("buffer_slots needs the host tier (offload=True)")
        self.fused = fused
        self.offload = offload
        if offload and (w.select_all or w.table == TABLE_PACKED_ROPE):
            raise ValueError("the host tier is built for selecting workloads with flat or two-level tables")
        self.P = int(splits or w.splits)
        self.dev = torch.device(device)
        self.stream = stream
        self.step_index = 0
        self.n_steps = 0  # steps run so far, eager or replayed (the graphs alternate with it)
        B, Hq, Hkv, D, bs, ss, MB = w.B, w.Hq, w.Hkv, w.D, w.bs, w.ss, w.max_blocks
        self.dims = nosa.make_dims(B, Hq, Hkv, D, bs, ss, MB)
        self.cap = MB if w.select_all else min(w.k, MB)
        CS = MB * w.nsub
        dev = self.dev
        fill = float("nan") if poison else 0.0

        # page pools (never-written slots hold NaN patterns when poisoned)
        self.k_pages = torch.full((w.num_pages, bs * D), BF16_NAN if poison else 0, dtype=torch.int16, device=dev)
        self.v_pages = torch.full_like(self.k_pages, BF16_NAN if poison else 0)
        self.e_pages = torch.full((w.num_pages, bs), fill, dtype=torch.float32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.table = self.directory = self.segments = self.packed = self.q_pos = None
        if w.table == TABLE_FLAT:
            self.table = torch.from_numpy(inp.pages).to(dev)
        elif w.table == TABLE_TWO_LEVEL:
            self.directory = torch.from_numpy(inp.directory).to(dev)
            self.segments = torch.from_numpy(inp.segments).to(dev)
        else:
            self.packed = _i32(inp.packed).to(dev)
            self.q_pos = torch.from_numpy(inp.q_pos).to(dev)
        self.kv = nosa.make_kv(self.k_pages, self.v_pages, self.e_pages, _KIND[w.table], **self._table_kw())

        self.seq_bufs = [torch.full((B,), w.T0, dtype=torch.int32, device=dev) for _ in range(2)]
        self.seq_lens = self.seq_bufs[0]
        self.k_summary = torch.full((B, Hkv, D // 4, CS, 4), fill, dtype=torch.float32, device=dev)
        self.e_summary = torch.full((B, Hkv, CS), fill, dtype=torch.float32, device=dev)
        self.score_q = torch.full((B, Hkv, MB), fill, dtype=torch.float32, device=dev)
        self.score_e = torch.full_like(self.score_q, fill)
        self.ev_bufs = [torch.zeros((B, Hkv, (MB + 31) // 32), dtype=torch.int32, device=dev) for _ in range(2)]
        self.evicted = self.ev_bufs[0]
        # nosa_select_decode where it supports the shape and, by default, at
        # few splits only: every workgroup of a pair repeats the selection and
        # the select variant keeps one wave per SIMD, so with many short
        # workgroups per pair nosa_select_swap + nosa_sparse_decode_combine
        # is faster.  select_decode=True takes it wherever it is supported.
        supported = MB <= nosa.SELECT_DECODE_MAX_BLOCKS and (w.table != TABLE_PACKED_ROPE or w.G <= 8)
        if select_decode is None:
            self.select_decode_ok = supported and self.P <= SELECT_DECODE_AUTO_MAX_SPLITS
        else:
            self.select_decode_ok = supported and bool(select_decode)
        # selections ping-pong between two buffers: step t writes buffer t % 2
        # and diffs against buffer (t - 1) % 2 (both start empty)
        self.sel_bufs = [torch.full((B, Hkv, self.cap), -1, dtype=torch.int32, device=dev) for _ in range(2)]
        self.cnt_bufs = [torch.zeros((B, Hkv), dtype=torch.int32, device=dev) for _ in range(2)]
        self.sel, self.sel_count = self.sel_bufs[0], self.cnt_bufs[0]
        self.prev, self.prev_count = self.sel_bufs[1], self.cnt_bufs[1]
        self.load = torch.full_like(self.sel, -1)
        self.load_count = torch.zeros_like(self.sel_count)
        self.evict = torch.full_like(self.sel, -1)
        self.evict_count = torch.zeros_like(self.sel_count)
        self.part_o = torch.full((B, Hq, self.P, D), fill, dtype=torch.float32, device=dev)
        self.part_m = torch.full((B, Hq, self.P), fill, dtype=torch.float32, device=dev)
        self.part_l = torch.full_like(self.part_m, fill)
        self.o = torch.full((B, Hq, D), fill, dtype=torch.float32, device=dev)
        self.m = torch.full((B, Hq), fill, dtype=torch.float32, device=dev)
        self.l = torch.full_like(self.m, fill)
        self.counters = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)  # fused combine arrivals
        if qkv:  # fused projection rows per step, the eviction head, the split query
            self.qkv_all = torch.from_numpy(np.stack([synth.qkv_rows(w, inp, t).view(np.int16)
                                                      for t in range(1, w.n_append + 1)])).to(dev)
            self.w_evict = torch.from_numpy(synth.eviction_head_weights(w, inp.seed)).to(dev)
            self.q_out = torch.zeros((B, Hq, D), dtype=torch.int16, device=dev)
        if w.prompt:  # prefill over reused documents: the prompt's queries and outputs
            M = w.prompt
            self.q_prefill = torch.from_numpy(synth.prefill_queries(w, inp.seed).view(np.int16)).to(dev)
            self.q_pos0 = torch.full((B,), w.T0 - M, dtype=torch.int32, device=dev)
            self.pf_o = torch.full((B, M, Hq, D), fill, dtype=torch.float32, device=dev)
            self.pf_m = torch.full((B, M, Hq), fill, dtype=torch.float32, device=dev)
            self.pf_l = torch.full_like(self.pf_m, fill)
        if alibi:  # per query head slopes
            self.alibi_slopes = torch.from_numpy(synth.alibi_slopes(Hq)).to(dev)
        if mass:  # softmax score step: per-tile workspace and the block masses
            self.tile_stats = torch.zeros(B * Hkv * self.cap * (bs // 64) * w.G * 2, dtype=torch.float32, device=dev)
            self.mass = torch.full((B, Hq, self.cap), fill, dtype=torch.float32, device=dev)

        # per-step queries and appended tokens, resident before timing
        n_steps = w.n_append if w.append else max(1, w.steps)
        self.q_all = torch.from_numpy(np.stack([inp.q(t).view(np.int16) for t in range(1, n_steps + 1)])).to(dev)
        if w.append:
            A = w.n_append
            self.k_new = torch.from_numpy(np.ascontiguousarray(
                inp.K[:, :, w.T0:w.T0 + A].transpose(2, 0, 1, 3)).view(np.int16)).to(dev)
            self.v_new = torch.from_numpy(np.ascontiguousarray(
                inp.V[:, :, w.T0:w.T0 + A].transpose(2, 0, 1, 3)).view(np.int16)).to(dev)
            self.e_new = torch.from_numpy(np.ascontiguousarray(inp.e[:, :, w.T0:w.T0 + A].transpose(2, 0, 1))).to(dev)
        if w.select_all:
            # every block, fixed: the static list and an empty "previous" one
            nb = -(-w.T0 // bs)
            sel = np.full((B, Hkv, self.cap), -1, dtype=np.int32)
            sel[:, :, :nb] = np.arange(nb, dtype=np.int32)
            self.all_sel = torch.from_numpy(sel).to(dev)
            self.all_count = torch.full((B, Hkv), nb, dtype=torch.int32, device=dev)
        self.prefill()
        if offload:
            self._init_offload(poison)

    def _table_kw(self) -> dict:
        w = self.w
        return dict(table=self.table, directory=self.directory, segments=self.segments, seg_log2=w.seg_log2,
                    blocks_log2=w.blocks_log2, packed=self.packed, q_pos=self.q_pos, rope_base=w.rope_base,
                    err_flags=self.err)

    def _init_offload(self, poison: bool):
        """Move the paged cache to pinned host memory; keep `cap` resident
        pages per (b, h) in HBM."""
        w = self.w
        self.host_k = torch.empty(self.k_pages.shape, dtype=torch.int16, pin_memory=True)
        self.host_v = torch.empty(self.v_pages.shape, dtype=torch.int16, pin_memory=True)
        self.host_e = torch.empty(self.e_pages.shape, dtype=torch.float32, pin_memory=True)
        self.host_k.copy_(self.k_pages)
        self.host_v.copy_(self.v_pages)
        self.host_e.copy_(self.e_pages)
        torch.cuda.synchronize()
        del self.k_pages, self.v_pages, self.e_pages
        hosts = (self.host_k, self.host_v, self.host_e)
        kw = self._table_kw()
        # the retrieve reads the host pools by their host addresses; the
        # append writes them (and reads older tokens) through their device mapping
        self.host_kv = nosa.make_kv(*hosts, _KIND[w.table], page_ptrs=[t.data_ptr() for t in hosts], **kw)
        self.kv = nosa.make_kv(*hosts, _KIND[w.table], page_ptrs=[nosa.nosa_host_device_pointer(t) for t in hosts],
                               **kw)
        self.slots = self.cap
        if self.buffered:
            if self.buffer_slots < self.cap:
                raise ValueError(f"buffer_slots must be at least the selection capacity {self.cap}")
            self.slots = int(self.buffer_slots)
            self.last_use = torch.zeros((w.B, w.Hkv, self.slots), dtype=torch.int32, device=self.dev)
            self.miss_count = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=self.dev)
        n = w.B * w.Hkv * self.slots
        fill = float("nan") if poison else 0.0
        self.k_pages = torch.full((n, w.bs * w.D), BF16_NAN if poison else 0, dtype=torch.int16, device=self.dev)
        self.v_pages = torch.full_like(self.k_pages, BF16_NAN if poison else 0)
        self.e_pages = torch.full((n, w.bs), fill, dtype=torch.float32, device=self.dev)
        self.resident = torch.full((w.B, w.Hkv, w.max_blocks), -1, dtype=torch.int32, device=self.dev)
        self.slot_owner = torch.full((w.B, w.Hkv, self.slots), -1, dtype=torch.int32, device=self.dev)
        self.dev_kv = nosa.make_kv(self.k_pages, self.v_pages, self.e_pages, nosa.NOSA_TABLE_FLAT,
                                   table=self.resident, err_flags=self.err)

    # ------------------------------------------------------------------
    def prefill(self):
        """Write the context into pages and build the summaries (Index)."""
        w, inp = self.w, self.inp
        k_src = torch.from_numpy(inp.K.view(np.int16)).to(self.dev)
        v_src = torch.from_numpy(inp.V.view(np.int16)).to(self.dev)
        e_src = torch.from_numpy(inp.e).to(self.dev)
        nosa.nosa_prefill_pages(self.dims, self.kv, k_src, v_src, e_src, self.seq_lens, self.stream)
        nosa.nosa_build_summaries(self.dims, self.kv, self.seq_lens, self.k_summary, self.e_summary, self.stream)
        torch.cuda.synchronize()
        del k_src, v_src, e_src

    def q(self, t: int) -> torch.Tensor:
        if self.qkv_on:  # the query the fused append split out of this step's rows
            return self.q_out
        return self.q_all[t - 1]

    # ------------------------------------------------------------------
    # individual stages (the step is their sequence)
    def append(self, t: int):
        nosa.nosa_append(self.dims, self.kv, self.k_new[t - 1], self.v_new[t - 1], self.e_new[t - 1],
                         self.seq_lens, self.k_summary, self.e_summary, self.stream)

    def score(self, t: int):
        if self.w.table == TABLE_PACKED_ROPE:
            # scores need the per-document query rotation: the descriptor-aware
            # scoring of nosa_append_score (no append on this table kind)
            nosa.nosa_append_score(self.dims, self.kv, None, None, None, self.seq_lens, None, self.k_summary,
                                   self.e_summary, self.q(t), self.score_q, self.score_e, self.stream)
            return
        nosa.nosa_score_blocks(self.dims, self.q(t), self.k_summary, self.e_summary, self.seq_lens,
                               self.score_q, self.score_e, self.stream)

    def select(self):
        nosa.nosa_select(self.dims, self.score_q, self.score_e, self.seq_lens, self.w.k_e, self.w.k_q,
                         self.evicted, self.sel, self.sel_count, self.stream)

    def swap_diff(self):
        nosa.nosa_swap_diff(self.dims, self.prev, self.prev_count, self.sel, self.sel_count,
                            self.load, self.load_count, self.evict, self.evict_count, self.stream)

    def decode(self, t: int):
        nosa.nosa_sparse_decode(self.dims, self.q(t), self.kv, self.sel, self.sel_count, self.seq_lens,
                                self.P, self.w.sm_scale, self.part_o, self.part_m, self.part_l, self.stream)

    def append_score(self, t: int):
        """Fused append + score; afterwards seq_lens is the other buffer."""
        w = self.w
        out = self.seq_bufs[1] if self.seq_lens is self.seq_bufs[0] else self.seq_bufs[0]
        if self.qkv_on:
            nosa.nosa_append_score_qkv(self.dims, self.kv, self.qkv_all[t - 1], self.w_evict, self.seq_lens, out,
                                       self.k_summary, self.e_summary, self.q_out, self.score_q, self.score_e,
                                       self.stream)
            self.seq_lens = out
            return
        if w.append:
            k_new, v_new, e_new, seq_out = self.k_new[t - 1], self.v_new[t - 1], self.e_new[t - 1], out
        else:
            k_new = v_new = e_new = seq_out = None
        nosa.nosa_append_score(self.dims, self.kv, k_new, v_new, e_new, self.seq_lens, seq_out, self.k_summary,
                               self.e_summary, self.q(t), self.score_q, self.score_e, self.stream)
        if w.append:
            self.seq_lens = out

    def select_swap(self):
        nosa.nosa_select_swap(self.dims, self.score_q, self.score_e, self.seq_lens, self.w.k_e, self.w.k_q,
                              self.evicted, self.sel, self.sel_count, self.prev, self.prev_count,
                              self.load, self.load_count, self.evict, self.evict_count, self.stream)

    def retrieve(self):
        """Host tier: bring the selection into the resident slots.  The
        lengths before this step's append are the other length buffer, so
        only the appended token is copied into a resident tail page."""
        prev = self.seq_bufs[1] if self.seq_lens is self.seq_bufs[0] else self.seq_bufs[0]
        if not self.w.append:
            prev = self.seq_lens
        if self.buffered:
            self.buffer_clock += 1
            nosa.nosa_retrieve_buffered(self.dims, self.host_kv, self.k_pages, self.v_pages, self.e_pages,
                                        self.slots, self.resident, self.slot_owner, self.last_use, self.sel,
                                        self.sel_count, self.buffer_clock, self.bucket_width, self.seq_lens,
                                        prev, self.miss_count, self.stream)
        else:
            nosa.nosa_retrieve(self.dims, self.host_kv, self.k_pages, self.v_pages, self.e_pages, self.slots,
                               self.resident, self.slot_owner, self.load, self.load_count, self.evict,
                               self.evict_count, self.seq_lens, prev, self.stream)

    def decode_combine(self, t: int):
        kv = self.dev_kv if self.offload else self.kv
        if self.alibi_on:
            nosa.nosa_sparse_decode_alibi(self.dims, self.q(t), kv, self.sel, self.sel_count, self.seq_lens, self.P,
                                          self.w.sm_scale, self.alibi_slopes, self.part_o, self.part_m, self.part_l,
                                          self.counters, self.o, self.m, self.l, self.stream)
            return
        if self.mass_on:
            nosa.nosa_sparse_decode_mass(self.dims, self.q(t), kv, self.sel, self.sel_count, self.seq_lens, self.P,
                                         self.w.sm_scale, self.part_o, self.part_m, self.part_l, self.counters,
                                         self.o, self.m, self.l, self.tile_stats, self.mass, self.stream)
            return
        nosa.nosa_sparse_decode_combine(self.dims, self.q(t), kv, self.sel, self.sel_count, self.seq_lens,
                                        self.P, self.w.sm_scale, self.part_o, self.part_m, self.part_l,
                                        self.counters, self.o, self.m, self.l, self.stream)

    def prefill_attention(self):
        """The prompt's causal attention over the reused documents (prefill
        workloads)."""
        nosa.nosa_prefill_attention(self.dims, self.kv, self.q_prefill, self.q_pos0, self.seq_lens, self.w.sm_scale,
                                    self.pf_o, self.pf_m, self.pf_l, self.stream)

    def select_decode(self, t: int):
        """Fused select + swap lists + decode + combine; afterwards evicted is
        the other buffer."""
        w = self.w
        out = self.ev_bufs[1] if self.evicted is self.ev_bufs[0] else self.ev_bufs[0]
        nosa.nosa_select_decode(self.dims, self.kv, self.q(t), self.score_q, self.score_e, self.seq_lens, w.k_e,
                                w.k_q, self.evicted, out, self.sel, self.sel_count, self.prev, self.prev_count,
                                self.load, self.load_count, self.evict, self.evict_count, self.P, w.sm_scale,
                                self.part_o, self.part_m, self.part_l, self.counters, self.o, self.m, self.l,
                                self.stream)
        self.evicted = out

    def combine(self):
        nosa.nosa_combine(self.dims, self.P, self.part_o, self.part_m, self.part_l, self.o, self.m, self.l,
                          self.stream)

    # ------------------------------------------------------------------
    # checkpoint / resume of the state one step hands to the next
    def _state_tensors(self) -> dict:
        """The cross-step state: everything a later step reads that an
        earlier one wrote.  The eviction bitmap is the strict policy's memory
        (a block left out once never returns to the eviction part), the
        previous selection is what the swap lists are taken against, and the
        pages and summaries hold the appended tokens."""
        st = {"seq_lens": self.seq_lens, "evicted": self.evicted,
              "sel0": self.sel_bufs[0], "sel1": self.sel_bufs[1],
              "count0": self.cnt_bufs[0], "count1": self.cnt_bufs[1],
              "k_summary": self.k_summary, "e_summary": self.e_summary,
              "k_pages": self.k_pages, "v_pages": self.v_pages, "e_pages": self.e_pages}
        if self.offload:
            st.update(host_k=self.host_k, host_v=self.host_v, host_e=self.host_e, resident=self.resident,
                      slot_owner=self.slot_owner)
            if self.buffered:
                st["last_use"] = self.last_use
        return st

    def save_state(self, path: str):
        """Write the cross-step state after the last step to a safetensors
        file (host copies; the stream is synchronised first)."""
        from safetensors.torch import save_file
        torch.cuda.synchronize()
        tensors = {k: v.detach().cpu().contiguous() for k, v in self._state_tensors().items()}
        meta = {"workload": self.w.name, "step_index": str(self.step_index), "n_steps": str(self.n_steps),
                "buffer_clock": str(self.buffer_clock), "splits": str(self.P)}
        save_file(tensors, str(path), metadata=meta)

    def load_state(self, path: str):
        """Resume from a file written by save_state for the same workload
        and inputs: the next step() continues where that session stopped.
        The current length and bitmap go to the first of their two buffers."""
        from safetensors import safe_open
        with safe_open(str(path), framework="pt") as f:
            meta = f.metadata()
            if meta.get("workload") != self.w.name or int(meta["splits"]) != self.P:
                raise ValueError(f"state of {meta.get('workload')} at {meta.get('splits')} splits, "
                                 f"not {self.w.name} at {self.P}")
            self.seq_lens, self.evicted = self.seq_bufs[0], self.ev_bufs[0]
            own = self._state_tensors()
            if set(f.keys()) != set(own):
                raise ValueError(f"state holds {sorted(f.keys())}, this session {sorted(own)}")
            for k, dst in own.items():
                src = f.get_tensor(k)
                if src.shape != dst.shape or src.dtype != dst.dtype:
                    raise ValueError(f"state tensor {k}: {tuple(src.shape)} {src.dtype}, "
                                     f"expected {tuple(dst.shape)} {dst.dtype}")
                dst.copy_(src)
        self.step_index, self.n_steps = int(meta["step_index"]), int(meta["n_steps"])
        self.buffer_clock = int(meta["buffer_clock"])
        self.counters.zero_()
        torch.cuda.synchronize()

    # ------------------------------------------------------------------
    # the step as HIP graphs
    _GRAPH_INPUTS = ("q_all", "k_new", "v_new", "e_new")

    def _state(self) -> tuple:
        return (self.seq_lens, self.evicted, self.sel, self.sel_count, self.prev, self.prev_count)

    def _set_state(self, st: tuple):
        self.seq_lens, self.evicted, self.sel, self.sel_count, self.prev, self.prev_count = st

    def capture_graphs(self):
        """Capture the step as two HIP graphs, one for each parity of the
        step index: the ping-pong buffers (lengths, eviction bitmaps,
        selections) repeat every two steps.  The graphs read the step's
        inputs (query, new key / value / logit) from static buffers that
        graph_step(t) refills before each replay.  The plain HBM-tier step
        only (no host tier, softmax mass, ALiBi or QKV rows), on the current
        stream, after at least one eager step.  Its launches allocate nothing
        and record no memset."""
        if self.offload or self.mass_on or self.alibi_on or self.qkv_on or self.stream is not None:
            raise ValueError("graphs cover the plain HBM-tier step on the current stream")
        if self.step_index < 1:
            raise ValueError("run one eager step before capturing")
        names = [n for n in self._GRAPH_INPUTS if hasattr(self, n) and (n == "q_all" or self.w.append)]
        self._g_real = {n: getattr(self, n) for n in names}
        self._g_static = {n: torch.empty_like(t) for n, t in self._g_real.items()}
        start, t0, n0 = self._state(), self.step_index, self.n_steps
        self.graphs = []
        self._g_n0 = n0
        # workloads without appends repeat step 1 (their eviction bitmaps
        # still alternate); the others advance one token per step
        for t in ((t0 + 1, t0 + 2) if self.w.append else (1, 1)):
            for n in names:
                setattr(self, n, self._g_static[n])
            g = torch.cuda.CUDAGraph()
            try:
                with torch.cuda.graph(g):
                    self.step(t)
            finally:
                for n in names:
                    setattr(self, n, self._g_real[n])
            self.graphs.append((t, g, self._state()))
        if any(a is not b for a, b in zip(self._state(), start)):
            raise RuntimeError("the step's buffers do not repeat every two steps")
        self._set_state(start)
        self.step_index, self.n_steps = t0, n0

    def graph_step(self, t: int | None = None, replay: bool = True):
        """The next decode step (t: its index, the next one; workloads
        without appends repeat step 1) by replaying the captured graph whose
        buffers it uses: the step's inputs are copied into the graph's static
        buffers (stream order), then the graph runs.  replay=False stages the
        inputs and advances the state only; the caller then replays
        self.next_graph before any other step.  Eager steps may come in
        between: the graph is chosen by the number of steps run since the
        capture."""
        t = (self.step_index + 1 if self.w.append else 1) if t is None else t
        if self.w.append and t != self.step_index + 1:
            raise ValueError("graph steps run in order")
        gt, g, after = self.graphs[(self.n_steps - self._g_n0) % 2]
        for n, real in self._g_real.items():
            self._g_static[n][gt - 1].copy_(real[t - 1])
        self.next_graph = g
        if replay:
            g.replay()
        self.n_steps += 1
        self._set_state(after)
        self.step_index = t
        return t

    @property
    def runs_select_decode(self) -> bool:
        """Whether step() makes the selection and the decode in one launch
        (nosa_select_decode)."""
        return (self.fused and not self.offload and not self.w.select_all and self.select_decode_ok
                and not self.mass_on and not self.alibi_on)

    def use_buffers(self, t: int):
        """Point sel / prev at the buffers of step t."""
        if self.w.select_all:
            self.sel, self.sel_count = self.all_sel, self.all_count
            if t == 1:
                self.prev, self.prev_count = self.sel_bufs[0], self.cnt_bufs[0]  # still empty
            else:
                self.prev, self.prev_count = self.all_sel, self.all_count
        else:
            self.sel, self.sel_count = self.sel_bufs[t % 2], self.cnt_bufs[t % 2]
            self.prev, self.prev_count = self.sel_bufs[(t - 1) % 2], self.cnt_bufs[(t - 1) % 2]

    def step(self, t: int | None = None):
        """One whole decode step (all hot-path stages), enqueued on the stream."""
        t = self.step_index + 1 if t is None else t
        w = self.w
        self.use_buffers(t)
        if self.offload:
            self.append_score(t)
            self.select_swap()
            self.retrieve()
            self.decode_combine(t)
        elif self.fused:
            if w.select_all:
                if w.append:
                    self.append(t)
                self.swap_diff()
                self.decode_combine(t)
            elif self.runs_select_decode:
                self.append_score(t)
                self.select_decode(t)
            else:
                self.append_score(t)
                self.select_swap()
                self.decode_combine(t)
        else:
            if w.append:
                self.append(t)
            if not w.select_all:
                self.score(t)
                self.select()
            self.swap_diff()
            self.decode(t)
            self.combine()
        self.step_index = t
        self.n_steps += 1
        return t
