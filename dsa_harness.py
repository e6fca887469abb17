"""Device-side workload setup for tests, smoke() and bench.py.

Uploads the seeded synthetic inputs of a dsa_synth.Workload, builds the INT8
latent cache and the pool cache through the library, allocates the step's
outputs and workspaces, and runs one decode/prefill step of the path:

  store_int8 (the step's new tokens) -> index_pools (pools those tokens
  complete) -> index_scores -> topk_select -> expand_selection -> sparse_mla

either as separate calls or with the last four in one dsa_decode_step launch.

This module only marshals data; every computation runs in libdsa's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

import dsa_synth as syn
import sparse_attention_store_amd as dsa


def _bits_to_bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(syn.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(device)


def _f32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class DeviceWorkload:
    """All device state of one workload (optionally R replicas of the caches)."""

    def __init__(self, wl: syn.Workload, device="cuda", replicas: int = 1, score_stride: int | None = None,
                 out_dtype=torch.float32, num_splits: int = 0, build: bool = True, gen_workers: int = 8,
                 canary: int | None = None, prefill_chunk: int = 512, pool_format: str = "bf16", share: int = 1):
        self.wl = wl
        self.share = share              # > 1: runs of consecutive queries of a sequence share the pool pass
        if pool_format not in ("bf16", "int8"):
            raise ValueError(pool_format)
        self.int8 = pool_format == "int8"
        self.prefill_chunk = prefill_chunk
        self.ws_chunk = None
        self.device = torch.device(device)
        d = wl.dims
        self.dims = dsa.Dims.of(d)
        dev = self.device
        self.num_splits = num_splits
        self.gen_workers = gen_workers
        self.seqs = dsa.Seqs(
            first_valid=torch.tensor(wl.first_valid, dtype=torch.int32, device=dev),
            row_base=torch.tensor(wl.row_base, dtype=torch.int64, device=dev),
            tok_base=torch.tensor(wl.tok_base, dtype=torch.int64, device=dev),
            pool_base=torch.tensor(wl.pool_base, dtype=torch.int64, device=dev))
        self.q_seq = torch.tensor(wl.q_seq, dtype=torch.int32, device=dev)
        self.q_pos = torch.tensor(wl.q_pos, dtype=torch.int32, device=dev)
        T = wl.T
        rows, toks, npools = wl.total_rows, wl.total_tokens, max(wl.total_pools, 1)
        fill = canary if canary is not None else 0
        self.caches = [torch.full((rows, d.row_bytes), fill, dtype=torch.int8, device=dev)
                       for _ in range(replicas)]
        if self.int8:
            # INT8 pool cache: code rows and one fp32 scale per pool
            self.pool_codes = [torch.zeros((npools, d.idx_dim), dtype=torch.int8, device=dev) for _ in range(replicas)]
            self.pool_scales = [torch.zeros(npools, dtype=torch.float32, device=dev) for _ in range(replicas)]
            self.pools = None
        else:
            self.pools = [torch.zeros((npools, d.idx_dim), dtype=torch.bfloat16, device=dev)
                          for _ in range(replicas)]
        self.k = torch.zeros((toks, d.idx_dim), dtype=torch.bfloat16, device=dev)
        self.gate = torch.zeros((toks, d.idx_dim), dtype=torch.bfloat16, device=dev)
        lw, lb = syn.gen_ln(wl)
        self.ln_w, self.ln_b = _f32(lw, dev), _f32(lb, dev)
        # Per-query inputs.
        self.q_idx = _bits_to_bf16(syn.gen_qidx(wl, 0, T), dev)
        self.w = _f32(syn.gen_w(wl, 0, T), dev)
        qv = syn.gen_q(wl, 0, T)
        self.q = _f32(qv, dev) if wl.fp32_mla else _bits_to_bf16(qv, dev)
        # The step's new tokens: the query positions themselves.
        lat = np.concatenate([syn.gen_latent(wl, int(b), int(x), int(x) + 1)
                              for b, x in zip(wl.q_seq, wl.q_pos)], axis=0) if T else \
            np.zeros((0, d.latent_dim), np.float32)
        self.latent_q = _f32(lat, dev) if wl.fp32_mla else _bits_to_bf16(lat, dev)
        self.slots_q = torch.tensor(wl.row_base[wl.q_seq] + wl.q_pos, dtype=torch.int64, device=dev)
        # Pools the step's tokens complete: pool p ends at position f + kpool*p + kpool - 1.
        pb, pe = [], []
        for b in range(wl.B):
            f = int(wl.first_valid[b])
            ends = [(int(x) - f + 1) // d.kpool for x in wl.q_pos[wl.q_seq == b]
                    if int(x) >= f and (int(x) - f + 1) % d.kpool == 0]
            if ends:
                pb.append(min(ends) - 1)
                pe.append(max(ends))
            else:
                pb.append(0)
                pe.append(0)
        self.step_pool_begin = torch.tensor(pb, dtype=torch.int32, device=dev)
        self.step_pool_end = torch.tensor(pe, dtype=torch.int32, device=dev)
        self.step_max_pools = max([e - s for s, e in zip(pb, pe)] + [0])
        # Outputs and workspaces.
        self.stride = score_stride or max(256, -(-max(wl.max_n_vis, 1) // 256) * 256)
        self.scores = torch.empty((T, self.stride), dtype=torch.float32, device=dev)
        self.pool_ids = torch.empty((T, d.select_k), dtype=torch.int32, device=dev)
        self.indices = torch.empty((T, d.out_width), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, d.mla_heads, d.latent_dim), dtype=out_dtype, device=dev)
        self.lse = torch.empty((T, d.mla_heads), dtype=torch.float32, device=dev)
        self.ws_topk = dsa.topk_workspace(self.dims, T, self.stride, device=dev)
        n = dsa.sparse_mla_workspace_bytes(self.dims, T, num_splits)
        self.ws_mla = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        self.ws_step = None
        self.ws_ss = None
        self._bound = {}
        if build:
            self.build_caches()

    # ------------------------------------------------------------------ setup
    def build_caches(self):
        """Store every position's INT8 row and build every complete pool (replica 0, then copies)."""
        wl, d, dev = self.wl, self.wl.dims, self.device
        cache = self.caches[0]
        for b in range(wl.B):
            n = int(wl.seq_len[b])
            rb, tb = int(wl.row_base[b]), int(wl.tok_base[b])
            for x0, lat in syn.gen_sequence_blocks(syn.gen_latent, wl, b, 0, n, workers=self.gen_workers):
                lt = _f32(lat, dev) if wl.fp32_mla else _bits_to_bf16(lat, dev)
                slots = torch.arange(rb + x0, rb + x0 + lat.shape[0], dtype=torch.int64, device=dev)
                dsa.store_int8(self.dims, lt, slots, cache)
            for x0, (k, g) in syn.gen_sequence_blocks(syn.gen_kgate, wl, b, 0, n, workers=self.gen_workers):
                self.k[tb + x0: tb + x0 + k.shape[0]] = _bits_to_bf16(k, dev)
                self.gate[tb + x0: tb + x0 + g.shape[0]] = _bits_to_bf16(g, dev)
        ends = [wl.n_pools(b) for b in range(wl.B)]
        if max(ends) > 0:
            begin = torch.zeros(wl.B, dtype=torch.int32, device=dev)
            end = torch.tensor(ends, dtype=torch.int32, device=dev)
            if self.int8:
                dsa.index_pools_int8(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs, begin, end,
                                     max(ends), self.pool_codes[0], self.pool_scales[0])
            else:
                dsa.index_pools(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs, begin, end,
                                max(ends), self.pools[0])
        for r in range(1, len(self.caches)):
            self.caches[r].copy_(cache)
            if self.int8:
                self.pool_codes[r].copy_(self.pool_codes[0])
                self.pool_scales[r].copy_(self.pool_scales[0])
            else:
                self.pools[r].copy_(self.pools[0])
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ the step
    # Every stage takes (r, prepare): with prepare=True it returns the prepared
    # call(s) of the binding instead of launching (see bound / run below).
    def step_store(self, r: int = 0, prepare: bool = False):
        return dsa.store_int8(self.dims, self.latent_q, self.slots_q, self.caches[r], prepare=prepare)

    def step_pools(self, r: int = 0, prepare: bool = False):
        if self.step_max_pools > 0 and self.int8:
            return dsa.index_pools_int8(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs,
                                        self.step_pool_begin, self.step_pool_end, self.step_max_pools,
                                        self.pool_codes[r], self.pool_scales[r], prepare=prepare)
        if self.step_max_pools > 0:
            return dsa.index_pools(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs,
                                   self.step_pool_begin, self.step_pool_end, self.step_max_pools, self.pools[r],
                                   prepare=prepare)
        return None

    def step_append(self, r: int = 0, prepare: bool = False):
        """The step's new tokens (INT8 rows and completed pools) in one launch
        (two calls when the latent rows and the indexer keys differ in dtype)."""
        if self.latent_q.dtype != self.k.dtype or self.int8:
            return [self.step_store(r, prepare), self.step_pools(r, prepare)]
        return dsa.append_tokens(self.dims, self.latent_q, self.slots_q, self.caches[r], self.k, self.gate,
                                 self.ln_w, self.ln_b, self.seqs, self.step_pool_begin, self.step_pool_end,
                                 self.step_max_pools, self.pools[r], prepare=prepare)

    def step_scores(self, r: int = 0, prepare: bool = False):
        if self.int8:
            return dsa.index_scores_int8(self.dims, self.q_idx, self.w, self.pool_codes[r], self.pool_scales[r],
                                         self.seqs, self.q_seq, self.q_pos, self.scores, prepare=prepare)
        return dsa.index_scores(self.dims, self.q_idx, self.w, self.pools[r], self.seqs, self.q_seq, self.q_pos,
                                self.scores, prepare=prepare)

    def step_topk(self, r: int = 0, prepare: bool = False):
        return dsa.topk_select(self.dims, self.scores, self.seqs, self.q_seq, self.q_pos, self.pool_ids,
                               self.ws_topk, prepare=prepare)

    def step_expand(self, r: int = 0, prepare: bool = False):
        return dsa.expand_selection(self.dims, self.pool_ids, self.seqs, self.q_seq, self.q_pos, self.indices,
                                    prepare=prepare)

    def step_attention(self, r: int = 0, prepare: bool = False):
        return dsa.sparse_mla(self.dims, self.q, self.caches[r], self.indices, self.wl.scale, self.out, self.lse,
                              self.num_splits, self.ws_mla, prepare=prepare)

    def _ws_ss(self):
        if self.ws_ss is None:
            self.ws_ss = dsa.index_scores_select_workspace(self.dims, self.wl.T, self.stride, device=self.device)
        return self.ws_ss

    def step_scores_groups(self, r: int = 0, prepare: bool = False):
        if self.int8:
            return dsa.index_scores_groups_int8(self.dims, self.q_idx, self.w, self.pool_codes[r],
                                                self.pool_scales[r], self.seqs, self.q_seq, self.q_pos, self.scores,
                                                self._ws_ss(), prepare=prepare)
        return dsa.index_scores_groups(self.dims, self.q_idx, self.w, self.pools[r], self.seqs, self.q_seq,
                                       self.q_pos, self.scores, self._ws_ss(), prepare=prepare)

    def step_append_scores(self, r: int = 0, prepare: bool = False):
        """The new tokens and the scoring pass with group lists (one launch for bf16 tokens)."""
        if self.share > 1:
            return dsa.append_scores_groups_shared(
                self.dims, self.latent_q, self.slots_q, self.caches[r], self.k, self.gate, self.ln_w, self.ln_b,
                self.step_pool_begin, self.step_pool_end, self.step_max_pools,
                self.pool_codes[r] if self.int8 else self.pools[r], self.pool_scales[r] if self.int8 else None,
                self.q_idx, self.w, self.seqs, self.q_seq, self.q_pos, self.scores, self._ws_ss(), self.share,
                prepare=prepare)
        if self.int8:
            return dsa.append_scores_groups_int8(self.dims, self.latent_q, self.slots_q, self.caches[r], self.k,
                                                 self.gate, self.ln_w, self.ln_b, self.step_pool_begin,
                                                 self.step_pool_end, self.step_max_pools, self.pool_codes[r],
                                                 self.pool_scales[r], self.q_idx, self.w, self.seqs, self.q_seq,
                                                 self.q_pos, self.scores, self._ws_ss(), prepare=prepare)
        if self.latent_q.dtype != self.k.dtype:
            return [self.step_store(r, prepare), self.step_pools(r, prepare), self.step_scores_groups(r, prepare)]
        return dsa.append_scores_groups(self.dims, self.latent_q, self.slots_q, self.caches[r], self.k, self.gate,
                                        self.ln_w, self.ln_b, self.step_pool_begin, self.step_pool_end,
                                        self.step_max_pools, self.pools[r], self.q_idx, self.w, self.seqs, self.q_seq,
                                        self.q_pos, self.scores, self._ws_ss(), prepare=prepare)

    def step_select_groups(self, r: int = 0, prepare: bool = False):
        return dsa.topk_select_groups(self.dims, self.scores, self.seqs, self.q_seq, self.q_pos, self.indices,
                                      self._ws_ss(), pool_ids=self.pool_ids, prepare=prepare)

    def step_select_attention(self, r: int = 0, prepare: bool = False):
        """Selection from the group lists, expansion and attention (dsa_topk_sparse_mla)."""
        return dsa.topk_sparse_mla(self.dims, self.scores, self.seqs, self.q_seq, self.q_pos, self.indices,
                                   self._ws_ss(), self.q, self.caches[r], self.wl.scale, self.out, self.lse,
                                   self.num_splits, self.ws_mla, pool_ids=self.pool_ids, prepare=prepare)

    def step_scores_select(self, r: int = 0, prepare: bool = False):
        """Scores, selection and expansion (dsa_index_scores_select: two launches for decode)."""
        if self.int8:
            return [self.step_scores_groups(r, prepare), self.step_select_groups(r, prepare)]
        return dsa.index_scores_select(self.dims, self.q_idx, self.w, self.pools[r], self.seqs, self.q_seq,
                                       self.q_pos, self.scores, self.indices, pool_ids=self.pool_ids,
                                       workspace=self._ws_ss(), prepare=prepare)

    def step_select(self, r: int = 0, prepare: bool = False):
        """Top-k and expansion in one launch (pool ids kept for the checks)."""
        return dsa.topk_select_expand(self.dims, self.scores, self.seqs, self.q_seq, self.q_pos, self.indices,
                                      self.pool_ids, self.ws_topk, prepare=prepare)

    def step_prefill_select(self, r: int = 0, prepare: bool = False):
        """Scores, top-k and expansion of every query, prefill_chunk queries at a
        time through a bounded scoring workspace (dsa_index_select_chunked)."""
        if self.ws_chunk is None:
            self.ws_chunk = dsa.index_select_chunked_workspace(self.dims, self.prefill_chunk, self.stride,
                                                               device=self.device)
        return dsa.index_select_chunked(self.dims, self.q_idx, self.w, self.pools[r], self.seqs, self.q_seq,
                                        self.q_pos, self.stride, self.prefill_chunk, self.indices, self.ws_chunk,
                                        pool_ids=self.pool_ids, prepare=prepare)

    def step_decode(self, r: int = 0, prepare: bool = False):
        """Scores, top-k, expansion and attention in one launch (dsa_decode_step)."""
        if self.ws_step is None:
            self.ws_step = dsa.decode_step_workspace(self.dims, self.wl.T, self.stride, device=self.device)
        return dsa.decode_step(self.dims, self.q_idx, self.w, self.pools[r], self.seqs, self.q_seq, self.q_pos,
                               self.stride, self.q, self.caches[r], self.wl.scale, self.out, self.ws_step,
                               lse=self.lse, pool_ids=self.pool_ids, indices=self.indices, prepare=prepare)

    def bound(self, stage: str, r: int = 0):
        """Stage `stage` (step_<stage>) of replica r as prepared calls: validated
        and converted once, then cached, so a timed loop pays one ctypes call
        per launch."""
        key = (stage, r)
        b = self._bound.get(key)
        if b is None:
            out = getattr(self, "step_" + stage)(r, prepare=True)
            b = tuple(x for x in (out if isinstance(out, list) else [out]) if x is not None)
            self._bound[key] = b
        return b

    def run(self, stage: str, r: int = 0):
        for call in self.bound(stage, r):
            call()

    # The launches bench.py times for a decode step (prepared calls): the new
    # tokens with the scoring pass and its group lists (dsa_append_scores_groups,
    # one launch), then the selection, expansion and attention
    # (dsa_topk_sparse_mla: k_select_mla, then the split merge).
    TIMED_STAGES = ("append_scores", "select_attention")

    def fast_supported(self) -> bool:
        """Group lists are kept for at most 64 queries of at most 262,144 pools
        (65,536 for shared runs)."""
        limit = 65536 if self.share > 1 else 262144
        return self.wl.T <= 64 and self.stride <= limit and self.wl.dims.idx_heads == 32 and \
            self.wl.dims.idx_dim == 128 and (not self.int8 or self.latent_q.dtype == torch.bfloat16)

    def step_fast(self, r: int = 0):
        """One decode step through exactly the launches the bench times."""
        for st in self.TIMED_STAGES:
            self.run(st, r)

    def timed_stages(self):
        """The stages bench.py times for this workload: the decode launches
        above when they apply; the new tokens, the chunked selection and the
        attention for many queries (prefill); else the general chain."""
        if self.fast_supported():
            return self.TIMED_STAGES
        if self.wl.T > 64:
            return ("append", "prefill_select", "attention")
        return ("append", "scores_select", "attention")

    def step_timed(self, r: int = 0):
        for st in self.timed_stages():
            self.run(st, r)

    def step_fused(self, r: int = 0):
        """One pass of the whole path: the new tokens, then the fused decode launch."""
        self.step_append(r)
        self.step_decode(r)

    def step(self, r: int = 0):
        """One pass of the whole path over replica r."""
        self.step_append(r)
        self.step_scores_select(r)
        self.step_attention(r)

    def step_calls(self, r: int = 0):
        """The same pass with scoring and selection as their own calls."""
        self.step_store(r)
        self.step_pools(r)
        self.step_scores(r)
        self.step_select()
        self.step_attention(r)

    def step_unfused(self, r: int = 0):
        """The same pass with top-k and expansion as separate calls."""
        self.step_store(r)
        self.step_pools(r)
        self.step_scores(r)
        self.step_topk()
        self.step_expand()
        self.step_attention(r)


class PagedWorkload:
    """The workload's caches in paged form: each sequence's positions in blocks
    of 256, the physical blocks a seeded permutation (with spare blocks that no
    sequence owns), built and stepped through the paged calls:

      store_int8 (physical slots) -> index_pools_paged -> index_scores_groups_paged
      -> topk_select_groups_paged -> sparse_mla

    This class only marshals data; every computation runs in libdsa."""

    def __init__(self, wl: syn.Workload, device="cuda", out_dtype=torch.float32, num_splits: int = 0,
                 spare_blocks: int = 3, seed: int = 5, gen_workers: int = 8):
        self.wl = wl
        d = wl.dims
        self.dims = dsa.Dims.of(d)
        dev = self.device = torch.device(device)
        self.num_splits = num_splits
        nblk = [max(1, -(-int(n) // 256)) for n in wl.seq_len]
        total = sum(nblk) + spare_blocks
        perm = np.random.default_rng(seed).permutation(total).astype(np.int32)
        table = np.full((wl.B, max(nblk)), perm[-1], dtype=np.int32)      # unused entries: a spare block
        off = 0
        for b, n in enumerate(nblk):
            table[b, :n] = perm[off:off + n]
            off += n
        self.table_np = table
        self.seqs = dsa.PagedSeqs(first_valid=torch.tensor(wl.first_valid, dtype=torch.int32, device=dev),
                                  block_table=torch.from_numpy(table).to(dev))
        self.q_seq = torch.tensor(wl.q_seq, dtype=torch.int32, device=dev)
        self.q_pos = torch.tensor(wl.q_pos, dtype=torch.int32, device=dev)
        T = wl.T
        self.cache = torch.full((total * 256, d.row_bytes), 0x11, dtype=torch.int8, device=dev)
        self.k = torch.zeros((total * 256, d.idx_dim), dtype=torch.bfloat16, device=dev)
        self.gate = torch.zeros((total * 256, d.idx_dim), dtype=torch.bfloat16, device=dev)
        self.pools = torch.zeros((total * 64, d.idx_dim), dtype=torch.bfloat16, device=dev)
        lw, lb = syn.gen_ln(wl)
        self.ln_w, self.ln_b = _f32(lw, dev), _f32(lb, dev)
        self.q_idx = _bits_to_bf16(syn.gen_qidx(wl, 0, T), dev)
        self.w = _f32(syn.gen_w(wl, 0, T), dev)
        self.q = _bits_to_bf16(syn.gen_q(wl, 0, T), dev)
        lat = np.concatenate([syn.gen_latent(wl, int(b), int(x), int(x) + 1) for b, x in zip(wl.q_seq, wl.q_pos)])
        self.latent_q = _bits_to_bf16(lat, dev)
        self.slots_q = torch.tensor([self.row(int(b), int(x)) for b, x in zip(wl.q_seq, wl.q_pos)], dtype=torch.int64,
                                    device=dev)
        pb, pe = [], []
        for b in range(wl.B):
            f = int(wl.first_valid[b])
            ends = [(int(x) - f + 1) // d.kpool for x in wl.q_pos[wl.q_seq == b]
                    if int(x) >= f and (int(x) - f + 1) % d.kpool == 0]
            pb.append(min(ends) - 1 if ends else 0)
            pe.append(max(ends) if ends else 0)
        self.step_pool_begin = torch.tensor(pb, dtype=torch.int32, device=dev)
        self.step_pool_end = torch.tensor(pe, dtype=torch.int32, device=dev)
        self.step_max_pools = max([e - s for s, e in zip(pb, pe)] + [0])
        self.stride = max(256, -(-max(wl.max_n_vis, 1) // 256) * 256)
        self.scores = torch.empty((T, self.stride), dtype=torch.float32, device=dev)
        self.pool_ids = torch.empty((T, d.select_k), dtype=torch.int32, device=dev)
        self.indices = torch.empty((T, d.out_width), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, d.mla_heads, d.latent_dim), dtype=out_dtype, device=dev)
        self.lse = torch.empty((T, d.mla_heads), dtype=torch.float32, device=dev)
        self.ws = dsa.index_scores_select_workspace(self.dims, T, self.stride, device=dev)
        n = dsa.sparse_mla_workspace_bytes(self.dims, T, num_splits)
        self.ws_mla = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        # caches: every position's INT8 row and indexer state at its physical row, then every pool
        for b in range(wl.B):
            n_b = int(wl.seq_len[b])
            for x0, lat_b in syn.gen_sequence_blocks(syn.gen_latent, wl, b, 0, n_b, workers=gen_workers):
                rows = torch.from_numpy(self.rows(b, np.arange(x0, x0 + lat_b.shape[0]))).to(dev)
                dsa.store_int8(self.dims, _bits_to_bf16(lat_b, dev), rows, self.cache)
            for x0, (kk, gg) in syn.gen_sequence_blocks(syn.gen_kgate, wl, b, 0, n_b, workers=gen_workers):
                rows = torch.from_numpy(self.rows(b, np.arange(x0, x0 + kk.shape[0]))).to(dev)
                self.k[rows] = _bits_to_bf16(kk, dev)
                self.gate[rows] = _bits_to_bf16(gg, dev)
        ends = [wl.n_pools(b) for b in range(wl.B)]
        if max(ends) > 0:
            dsa.index_pools_paged(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs,
                                  torch.zeros(wl.B, dtype=torch.int32, device=dev),
                                  torch.tensor(ends, dtype=torch.int32, device=dev), max(ends), self.pools)
        torch.cuda.synchronize()

    def row(self, b: int, x: int) -> int:
        return int(self.table_np[b, x >> 8]) * 256 + (x & 255)

    def rows(self, b: int, xs: np.ndarray) -> np.ndarray:
        xs = np.asarray(xs, dtype=np.int64)
        return self.table_np[b, xs >> 8].astype(np.int64) * 256 + (xs & 255)

    def step(self):
        """One decode step through the paged calls."""
        dsa.store_int8(self.dims, self.latent_q, self.slots_q, self.cache)
        if self.step_max_pools > 0:
            dsa.index_pools_paged(self.dims, self.k, self.gate, self.ln_w, self.ln_b, self.seqs, self.step_pool_begin,
                                  self.step_pool_end, self.step_max_pools, self.pools)
        dsa.index_scores_groups_paged(self.dims, self.q_idx, self.w, self.pools, self.seqs, self.q_seq, self.q_pos,
                                      self.scores, self.ws)
        dsa.topk_select_groups_paged(self.dims, self.scores, self.seqs, self.q_seq, self.q_pos, self.indices, self.ws,
                                     pool_ids=self.pool_ids)
        dsa.sparse_mla(self.dims, self.q, self.cache, self.indices, self.wl.scale, self.out, self.lse,
                       self.num_splits, self.ws_mla)
