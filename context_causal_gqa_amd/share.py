"""Device buffers and the call sequence of one rank share.

``RankShare`` holds one rank's inputs in HBM (its query rows, the request's
all-gathered new-token K/V, this DCP rank's paged cache and block table) and
runs the hot path through the C ABI:

  1. ``pcp_plan_rows``           (host) the rank-local row plan
  2. ``pcp_attn_context_paged``  context pass over this DCP rank's cache shard
  3. ``pcp_attn_prefill``        end-aligned causal new-token pass
  4. ``lse_merge``               combine the two partials

or, in one launch, ``pcp_attn_rank_share`` (steps 2-4 fused; ``step_fused``).
With FP8 inputs the same steps call the ``_fp8`` entry points.

Every arithmetic step runs in libpcpattn; this module only moves tensors.
The query rows of the rank are gathered from natural-order queries with the
plan's own offsets when the buffers are set up (in a serving system they are
already local to the rank).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import (PASS_CONTEXT, PASS_FUSED, PASS_NEW_TOKENS, ROW_FIELDS, lse_merge,
               pcp_choose_decode_splits, pcp_attn_context_paged, pcp_attn_context_paged_fp8,
               pcp_attn_prefill, pcp_attn_prefill_fp8, pcp_attn_rank_share,
               pcp_attn_rank_share_fp8, pcp_attn_schedule, pcp_context_workspace_bytes,
               pcp_kv_cache_write, pcp_kv_cache_write_fp8, pcp_plan_rows, pcp_plan_rows_resplit,
               pcp_slot_mapping, plan_max_q_len)


def local_query_index(rows: np.ndarray, cu_seqlens_new, ctx_lens) -> np.ndarray:
    """Natural-order new-token index of every rank-local query, in plan order."""
    parts = []
    for r in rows:
        req, q_len, pos = int(r[0]), int(r[3]), int(r[4])
        first = int(cu_seqlens_new[req]) + pos - int(ctx_lens[req])
        parts.append(np.arange(first, first + q_len, dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _upload_descales(f, dev):
    """The (q, k, v) descale tables on the device. They are host arrays here,
    so the FP8 calls' contract -- every descale finite and > 0 -- is checked
    before upload (the C ABI cannot read device tables without a sync)."""
    import torch

    out = []
    for name in ("q_descale", "k_descale", "v_descale"):
        t = np.ascontiguousarray(getattr(f, name), dtype=np.float32)
        if not (np.isfinite(t).all() and (t > 0).all()):
            raise ValueError("%s: FP8 descales must be finite and > 0" % name)
        out.append(torch.from_numpy(t).to(dev))
    return tuple(out)


class RankShare:
    """One rank's share of a workload, resident in HBM.

    ``inputs`` is a ``pcp_workloads.Inputs``-like object with host tensors:
    cu_seqlens_new, ctx_lens, q [tot, Hq, d], k_new / v_new [tot, Hkv, d],
    k_pool / v_pool [blocks, bs, Hkv, d] and rank_block_tables.

    ``fp8`` (a ``pcp_workloads.Fp8Inputs``-like object: E4M3 codes q8,
    k8_new, v8_new, k8_pool, v8_pool and float32 [B, Hkv] descales) makes the
    share hold the codes instead of the bf16 tensors and run the FP8 calls.
    """

    def __init__(self, inputs, device="cuda", pcp_rank: Optional[int] = None,
                 dcp_rank: Optional[int] = None, q_full_device=None,
                 decode_splits: Optional[int] = None, schedule: bool = True, fp8=None):
        import torch

        w = inputs.workload
        self.device = torch.device(device)
        self.pcp_rank = w.pcp_rank if pcp_rank is None else pcp_rank
        self.dcp_rank = w.dcp_rank if dcp_rank is None else dcp_rank
        self.hq, self.hkv, self.d = w.num_q_heads, w.num_kv_heads, w.head_dim
        self.scale = w.softmax_scale
        self.rows_host = pcp_plan_rows(inputs.cu_seqlens_new, inputs.ctx_lens, w.pcp_size,
                                       self.pcp_rank, w.dcp_size, self.dcp_rank, w.block_size)
        self.num_rows = len(self.rows_host)
        self.max_q_len = plan_max_q_len(self.rows_host)
        self.qidx = local_query_index(self.rows_host, inputs.cu_seqlens_new, inputs.ctx_lens)
        self.total_q = len(self.qidx)
        dev = self.device
        self.rows = torch.from_numpy(np.ascontiguousarray(self.rows_host)).to(dev)
        self.fp8 = fp8 is not None
        src = fp8 if self.fp8 else inputs
        q_all, k_all, v_all, kp, vp = ((fp8.q8, fp8.k8_new, fp8.v8_new, fp8.k8_pool, fp8.v8_pool)
                                       if self.fp8 else
                                       (inputs.q, inputs.k_new, inputs.v_new, inputs.k_pool,
                                        inputs.v_pool))
        if q_full_device is not None:
            self.q = q_full_device.index_select(0, torch.from_numpy(self.qidx).to(dev)).contiguous()
        else:
            self.q = q_all[torch.from_numpy(self.qidx)].contiguous().to(dev)
        self.k = k_all.to(dev)
        self.v = v_all.to(dev)
        self.k_cache = kp.to(dev)
        self.v_cache = vp.to(dev)
        self.descales = ()
        if self.fp8:
            self.descales = _upload_descales(src, dev)
        self.block_tables = torch.from_numpy(inputs.rank_block_tables[self.dcp_rank]).to(dev)
        tq = self.total_q
        bf, f32 = torch.bfloat16, torch.float32
        self.out_new = torch.empty((tq, self.hq, self.d), dtype=bf, device=dev)
        self.lse_new = torch.empty((self.hq, tq), dtype=f32, device=dev)
        self.out_ctx = torch.empty((tq, self.hq, self.d), dtype=bf, device=dev)
        self.lse_ctx = torch.empty((self.hq, tq), dtype=f32, device=dev)
        self.out = torch.empty((tq, self.hq, self.d), dtype=bf, device=dev)
        self.lse = torch.empty((self.hq, tq), dtype=f32, device=dev)
        # decode rows: key-range splits of the context pass and of the fused
        # launch, and their scratch
        if decode_splits is None:
            self.decode_splits = pcp_choose_decode_splits(self.rows_host, self.hkv)
            self.decode_splits_fused = pcp_choose_decode_splits(self.rows_host, self.hkv,
                                                                fused=True)
        else:
            self.decode_splits = self.decode_splits_fused = int(decode_splits)
        ws_bytes = max(pcp_context_workspace_bytes(self.num_rows, self.hq, self.d, s)
                       for s in (self.decode_splits, self.decode_splits_fused))
        self.workspace = (torch.empty(ws_bytes // 4, dtype=f32, device=dev)
                          if ws_bytes else None)
        # launch orders of the passes (longest units first per XCD), made once per plan
        self.order_new = self.order_ctx = self.order_fused = None
        if schedule:
            geo = (self.max_q_len, self.hq, self.hkv, self.d)
            eb = 1 if self.fp8 else 2
            self.order_new = torch.from_numpy(pcp_attn_schedule(
                PASS_NEW_TOKENS, self.rows_host, *geo, kv_elem_bytes=eb)).to(dev)
            self.order_ctx = torch.from_numpy(pcp_attn_schedule(
                PASS_CONTEXT, self.rows_host, *geo, self.decode_splits, kv_elem_bytes=eb)).to(dev)
            self.order_fused = torch.from_numpy(pcp_attn_schedule(
                PASS_FUSED, self.rows_host, *geo, self.decode_splits_fused,
                kv_elem_bytes=eb)).to(dev)

    @property
    def rows_table(self) -> np.ndarray:
        return self.rows_host

    def context_pass(self, stream=None):
        fn = pcp_attn_context_paged_fp8 if self.fp8 else pcp_attn_context_paged
        fn(self.q, self.k_cache, self.v_cache, self.block_tables, self.rows, self.out_ctx,
           self.lse_ctx, self.scale, self.max_q_len, *self.descales, rows_host=self.rows_host,
           stream=stream, workspace=self.workspace, decode_splits=self.decode_splits,
           unit_order=self.order_ctx)

    def new_token_pass(self, stream=None):
        fn = pcp_attn_prefill_fp8 if self.fp8 else pcp_attn_prefill
        fn(self.q, self.k, self.v, self.rows, self.out_new, self.lse_new, self.scale,
           self.max_q_len, *self.descales, rows_host=self.rows_host, stream=stream,
           unit_order=self.order_new)

    def merge(self, stream=None):
        lse_merge([self.out_ctx, self.out_new], [self.lse_ctx, self.lse_new], self.out, self.lse,
                  stream=stream)

    def step(self, stream=None):
        """The whole hot path on the device: context pass, new-token pass, merge."""
        self.context_pass(stream)
        self.new_token_pass(stream)
        self.merge(stream)

    def step_fused(self, out=None, lse=None, stream=None):
        """The whole hot path in one launch (pcp_attn_rank_share) into ``out`` /
        ``lse`` (default: the same buffers ``step`` merges into)."""
        fn = pcp_attn_rank_share_fp8 if self.fp8 else pcp_attn_rank_share
        fn(self.q, self.k, self.v, self.k_cache, self.v_cache, self.block_tables, self.rows,
           self.out if out is None else out, self.lse if lse is None else lse, self.scale,
           self.max_q_len, *self.descales, rows_host=self.rows_host, stream=stream,
           workspace=self.workspace, decode_splits=self.decode_splits_fused,
           unit_order=self.order_fused)


class ResplitShare:
    """One rank's share on the re-split path, resident in HBM.

    Each prefill row attends over [0, row_start) read from this DCP rank's
    paged cache -- the cached prefix and every earlier new token, which the
    cache write puts there first -- plus its own new tokens, square causal
    (pcp_plan_rows_resplit). A step is

      1. ``pcp_kv_cache_write``   the all-gathered new K/V into the blocks this
                                  DCP rank owns (``pcp_slot_mapping``)
      2. ``pcp_attn_rank_share``  one launch: context tiles, then own tokens

    ``cache`` is a ``pcp_workloads.ResplitCache``-like object (global block
    table, pools holding the prefix, per-DCP-rank block tables); the pools
    are copied to the device, so several shares may be built from one cache.
    With ``fp8`` (E4M3 codes and descales, as for ``RankShare``) the cache
    pools hold codes too and the FP8 cache write and attention run.
    """

    def __init__(self, inputs, cache, device="cuda", pcp_rank: Optional[int] = None,
                 dcp_rank: Optional[int] = None, k_pool=None, v_pool=None,
                 decode_splits: Optional[int] = None, schedule: bool = True, fp8=None):
        import torch

        w = inputs.workload
        dev = self.device = torch.device(device)
        self.pcp_rank = w.pcp_rank if pcp_rank is None else pcp_rank
        self.dcp_rank = w.dcp_rank if dcp_rank is None else dcp_rank
        self.hq, self.hkv, self.d = w.num_q_heads, w.num_kv_heads, w.head_dim
        self.scale = w.softmax_scale
        cu, ctx = inputs.cu_seqlens_new, inputs.ctx_lens
        self.rows_host = pcp_plan_rows_resplit(cu, ctx, w.pcp_size, self.pcp_rank, w.dcp_size,
                                               self.dcp_rank, w.block_size)
        self.num_rows = len(self.rows_host)
        self.max_q_len = plan_max_q_len(self.rows_host)
        self.qidx = local_query_index(self.rows_host, cu, ctx)
        self.total_q = len(self.qidx)
        self.rows = torch.from_numpy(np.ascontiguousarray(self.rows_host)).to(dev)
        sel = torch.from_numpy(self.qidx)
        self.fp8 = fp8 is not None
        q_all, k_all, v_all = ((fp8.q8, fp8.k8_new, fp8.v8_new) if self.fp8 else
                               (inputs.q, inputs.k_new, inputs.v_new))
        # the rank's queries and its own tokens' K/V, in plan order
        self.q = q_all[sel].contiguous().to(dev)
        self.k_local = k_all[sel].contiguous().to(dev)
        self.v_local = v_all[sel].contiguous().to(dev)
        # every new token (as after the K/V all-gather) and where this rank writes it
        self.k_new = k_all.to(dev)
        self.v_new = v_all.to(dev)
        self.descales = ()
        if self.fp8:
            self.descales = _upload_descales(fp8, dev)
        self.slots_host = pcp_slot_mapping(cu, ctx, cache.block_table, w.dcp_size,
                                           self.dcp_rank, w.block_size)
        self.slots = torch.from_numpy(self.slots_host).to(dev)
        self.k_cache = cache.k_pool.to(dev) if k_pool is None else k_pool
        self.v_cache = cache.v_pool.to(dev) if v_pool is None else v_pool
        self.block_tables = torch.from_numpy(cache.rank_block_tables[self.dcp_rank]).to(dev)
        tq = self.total_q
        self.out = torch.empty((tq, self.hq, self.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.hq, tq), dtype=torch.float32, device=dev)
        if decode_splits is None:
            decode_splits = pcp_choose_decode_splits(self.rows_host, self.hkv, fused=True)
        self.decode_splits = int(decode_splits)
        ws = pcp_context_workspace_bytes(self.num_rows, self.hq, self.d, self.decode_splits)
        self.workspace = torch.empty(ws // 4, dtype=torch.float32, device=dev) if ws else None
        self.order = None
        if schedule:
            self.order = torch.from_numpy(pcp_attn_schedule(
                PASS_FUSED, self.rows_host, self.max_q_len, self.hq, self.hkv, self.d,
                self.decode_splits, kv_elem_bytes=1 if self.fp8 else 2)).to(dev)

    def cache_write(self, stream=None):
        fn = pcp_kv_cache_write_fp8 if self.fp8 else pcp_kv_cache_write
        fn(self.k_new, self.v_new, self.slots, self.k_cache, self.v_cache, stream=stream)

    def attend(self, out=None, lse=None, stream=None):
        fn = pcp_attn_rank_share_fp8 if self.fp8 else pcp_attn_rank_share
        fn(self.q, self.k_local, self.v_local, self.k_cache, self.v_cache, self.block_tables,
           self.rows, self.out if out is None else out, self.lse if lse is None else lse,
           self.scale, self.max_q_len, *self.descales, rows_host=self.rows_host, stream=stream,
           workspace=self.workspace, decode_splits=self.decode_splits, unit_order=self.order)

    def step(self, stream=None):
        """The cache write, then the attention of every row."""
        self.cache_write(stream)
        self.attend(stream=stream)


__all__ = ["RankShare", "ResplitShare", "local_query_index", "ROW_FIELDS"]
