"""Seeded synthetic workloads for one prefill-context-parallel (PCP) rank's share
of causal grouped-query attention.

This module only draws random numbers and lays them out in memory. It holds no
attention, row-plan or merge arithmetic, so both the HIP path and the fp64
oracle can take their inputs from it without sharing any of the method.

What it produces, per workload:

* the batch: per-request new-token counts (the scheduled prompt tokens that are
  split across PCP ranks) and cached-prefix lengths (tokens already in the
  paged KV cache);
* Q for every new token of every request, in natural order
  ``[sum(new), Hq, d]``, and the new tokens' K/V ``[sum(new), Hkv, d]`` in natural
  order, i.e. as they stand after the K/V all-gather across PCP ranks
  ("Feat/pcp qwen36 hybrid", Changes: full-attention layers all-gather K/V);
* the cached prefix of each request in natural order ``[sum(cached), Hkv, d]``,
  and the same values scattered into a paged pool ``[num_blocks, bs, Hkv, d]``
  through a randomly permuted block table. A decode request's own token is the
  last cached token: the cache write happens before attention runs
  ("[MRv2][PCP] Carry the row plan ...", "What made it removable").
* per decode-context-parallel (DCP) rank, that rank's block table: the rank
  keeps every ``dcp_size``-th logical block of each request, starting at block
  ``dcp_rank``, in logical order. This is how a DCP-sharded KV cache is laid
  out; the consumer of the table never needs to know the rule.

Values are fp32 standard normal rounded to bf16 (round-to-nearest-even, done by
torch). Slots of the pool that hold no token, and a few spare blocks, are NaN,
so that any read outside the valid context poisons the result.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    """Shape and structure of one rank-share workload."""

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    pcp_size: int
    pcp_rank: int
    dcp_size: int
    dcp_rank: int
    block_size: int
    # Fixed lengths (used when the draw below is None).
    new_lens: tuple = ()
    ctx_lens: tuple = ()
    # Random-length recipe: (num_prefill, new_lo, new_hi, ctx_lo, ctx_hi,
    # num_decode, dec_ctx_lo, dec_ctx_hi), all bounds inclusive. Decode context
    # counts the decode token itself.
    draw: Optional[tuple] = None
    description: str = ""

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="tiny_t512_pcp2_r0",
            seed=1,
            num_q_heads=4,
            num_kv_heads=2,
            head_dim=64,
            pcp_size=2,
            pcp_rank=0,
            dcp_size=1,
            dcp_rank=0,
            block_size=16,
            new_lens=(512,),
            ctx_lens=(0,),
            description="1 request of 512 tokens, pcp=2 zigzag (4 chunks of 128), rank 0; "
            "4 Q / 2 KV heads, d=64; no cached prefix",
        ),
        Workload(
            name="qwen3_0p6b_8x4096_pcp2_r1",
            seed=2,
            num_q_heads=16,
            num_kv_heads=8,
            head_dim=128,
            pcp_size=2,
            pcp_rank=1,
            dcp_size=1,
            dcp_rank=0,
            block_size=16,
            new_lens=(4096,) * 8,
            ctx_lens=(0,) * 8,
            description="Qwen3-0.6B-shaped layer (16 Q / 8 KV heads, d=128); 8 requests x 4096 "
            "tokens, pcp=2, rank 1 (16 rows of 1024); no cached prefix",
        ),
        Workload(
            name="mixed_pcp2_dcp2_8prefill_4decode",
            seed=3,
            num_q_heads=16,
            num_kv_heads=8,
            head_dim=128,
            pcp_size=2,
            pcp_rank=0,
            dcp_size=2,
            dcp_rank=0,
            block_size=16,
            draw=(8, 1024, 8192, 0, 4096, 4, 512, 8192),
            description="mixed batch, pcp=2 dcp=2, rank 0: 8 prefill requests with new lengths "
            "U[1024,8192] and cached prefixes U[0,4096], plus 4 decode requests with "
            "context U[512,8192]; paged bf16 cache, block 16, permuted; 16 Q / 8 KV heads, d=128",
        ),
        Workload(
            name="hybrid_fullattn_128k_pcp4_r1",
            seed=4,
            num_q_heads=8,
            num_kv_heads=1,
            head_dim=256,
            pcp_size=4,
            pcp_rank=1,
            dcp_size=1,
            dcp_rank=0,
            block_size=16,
            new_lens=(131072,),
            ctx_lens=(0,),
            description="hybrid-model full-attention layer, per-GPU head share 8 Q / 1 KV, d=256; "
            "1 request of 131072 tokens, pcp=4 (8 chunks of 16384), rank 1 (32768 query rows)",
        ),
        Workload(
            name="hybrid_fullattn_256k_ctx64k_pcp4_dcp4_r3",
            seed=5,
            num_q_heads=8,
            num_kv_heads=1,
            head_dim=256,
            pcp_size=4,
            pcp_rank=3,
            dcp_size=4,
            dcp_rank=3,
            block_size=16,
            new_lens=(262144,),
            ctx_lens=(65536,),
            description="same layer, 262144 new tokens after a 65536-token cached prefix "
            "(4096 blocks of 16, sharded 4 ways); pcp=4 dcp=4, rank 3 (65536 query rows)",
        ),
    ]
}


def scaled_workload(base: Workload, name: str, new_lens, ctx_lens, **overrides) -> Workload:
    """A copy of ``base`` with other lengths (used for small parity cases)."""
    fields = dict(base.__dict__)
    fields.update(name=name, new_lens=tuple(int(x) for x in new_lens),
                  ctx_lens=tuple(int(x) for x in ctx_lens), draw=None)
    fields.update(overrides)
    return Workload(**fields)


@dataclass
class Inputs:
    """Host-side tensors of one workload (torch CPU tensors; bf16 for activations)."""

    workload: Workload
    new_lens: np.ndarray  # int64 [B]
    ctx_lens: np.ndarray  # int64 [B]: tokens before the new ones (num computed)
    is_decode: np.ndarray  # bool [B]
    cu_seqlens_new: np.ndarray  # int32 [B+1]
    q: torch.Tensor  # bf16 [sum(new), Hq, d]
    k_new: torch.Tensor  # bf16 [sum(new), Hkv, d]
    v_new: torch.Tensor
    cache_lens: np.ndarray  # int64 [B]: tokens held in the paged cache per request
    cu_cache: np.ndarray  # int64 [B+1]
    k_cached: torch.Tensor  # bf16 [sum(cache_lens), Hkv, d], natural order
    v_cached: torch.Tensor
    k_pool: torch.Tensor  # bf16 [num_blocks, bs, Hkv, d]
    v_pool: torch.Tensor
    block_table: np.ndarray  # int32 [B, max_blocks]: logical block -> pool block, -1 unused
    rank_block_tables: Dict[int, np.ndarray] = field(default_factory=dict)


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _normal(rng: np.random.Generator, shape) -> torch.Tensor:
    return _bf16(rng.standard_normal(size=shape, dtype=np.float32))


def draw_lengths(w: Workload, rng: np.random.Generator):
    """Per-request new-token and cached-prefix lengths, and the decode flags."""
    if w.draw is None:
        new = np.asarray(w.new_lens, dtype=np.int64)
        ctx = np.asarray(w.ctx_lens, dtype=np.int64)
        dec = new == 1
        return new, ctx, dec
    npre, nlo, nhi, clo, chi, ndec, dlo, dhi = w.draw
    new_p = rng.integers(nlo, nhi, size=npre, endpoint=True)
    ctx_p = rng.integers(clo, chi, size=npre, endpoint=True)
    dec_total = rng.integers(dlo, dhi, size=ndec, endpoint=True)
    new = np.concatenate([new_p, np.ones(ndec, dtype=np.int64)])
    # A decode request has computed every context token but its own.
    ctx = np.concatenate([ctx_p, dec_total - 1])
    dec = np.concatenate([np.zeros(npre, dtype=bool), np.ones(ndec, dtype=bool)])
    return new.astype(np.int64), ctx.astype(np.int64), dec


def generate(w: Workload, spare_blocks: int = 4) -> Inputs:
    """Draw every input of ``w`` from ``numpy.random.default_rng(w.seed)``.

    Order of draws: lengths, Q, K_new, V_new, cached K, cached V, block permutation.
    """
    rng = np.random.default_rng(w.seed)
    hq, hkv, d, bs = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    new, ctx, dec = draw_lengths(w, rng)
    b = len(new)
    cu_new = np.zeros(b + 1, dtype=np.int64)
    cu_new[1:] = np.cumsum(new)
    tot_new = int(cu_new[-1])

    q = _normal(rng, (tot_new, hq, d))
    k_new = _normal(rng, (tot_new, hkv, d))
    v_new = _normal(rng, (tot_new, hkv, d))

    # The paged cache holds the computed prefix; for a decode request also the
    # decode token itself (written before attention).
    cache_lens = ctx + dec.astype(np.int64)
    cu_cache = np.zeros(b + 1, dtype=np.int64)
    cu_cache[1:] = np.cumsum(cache_lens)
    tot_cache = int(cu_cache[-1])
    k_cached = _normal(rng, (tot_cache, hkv, d))
    v_cached = _normal(rng, (tot_cache, hkv, d))
    for i in np.nonzero(dec)[0]:
        last = int(cu_cache[i + 1]) - 1
        k_cached[last] = k_new[int(cu_new[i])]
        v_cached[last] = v_new[int(cu_new[i])]

    nblk = [(int(c) + bs - 1) // bs for c in cache_lens]
    total_blocks = sum(nblk) + spare_blocks
    perm = rng.permutation(total_blocks).astype(np.int64)
    max_blocks = max(nblk) if nblk else 0
    table = np.full((b, max(max_blocks, 1)), -1, dtype=np.int32)
    k_pool = torch.full((total_blocks, bs, hkv, d), float("nan"), dtype=torch.bfloat16)
    v_pool = torch.full((total_blocks, bs, hkv, d), float("nan"), dtype=torch.bfloat16)
    nxt = 0
    for i in range(b):
        base = int(cu_cache[i])
        for j in range(nblk[i]):
            phys = int(perm[nxt])
            nxt += 1
            table[i, j] = phys
            lo = j * bs
            hi = min(int(cache_lens[i]), lo + bs)
            k_pool[phys, : hi - lo] = k_cached[base + lo: base + hi]
            v_pool[phys, : hi - lo] = v_cached[base + lo: base + hi]

    inp = Inputs(
        workload=w,
        new_lens=new,
        ctx_lens=ctx,
        is_decode=dec,
        cu_seqlens_new=cu_new.astype(np.int32),
        q=q,
        k_new=k_new,
        v_new=v_new,
        cache_lens=cache_lens,
        cu_cache=cu_cache,
        k_cached=k_cached,
        v_cached=v_cached,
        k_pool=k_pool,
        v_pool=v_pool,
        block_table=table,
    )
    for r in range(w.dcp_size):
        inp.rank_block_tables[r] = rank_block_table(table, w.dcp_size, r)
    return inp


@dataclass
class ResplitCache:
    """Paged cache laid out for the re-split path: every request owns blocks
    for all of its positions (cached prefix and new tokens); the prefix is
    filled, the new positions hold NaN until the cache write."""

    block_table: np.ndarray  # int32 [B, max_blocks], all logical blocks of each request
    k_pool: torch.Tensor  # bf16 [num_blocks, block_size, Hkv, d]
    v_pool: torch.Tensor
    rank_block_tables: dict = field(default_factory=dict)  # DCP rank -> int32 [B, cols]


def resplit_cache(inp: "Inputs", spare_blocks: int = 3) -> ResplitCache:
    """A paged cache with room for each request's ctx + new tokens, the
    cached prefix (``inp.k_cached``, first ctx_lens[b] tokens) written into
    seeded, permuted blocks. Deterministic in the workload's seed."""
    w = inp.workload
    bs = w.block_size
    rng = np.random.default_rng(w.seed + 7919)
    b = len(inp.new_lens)
    spans = [int(c) + int(n) for c, n in zip(inp.ctx_lens, inp.new_lens)]
    nblk = [(x + bs - 1) // bs for x in spans]
    total_blocks = sum(nblk) + spare_blocks
    perm = rng.permutation(total_blocks).astype(np.int64)
    table = np.full((b, max(max(nblk) if nblk else 0, 1)), -1, dtype=np.int32)
    hkv, d = inp.k_new.shape[1], inp.k_new.shape[2]
    k_pool = torch.full((total_blocks, bs, hkv, d), float("nan"), dtype=torch.bfloat16)
    v_pool = torch.full((total_blocks, bs, hkv, d), float("nan"), dtype=torch.bfloat16)
    nxt = 0
    for i in range(b):
        base = int(inp.cu_cache[i])
        c = int(inp.ctx_lens[i])
        for j in range(nblk[i]):
            phys = int(perm[nxt])
            nxt += 1
            table[i, j] = phys
            lo, hi = j * bs, min(c, j * bs + bs)
            if hi > lo:
                k_pool[phys, : hi - lo] = inp.k_cached[base + lo: base + hi]
                v_pool[phys, : hi - lo] = inp.v_cached[base + lo: base + hi]
    out = ResplitCache(block_table=table, k_pool=k_pool, v_pool=v_pool)
    for r in range(w.dcp_size):
        out.rank_block_tables[r] = rank_block_table(table, w.dcp_size, r)
    return out


E4M3_MAX = 448.0  # largest finite E4M3 ("fn") magnitude


@dataclass
class Fp8Inputs:
    """FP8 (E4M3) versions of a workload's Q/K/V with their descales.

    Codes are uint8 torch CPU tensors in the bf16 tensors' layouts; the pools
    keep the bf16 pools' block mapping and hold the NaN code 0x7F where no
    token lives. Descales are float32 [B, Hkv]: a value is code * descale of
    its (request, KV head) -- for a query, of the KV head its head reads."""

    q8: torch.Tensor  # [sum(new), Hq, d]
    k8_new: torch.Tensor  # [sum(new), Hkv, d]
    v8_new: torch.Tensor
    k8_cached: torch.Tensor  # [sum(cache_lens), Hkv, d]
    v8_cached: torch.Tensor
    k8_pool: torch.Tensor  # [num_blocks, bs, Hkv, d]
    v8_pool: torch.Tensor
    q_descale: np.ndarray  # float32 [B, Hkv]
    k_descale: np.ndarray
    v_descale: np.ndarray


def _to_e4m3(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """x / scale rounded to E4M3 codes (torch's cast, round to nearest even)."""
    y = (x.float() / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_fp8(inp: "Inputs") -> Fp8Inputs:
    """Per-tensor-style FP8 quantisation of ``inp`` at (request, KV head)
    granularity: descale = amax / 448 over the request's tokens of that KV
    head (Q: the query heads reading it; K, V: new and cached tokens
    together, so a decode token's new and cached codes agree)."""
    w = inp.workload
    b = len(inp.new_lens)
    hkv, g = w.num_kv_heads, w.num_q_heads // w.num_kv_heads
    cu_new, cu_c = inp.cu_seqlens_new.astype(np.int64), inp.cu_cache
    q_ds = np.ones((b, hkv), dtype=np.float32)
    k_ds = np.ones((b, hkv), dtype=np.float32)
    v_ds = np.ones((b, hkv), dtype=np.float32)
    q8 = torch.empty(inp.q.shape, dtype=torch.uint8)
    k8n = torch.empty(inp.k_new.shape, dtype=torch.uint8)
    v8n = torch.empty(inp.v_new.shape, dtype=torch.uint8)
    k8c = torch.empty(inp.k_cached.shape, dtype=torch.uint8)
    v8c = torch.empty(inp.v_cached.shape, dtype=torch.uint8)
    for i in range(b):
        n0, n1, c0, c1 = int(cu_new[i]), int(cu_new[i + 1]), int(cu_c[i]), int(cu_c[i + 1])
        for h in range(hkv):
            qs = inp.q[n0:n1, h * g:(h + 1) * g]
            amax = float(qs.float().abs().max()) if n1 > n0 else 0.0
            q_ds[i, h] = amax / E4M3_MAX if amax > 0 else 1.0
            q8[n0:n1, h * g:(h + 1) * g] = _to_e4m3(qs, torch.tensor(q_ds[i, h]))
            for src_n, src_c, dst_n, dst_c, ds in ((inp.k_new, inp.k_cached, k8n, k8c, k_ds),
                                                   (inp.v_new, inp.v_cached, v8n, v8c, v_ds)):
                parts = [src_n[n0:n1, h].float().abs(), src_c[c0:c1, h].float().abs()]
                amax = max([float(p.max()) for p in parts if p.numel()] + [0.0])
                ds[i, h] = amax / E4M3_MAX if amax > 0 else 1.0
                sc = torch.tensor(ds[i, h])
                dst_n[n0:n1, h] = _to_e4m3(src_n[n0:n1, h], sc)
                dst_c[c0:c1, h] = _to_e4m3(src_c[c0:c1, h], sc)
    nan_code = 0x7F
    k8p = torch.full(inp.k_pool.shape, nan_code, dtype=torch.uint8)
    v8p = torch.full(inp.v_pool.shape, nan_code, dtype=torch.uint8)
    bs = w.block_size
    for i in range(b):
        base, n = int(cu_c[i]), int(inp.cache_lens[i])
        for j in range((n + bs - 1) // bs):
            phys = int(inp.block_table[i, j])
            lo, hi = j * bs, min(n, j * bs + bs)
            k8p[phys, : hi - lo] = k8c[base + lo: base + hi]
            v8p[phys, : hi - lo] = v8c[base + lo: base + hi]
    return Fp8Inputs(q8=q8, k8_new=k8n, v8_new=v8n, k8_cached=k8c, v8_cached=v8c, k8_pool=k8p,
                     v8_pool=v8p, q_descale=q_ds, k_descale=k_ds, v_descale=v_ds)


def resplit_cache_fp8(inp: "Inputs", cache: ResplitCache, f: Fp8Inputs) -> ResplitCache:
    """``cache`` with E4M3 pools: the same blocks hold the cached prefix's
    codes (``f.k8_cached`` / ``f.v8_cached``); every other slot holds the NaN
    code 0x7F until the cache write."""
    bs = inp.workload.block_size
    k8 = torch.full(cache.k_pool.shape, 0x7F, dtype=torch.uint8)
    v8 = torch.full(cache.v_pool.shape, 0x7F, dtype=torch.uint8)
    for i in range(len(inp.new_lens)):
        base, c = int(inp.cu_cache[i]), int(inp.ctx_lens[i])
        for j in range((c + bs - 1) // bs):
            phys = int(cache.block_table[i, j])
            lo, hi = j * bs, min(c, j * bs + bs)
            k8[phys, : hi - lo] = f.k8_cached[base + lo: base + hi]
            v8[phys, : hi - lo] = f.v8_cached[base + lo: base + hi]
    return ResplitCache(block_table=cache.block_table, k_pool=k8, v_pool=v8,
                        rank_block_tables=dict(cache.rank_block_tables))


def rank_block_table(table: np.ndarray, dcp_size: int, dcp_rank: int) -> np.ndarray:
    """Block table of one DCP rank's cache: every ``dcp_size``-th logical block,
    starting at ``dcp_rank``, in logical order (-1 where unused)."""
    sub = table[:, dcp_rank::dcp_size]
    if sub.shape[1] == 0:
        sub = np.full((table.shape[0], 1), -1, dtype=np.int32)
    return np.ascontiguousarray(sub, dtype=np.int32)


def random_batch(rng: np.random.Generator, max_requests: int = 8, max_new: int = 300,
                 max_ctx: int = 200, p_decode: float = 0.25):
    """Random (new_lens, ctx_lens) for plan and small parity cases.

    Includes empty requests, single-token (decode) requests and lengths that
    are not multiples of anything."""
    b = int(rng.integers(1, max_requests + 1))
    new = []
    ctx = []
    for _ in range(b):
        u = rng.random()
        if u < p_decode:
            new.append(1)
        elif u < p_decode + 0.05:
            new.append(0)
        else:
            new.append(int(rng.integers(2, max_new + 1)))
        ctx.append(int(rng.integers(0, max_ctx + 1)) if rng.random() < 0.7 else 0)
    return np.asarray(new, dtype=np.int64), np.asarray(ctx, dtype=np.int64)
