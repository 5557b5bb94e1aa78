"""fp64 CPU oracle for one prefill-context-parallel rank's share of causal GQA attention.

TEST INFRASTRUCTURE ONLY. It may be imported, called or executed only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The product (``context_causal_gqa_amd``) never imports it and it
imports nothing from the product; the two share no code. Inputs reach both
sides from the seeded generator ``pcp_workloads``, which holds no part of the
method.

Everything here is the plain definition of the computation, in float64 numpy,
written to be checked by eye against the pages:

* "Feat/pcp qwen36 hybrid" (vllm-plugin-FL PR #299), section Changes: each PCP
  rank holds a slice of the prompt, full-attention layers all-gather K/V and run
  causal attention whose mask is aligned to the end of the key range.
* "[MRv2] FlashAttention PCP support for GQA on MRv2" (vLLM PR #49564), pull
  request overview and review thread: an optional attention pass over the
  sharded cached prefix that returns (out, lse), mixed prefill + decode
  batches, and an LSE combine of partial results over cache shards
  (benchmark section on Qwen3-30B-A3B-FP8: the per-step LSE-combine collective).
* "[MRv2][PCP] Carry the row plan in attention metadata; fix mixed
  prefill+decode crash" (fork PR #2): section "Two things that fell out of
  (1)" -- a rank-local batch holds up to two rows per prefilling request;
  comment on commit 97aad2056e -- decode rows are replicated across PCP ranks;
  "What made it removable" -- DualChunkSwap gives each rank a different row
  set, cached context of a row is everything before it, and the cache write
  happens before attention.

Readings taken where the pages are silent (each is also listed in the design doc):

R1  The zigzag (DualChunkSwap) split cuts the *new* tokens of a request into
    2P chunks; rank r owns chunk r (head) and chunk 2P-1-r (tail). When 2P does
    not divide N, chunk c holds floor(N/2P) + [c < N mod 2P] tokens.
R2  A request with exactly one new token is a decode row: it appears on every
    PCP rank, its token's K/V already sits in the paged cache, so it attends
    only to the cache (C+1 tokens, itself included) and its new-token pass is
    empty.
R3  DCP ownership: logical cache block j of a request lives on DCP rank
    j mod D.
R4  LSE is the natural log of the softmax denominator, stored [Hq, total_q].
R5  GQA: query head h reads KV head h // (Hq / Hkv).
R6  An empty key set gives out = 0 and LSE = -inf; merging with it is the
    identity.
R12 Re-split rows ("[MRv2][PCP] Carry the row plan ...", "What made it
    removable"): once the new tokens are written to the cache, a row's context
    is every position before its first query, [0, pos_start), read from this
    DCP rank's cache shard, and its new-token part is its own tokens only,
    square causal. The cache write masks every token whose block this DCP
    rank does not own (slot -1) and the writer skips those; the gathered list
    holds each token once, so a decode token is written by its block's owner
    like any other.

Parity pins: every function below is pinned by CPU tests against closed forms,
brute force, torch's SDPA and hand-derived plan fixtures (tests/golden/).
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

KIND_HEAD, KIND_TAIL, KIND_DECODE = 0, 1, 2
ROW_FIELDS = (
    "req",
    "kind",
    "q_start",
    "q_len",
    "pos_start",
    "k_start",
    "k_len",
    "ctx_len",
    "ctx_len_local",
)
F = {name: i for i, name in enumerate(ROW_FIELDS)}


# --------------------------------------------------------------------------
# Row plan
# --------------------------------------------------------------------------


def zigzag_chunks(n_new: int, pcp_size: int) -> List[Tuple[int, int]]:
    """[start, end) of the 2P chunks of a request's new tokens (reading R1)."""
    n_chunks = 2 * pcp_size
    base, rem = divmod(int(n_new), n_chunks)
    bounds = []
    start = 0
    for c in range(n_chunks):
        size = base + (1 if c < rem else 0)
        bounds.append((start, start + size))
        start += size
    assert start == n_new
    return bounds


def owned_cached_positions(cache_len: int, dcp_size: int, dcp_rank: int,
                           block_size: int) -> np.ndarray:
    """Positions of a request's cached tokens that DCP rank ``dcp_rank`` holds
    (reading R3: block j of the cache lives on rank j mod D)."""
    pos = np.arange(int(cache_len), dtype=np.int64)
    return pos[(pos // block_size) % dcp_size == dcp_rank]


def plan_rows(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int], pcp_size: int,
              pcp_rank: int, dcp_size: int, dcp_rank: int, block_size: int) -> np.ndarray:
    """Rank-local row plan, int64 [R, 9] with columns ``ROW_FIELDS``.

    Rows come in batch order; within a prefill request the head chunk precedes
    the tail chunk. ``q_start`` is the running sum of ``q_len`` (the row's
    offset into the rank-local query buffer). ``k_start`` is the request's
    offset in the all-gathered new-token K/V; ``k_len`` counts the new keys
    visible to the row's last query (the chunk end); ``ctx_len`` counts cached
    tokens visible to every query of the row; ``ctx_len_local`` the part of
    those held by this DCP rank.
    """
    cu = [int(x) for x in cu_seqlens_new]
    rows = []
    q_start = 0
    for b in range(len(cu) - 1):
        n_new = cu[b + 1] - cu[b]
        ctx = int(ctx_lens[b])
        if n_new == 0:
            continue
        if n_new == 1:  # decode row, reading R2
            cache_len = ctx + 1
            local = len(owned_cached_positions(cache_len, dcp_size, dcp_rank, block_size))
            rows.append((b, KIND_DECODE, q_start, 1, ctx, cu[b], 0, cache_len, local))
            q_start += 1
            continue
        chunks = zigzag_chunks(n_new, pcp_size)
        local = len(owned_cached_positions(ctx, dcp_size, dcp_rank, block_size))
        for kind, c in ((KIND_HEAD, pcp_rank), (KIND_TAIL, 2 * pcp_size - 1 - pcp_rank)):
            lo, hi = chunks[c]
            if hi == lo:
                continue
            rows.append((b, kind, q_start, hi - lo, ctx + lo, cu[b], hi, ctx, local))
            q_start += hi - lo
    return np.asarray(rows, dtype=np.int64).reshape(-1, len(ROW_FIELDS))


def row_new_token_offset(row: np.ndarray, ctx_lens: Sequence[int]) -> int:
    """Index, among its request's new tokens, of the row's first query."""
    return int(row[F["pos_start"]]) - int(ctx_lens[int(row[F["req"]])])


def gather_local_queries(q_full: np.ndarray, cu_seqlens_new: Sequence[int],
                         ctx_lens: Sequence[int], plan: np.ndarray) -> np.ndarray:
    """Rank-local query buffer: the plan's rows, in plan order, taken from the
    natural-order queries of every new token."""
    total_q = int(plan[:, F["q_len"]].sum()) if len(plan) else 0
    out = np.empty((total_q,) + q_full.shape[1:], dtype=q_full.dtype)
    for row in plan:
        b = int(row[F["req"]])
        off = int(cu_seqlens_new[b]) + row_new_token_offset(row, ctx_lens)
        qs, ql = int(row[F["q_start"]]), int(row[F["q_len"]])
        out[qs:qs + ql] = q_full[off:off + ql]
    return out


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray,
                      scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """out[i] = sum_j softmax_j(scale * q_i . k_j) v_j over the keys j with
    visible[i, j]; lse[i] = log sum_j exp(scale * q_i . k_j). A query that sees
    no key gets (0, -inf) (reading R6). q [m, d], k and v [n, d], visible
    [m, n] bool; float64 throughout."""
    m = q.shape[0]
    out = np.zeros((m, v.shape[1]), dtype=np.float64)
    lse = np.full(m, -np.inf, dtype=np.float64)
    if k.shape[0] == 0 or m == 0:
        return out, lse
    s = scale * (q @ k.T)
    s = np.where(visible, s, -np.inf)
    has = visible.any(axis=1)
    row_max = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.exp(s - row_max[:, None])
    denom = p.sum(axis=1)
    out[has] = (p[has] @ v) / denom[has, None]
    lse[has] = row_max[has] + np.log(denom[has])
    return out, lse


def _as64(x) -> np.ndarray:
    """float64 numpy copy of an array or torch tensor (bf16 upcasts exactly)."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _rows_of_queries(plan: np.ndarray, query_ids: np.ndarray):
    """Map rank-local query indices to (row index, t within row)."""
    starts = plan[:, F["q_start"]]
    ridx = np.searchsorted(starts, query_ids, side="right") - 1
    t = query_ids - starts[ridx]
    assert np.all(t < plan[ridx, F["q_len"]])
    return ridx, t


def new_token_pass(q_local, k_new, v_new, plan: np.ndarray, num_q_heads: int,
                   num_kv_heads: int, scale: float, query_ids=None, query_block: int = 256):
    """Attention of the plan's queries over their request's new-token keys with
    end-aligned causal masking ("Feat/pcp qwen36 hybrid", Changes): query t of a
    row with q_len m and k_len n sees new keys 0 .. n - m + t.

    Returns out [len(ids), Hq, d] and lse [Hq, len(ids)] (float64) for the
    rank-local query indices ``query_ids`` (all queries when None)."""
    q_local, k_new, v_new = _as64(q_local), _as64(k_new), _as64(v_new)
    total_q = q_local.shape[0]
    ids = np.arange(total_q) if query_ids is None else np.asarray(query_ids, dtype=np.int64)
    g = num_q_heads // num_kv_heads
    d = v_new.shape[-1]
    out = np.zeros((len(ids), num_q_heads, d))
    lse = np.full((num_q_heads, len(ids)), -np.inf)
    if len(ids) == 0:
        return out, lse
    ridx, tq = _rows_of_queries(plan, ids)
    for r in np.unique(ridx):
        row = plan[r]
        m, n, k0 = int(row[F["q_len"]]), int(row[F["k_len"]]), int(row[F["k_start"]])
        sel = np.nonzero(ridx == r)[0]
        for b0 in range(0, len(sel), query_block):
            part = sel[b0:b0 + query_block]
            t = tq[part]
            nvis = int(min(n, max(0, n - m + int(t.max()) + 1)))
            if nvis == 0:
                continue
            j = np.arange(nvis)
            visible = j[None, :] <= (n - m + t)[:, None]
            for h in range(num_q_heads):
                kvh = h // g
                o, l = softmax_attention(q_local[ids[part], h], k_new[k0:k0 + nvis, kvh],
                                         v_new[k0:k0 + nvis, kvh], visible, scale)
                out[part, h] = o
                lse[h, part] = l
    return out, lse


def context_pass(q_local, k_cached, v_cached, cu_cache: Sequence[int], plan: np.ndarray,
                 dcp_size: int, dcp_rank: int, block_size: int, num_q_heads: int,
                 num_kv_heads: int, scale: float, query_ids=None, query_block: int = 256):
    """Attention of the plan's queries over the cached tokens of their request
    that DCP rank ``dcp_rank`` holds ("[MRv2] FlashAttention PCP support for GQA
    on MRv2", overview: sharded cached-prefix attention returning (out, lse)).
    Every cached position precedes every new one, so no mask applies beyond
    the shard. ``k_cached``/``v_cached`` hold each request's cache in natural
    order, request b at rows cu_cache[b] ..; the row's ``ctx_len`` says how many
    of them its queries see."""
    q_local, k_cached, v_cached = _as64(q_local), _as64(k_cached), _as64(v_cached)
    total_q = q_local.shape[0]
    ids = np.arange(total_q) if query_ids is None else np.asarray(query_ids, dtype=np.int64)
    g = num_q_heads // num_kv_heads
    d = v_cached.shape[-1]
    out = np.zeros((len(ids), num_q_heads, d))
    lse = np.full((num_q_heads, len(ids)), -np.inf)
    if len(ids) == 0:
        return out, lse
    ridx, _ = _rows_of_queries(plan, ids)
    for r in np.unique(ridx):
        row = plan[r]
        b = int(row[F["req"]])
        pos = owned_cached_positions(int(row[F["ctx_len"]]), dcp_size, dcp_rank, block_size)
        if len(pos) == 0:
            continue
        rows_k = int(cu_cache[b]) + pos
        sel = np.nonzero(ridx == r)[0]
        for b0 in range(0, len(sel), query_block):
            part = sel[b0:b0 + query_block]
            visible = np.ones((len(part), len(pos)), dtype=bool)
            for h in range(num_q_heads):
                kvh = h // g
                o, l = softmax_attention(q_local[ids[part], h], k_cached[rows_k, kvh],
                                         v_cached[rows_k, kvh], visible, scale)
                out[part, h] = o
                lse[h, part] = l
    return out, lse


def lse_merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Combine partial results over disjoint key sets ("[MRv2] FlashAttention
    PCP support for GQA on MRv2", Qwen3-30B-A3B-FP8 benchmark: LSE combine of
    DCP partials). Each part is (out [N, Hq, d], lse [Hq, N]). With
    M = max_i lse_i: w_i = exp(lse_i - M), lse = M + log sum_i w_i,
    out = sum_i w_i out_i / sum_i w_i; when every lse_i is -inf the result is
    (0, -inf)."""
    outs = np.stack([_as64(o) for o, _ in parts])  # [k, N, Hq, d]
    lses = np.stack([_as64(l) for _, l in parts])  # [k, Hq, N]
    mx = lses.max(axis=0)  # [Hq, N]
    empty = np.isneginf(mx)
    mx_safe = np.where(empty, 0.0, mx)
    w = np.exp(lses - mx_safe[None])  # exp(-inf) = 0
    wsum = w.sum(axis=0)
    wsum_safe = np.where(empty, 1.0, wsum)
    wt = np.transpose(w / wsum_safe[None], (0, 2, 1))[..., None]  # [k, N, Hq, 1]
    out = (wt * outs).sum(axis=0)
    lse = np.where(empty, -np.inf, mx_safe + np.log(wsum_safe))
    out[np.transpose(empty)] = 0.0
    return out, lse


def rank_share(q_local, k_new, v_new, k_cached, v_cached, cu_cache, plan: np.ndarray,
               dcp_size: int, dcp_rank: int, block_size: int, num_q_heads: int,
               num_kv_heads: int, scale: float, query_ids=None):
    """One rank's share: new-token pass, context pass over this DCP rank's
    shard, and their LSE merge. Returns dict of the three (out, lse) pairs."""
    new = new_token_pass(q_local, k_new, v_new, plan, num_q_heads, num_kv_heads, scale,
                         query_ids=query_ids)
    ctx = context_pass(q_local, k_cached, v_cached, cu_cache, plan, dcp_size, dcp_rank,
                       block_size, num_q_heads, num_kv_heads, scale, query_ids=query_ids)
    merged = lse_merge([ctx, new])
    return {"new": new, "ctx": ctx, "merged": merged}


# --------------------------------------------------------------------------
# Re-split rows: cache write, then [0, row_start) from the cache + own tokens
# --------------------------------------------------------------------------


def plan_rows_resplit(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int], pcp_size: int,
                      pcp_rank: int, dcp_size: int, dcp_rank: int,
                      block_size: int) -> np.ndarray:
    """Row plan of the re-split path (reading R12): the same rows as
    ``plan_rows``; a prefill row's context is [0, pos_start) (cached prefix
    and earlier new tokens, all in the cache after the write) and its
    new-token keys are its own q_len tokens, which sit in the rank-local K/V
    buffer at the row's own q_start. Decode rows are unchanged."""
    plan = plan_rows(cu_seqlens_new, ctx_lens, pcp_size, pcp_rank, dcp_size, dcp_rank,
                     block_size).copy()
    for row in plan:
        if row[F["kind"]] == KIND_DECODE:
            row[F["k_start"]] = row[F["q_start"]]
            continue
        row[F["k_start"]] = row[F["q_start"]]
        row[F["k_len"]] = row[F["q_len"]]
        row[F["ctx_len"]] = row[F["pos_start"]]
        row[F["ctx_len_local"]] = len(owned_cached_positions(int(row[F["pos_start"]]), dcp_size,
                                                             dcp_rank, block_size))
    return plan


def slot_mapping(cu_seqlens_new: Sequence[int], ctx_lens: Sequence[int],
                 block_table: np.ndarray, dcp_size: int, dcp_rank: int,
                 block_size: int) -> np.ndarray:
    """Cache slot of every new token (natural order), or -1 where this DCP
    rank must not write (reading R12): token i of request b sits at position
    p = ctx_lens[b] + i, in logical block j = p // block_size, which DCP rank
    j mod D owns; its slot is block_table[b, j] * block_size + p % block_size
    (``block_table`` maps a request's logical blocks to pool blocks)."""
    cu = [int(x) for x in cu_seqlens_new]
    out = np.full(cu[-1], -1, dtype=np.int64)
    for b in range(len(cu) - 1):
        for i in range(cu[b + 1] - cu[b]):
            p = int(ctx_lens[b]) + i
            j = p // block_size
            if j % dcp_size == dcp_rank:
                out[cu[b] + i] = int(block_table[b, j]) * block_size + p % block_size
    return out


def kv_cache_write(k_new, v_new, slots: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray):
    """Write token t's K and V to slot ``slots[t]`` of the pools
    ([num_blocks, block_size, Hkv, d], flattened over the first two axes);
    negative slots are skipped. Returns new pools (float64)."""
    kp = _as64(k_pool).copy()
    vp = _as64(v_pool).copy()
    nb, bs = kp.shape[0], kp.shape[1]
    kf = kp.reshape(nb * bs, *kp.shape[2:])
    vf = vp.reshape(nb * bs, *vp.shape[2:])
    k64, v64 = _as64(k_new), _as64(v_new)
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s >= 0:
            kf[s] = k64[t]
            vf[s] = v64[t]
    return kp, vp


def context_pass_resplit(q_local, k_new, v_new, cu_seqlens_new, k_cached, v_cached,
                         cu_cache, ctx_lens, plan: np.ndarray, dcp_size: int, dcp_rank: int,
                         block_size: int, num_q_heads: int, num_kv_heads: int, scale: float,
                         query_ids=None, query_block: int = 256):
    """Context pass of re-split rows: each query attends, unmasked, over the
    positions below its row's ctx_len that this DCP rank holds. Position p of
    request b is cached token p (p < ctx_lens[b]) or new token p - ctx_lens[b]
    -- the cache content after the write."""
    q_local = _as64(q_local)
    k_new, v_new, k_cached, v_cached = _as64(k_new), _as64(v_new), _as64(k_cached), _as64(v_cached)
    total_q = q_local.shape[0]
    ids = np.arange(total_q) if query_ids is None else np.asarray(query_ids, dtype=np.int64)
    g = num_q_heads // num_kv_heads
    d = v_new.shape[-1]
    out = np.zeros((len(ids), num_q_heads, d))
    lse = np.full((num_q_heads, len(ids)), -np.inf)
    if len(ids) == 0:
        return out, lse
    ridx, _ = _rows_of_queries(plan, ids)
    for r in np.unique(ridx):
        row = plan[r]
        b = int(row[F["req"]])
        c = int(ctx_lens[b])
        pos = owned_cached_positions(int(row[F["ctx_len"]]), dcp_size, dcp_rank, block_size)
        if len(pos) == 0:
            continue
        from_cache = pos < c
        keys = np.empty((len(pos),) + k_new.shape[1:])
        vals = np.empty_like(keys)
        keys[from_cache] = k_cached[int(cu_cache[b]) + pos[from_cache]]
        vals[from_cache] = v_cached[int(cu_cache[b]) + pos[from_cache]]
        new_idx = int(cu_seqlens_new[b]) + pos[~from_cache] - c
        keys[~from_cache] = k_new[new_idx]
        vals[~from_cache] = v_new[new_idx]
        sel = np.nonzero(ridx == r)[0]
        for b0 in range(0, len(sel), query_block):
            part = sel[b0:b0 + query_block]
            visible = np.ones((len(part), len(pos)), dtype=bool)
            for h in range(num_q_heads):
                kvh = h // g
                o, l = softmax_attention(q_local[ids[part], h], keys[:, kvh], vals[:, kvh],
                                         visible, scale)
                out[part, h] = o
                lse[h, part] = l
    return out, lse


def rank_share_resplit(q_local, k_local, v_local, k_new, v_new, cu_seqlens_new, k_cached,
                       v_cached, cu_cache, ctx_lens, plan: np.ndarray, dcp_size: int,
                       dcp_rank: int, block_size: int, num_q_heads: int, num_kv_heads: int,
                       scale: float, query_ids=None):
    """One rank's share on the re-split path: the own-token pass (the row's
    own K/V, ``k_local``/``v_local`` in the rank-local order of the queries,
    square causal), the context pass over this DCP rank's shard of
    [0, row_start), and their LSE merge."""
    own = new_token_pass(q_local, k_local, v_local, plan, num_q_heads, num_kv_heads, scale,
                         query_ids=query_ids)
    ctx = context_pass_resplit(q_local, k_new, v_new, cu_seqlens_new, k_cached, v_cached,
                               cu_cache, ctx_lens, plan, dcp_size, dcp_rank, block_size,
                               num_q_heads, num_kv_heads, scale, query_ids=query_ids)
    return {"new": own, "ctx": ctx, "merged": lse_merge([ctx, own])}


def reassemble_resplit(q_full, k_new, v_new, k_cached, v_cached, cu_seqlens_new, ctx_lens,
                       cu_cache, pcp_size: int, dcp_size: int, block_size: int,
                       num_q_heads: int, num_kv_heads: int, scale: float):
    """Re-split path over every PCP rank and DCP shard, scattered back to
    natural order: each rank's own-token pass merged with the context passes
    of all shards. Returns (out, lse, seen) as ``reassemble_all_ranks``."""
    cu = np.asarray(cu_seqlens_new, dtype=np.int64)
    tot = int(cu[-1])
    d = _as64(v_new).shape[-1]
    out = np.zeros((tot, num_q_heads, d))
    lse = np.full((num_q_heads, tot), -np.inf)
    seen = np.zeros(tot, dtype=np.int64)
    q64, k64, v64 = _as64(q_full), _as64(k_new), _as64(v_new)
    for r in range(pcp_size):
        plan = plan_rows_resplit(cu, ctx_lens, pcp_size, r, dcp_size, 0, block_size)
        if len(plan) == 0:
            continue
        q_local = gather_local_queries(q64, cu, ctx_lens, plan)
        k_local = gather_local_queries(k64, cu, ctx_lens, plan)
        v_local = gather_local_queries(v64, cu, ctx_lens, plan)
        parts = [new_token_pass(q_local, k_local, v_local, plan, num_q_heads, num_kv_heads,
                                scale)]
        for rd in range(dcp_size):
            parts.append(context_pass_resplit(q_local, k64, v64, cu, k_cached, v_cached,
                                              cu_cache, ctx_lens, plan, dcp_size, rd,
                                              block_size, num_q_heads, num_kv_heads, scale))
        o, l = lse_merge(parts)
        for row in plan:
            b = int(row[F["req"]])
            off = int(cu[b]) + row_new_token_offset(row, ctx_lens)
            qs, ql = int(row[F["q_start"]]), int(row[F["q_len"]])
            out[off:off + ql] = o[qs:qs + ql]
            lse[:, off:off + ql] = l[:, qs:qs + ql]
            seen[off:off + ql] += 1
    return out, lse, seen


# --------------------------------------------------------------------------
# Unsplit reference and reassembly
# --------------------------------------------------------------------------


def full_causal_attention(q_full, k_new, v_new, k_cached, v_cached, cu_seqlens_new,
                          ctx_lens, cu_cache, num_q_heads: int, num_kv_heads: int,
                          scale: float, token_ids=None):
    """Unsplit causal attention of every new token: new token i of request b
    sits at position ctx_lens[b] + i and sees the first ctx_lens[b] cached
    tokens and new tokens 0..i. Returns out [len(ids), Hq, d] and lse
    [Hq, len(ids)] for natural-order new-token indices ``token_ids``."""
    q_full, k_new, v_new = _as64(q_full), _as64(k_new), _as64(v_new)
    k_cached, v_cached = _as64(k_cached), _as64(v_cached)
    cu = np.asarray(cu_seqlens_new, dtype=np.int64)
    tot = int(cu[-1])
    ids = np.arange(tot) if token_ids is None else np.asarray(token_ids, dtype=np.int64)
    g = num_q_heads // num_kv_heads
    d = v_new.shape[-1]
    out = np.zeros((len(ids), num_q_heads, d))
    lse = np.full((num_q_heads, len(ids)), -np.inf)
    req = np.searchsorted(cu, ids, side="right") - 1
    for b in np.unique(req):
        sel = np.nonzero(req == b)[0]
        c = int(ctx_lens[b])
        cb = int(cu_cache[b])
        keys = np.concatenate([k_cached[cb:cb + c], k_new[cu[b]:cu[b + 1]]])
        vals = np.concatenate([v_cached[cb:cb + c], v_new[cu[b]:cu[b + 1]]])
        i = ids[sel] - cu[b]
        visible = np.arange(keys.shape[0])[None, :] <= (c + i)[:, None]
        for h in range(num_q_heads):
            o, l = softmax_attention(q_full[ids[sel], h], keys[:, h // g], vals[:, h // g],
                                     visible, scale)
            out[sel, h] = o
            lse[h, sel] = l
    return out, lse


def reassemble_all_ranks(q_full, k_new, v_new, k_cached, v_cached, cu_seqlens_new,
                         ctx_lens, cu_cache, pcp_size: int, dcp_size: int, block_size: int,
                         num_q_heads: int, num_kv_heads: int, scale: float):
    """Every PCP rank's rows, each merged over its new-token pass and the
    context passes of all DCP shards, scattered back to natural order.

    Returns (out [tot, Hq, d], lse [Hq, tot], seen [tot] int) where ``seen``
    counts how many ranks produced each token (1 for prefill tokens, pcp_size
    for decode tokens, which every rank evaluates; reading R2)."""
    cu = np.asarray(cu_seqlens_new, dtype=np.int64)
    tot = int(cu[-1])
    d = _as64(v_new).shape[-1]
    out = np.zeros((tot, num_q_heads, d))
    lse = np.full((num_q_heads, tot), -np.inf)
    seen = np.zeros(tot, dtype=np.int64)
    q64 = _as64(q_full)
    for r in range(pcp_size):
        plan = plan_rows(cu, ctx_lens, pcp_size, r, dcp_size, 0, block_size)
        if len(plan) == 0:
            continue
        q_local = gather_local_queries(q64, cu, ctx_lens, plan)
        parts = [new_token_pass(q_local, k_new, v_new, plan, num_q_heads, num_kv_heads, scale)]
        for rd in range(dcp_size):
            parts.append(context_pass(q_local, k_cached, v_cached, cu_cache, plan, dcp_size, rd,
                                      block_size, num_q_heads, num_kv_heads, scale))
        o, l = lse_merge(parts)
        for row in plan:
            b = int(row[F["req"]])
            off = int(cu[b]) + row_new_token_offset(row, ctx_lens)
            qs, ql = int(row[F["q_start"]]), int(row[F["q_len"]])
            out[off:off + ql] = o[qs:qs + ql]
            lse[:, off:off + ql] = l[:, qs:qs + ql]
            seen[off:off + ql] += 1
    return out, lse, seen


# --------------------------------------------------------------------------
# Work accounting (used for FLOP counts)
# --------------------------------------------------------------------------


def visible_pairs(plan: np.ndarray) -> Tuple[int, int]:
    """(new-token pairs, context pairs) of a plan: the number of (query, key)
    pairs each pass attends over, per query head."""
    new = 0
    ctx = 0
    for row in plan:
        m, n = int(row[F["q_len"]]), int(row[F["k_len"]])
        for_t = np.clip(n - m + np.arange(m) + 1, 0, n)
        new += int(for_t.sum())
        ctx += m * int(row[F["ctx_len_local"]])
    return new, ctx


def causal_flops(plan: np.ndarray, num_q_heads: int, head_dim: int) -> int:
    """Useful FLOPs of a rank share: 2 * d for QK^T plus 2 * d for PV per
    visible pair and query head."""
    new, ctx = visible_pairs(plan)
    return 4 * head_dim * num_q_heads * (new + ctx)

