"""fp64 CPU oracle of the rank share with FP8 (E4M3) Q, K and V.

TEST INFRASTRUCTURE ONLY, under the same rules as pcp_oracle (imported only by
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg; shares no code
with the product).

Source: "[MRv2] FlashAttention PCP support for GQA on MRv2" (vLLM PR #49564),
review thread on the context-attention call: the FP8 descale tensors handed
to the varlen flash-attention call are shaped (number of sequences in the
call, number of KV heads); the benchmark sections run FP8 checkpoints
(Hy3-FP8, Qwen3-30B-A3B-FP8).

Readings (also listed in the design doc):

R13 Each descale is indexed by (request, KV head). A query of head h of
    request b is q_code * q_descale[b, h // G] (G = Hq / Hkv); every key and
    value of request b -- new tokens and cached prefix alike -- is
    k_code * k_descale[b, kvh], v_code * v_descale[b, kvh]. The attention is
    then exactly the bf16 rank share's definition applied to these dequantized
    values (a per-layer scalar scale, as FP8 checkpoints carry, is the special
    case of a constant table). Indexing by request rather than by row keeps a
    key's value the same for both rows of a request and on every rank.
R14 The codes are OCP 8-bit floating point E4M3 ("fn" variant): sign bit, 4
    exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes the
    subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities; the
    largest finite magnitude is 448.

The attention itself is pcp_oracle.rank_share on the dequantized float64
tensors; the functions here only decode and scale.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .pcp_oracle import F, rank_share, rank_share_resplit


def e4m3_to_float(codes) -> np.ndarray:
    """float64 values of E4M3 codes (reading R14), elementwise, any shape."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def token_requests(cu_seqlens: Sequence[int]) -> np.ndarray:
    """Request index of every token of a batch laid out by ``cu_seqlens``."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return np.repeat(np.arange(len(cu) - 1), np.diff(cu))


def query_requests(plan: np.ndarray) -> np.ndarray:
    """Request index of every rank-local query of a row plan."""
    total_q = int(plan[:, F["q_len"]].sum()) if len(plan) else 0
    req = np.empty(total_q, dtype=np.int64)
    for row in plan:
        qs, ql = int(row[F["q_start"]]), int(row[F["q_len"]])
        req[qs:qs + ql] = int(row[F["req"]])
    return req


def dequantize(codes, descale: np.ndarray, tok_req: np.ndarray, group: int) -> np.ndarray:
    """codes [T, H, d] (E4M3) -> float64 value * descale[tok_req[t], h // group]
    (reading R13; group = 1 for K and V, Hq / Hkv for Q)."""
    if hasattr(codes, "numpy"):
        codes = codes.numpy()
    x = e4m3_to_float(codes)
    ds = np.asarray(descale, dtype=np.float64)
    heads = np.arange(x.shape[1]) // group
    return x * ds[tok_req][:, heads][..., None]


def rank_share_fp8(q8_local, k8_new, v8_new, k8_cached, v8_cached, cu_seqlens_new,
                   cu_cache, plan: np.ndarray, q_descale, k_descale, v_descale,
                   dcp_size: int, dcp_rank: int, block_size: int, num_q_heads: int,
                   num_kv_heads: int, scale: float, query_ids=None):
    """The rank share (new-token pass, context pass over this DCP rank's
    shard, their LSE merge) of dequantized FP8 inputs. q8_local holds the
    rank-local query codes [total_q, Hq, d] in plan order; k8/v8 new and
    cached codes are laid out as in pcp_oracle.rank_share. Returns the same
    dict of (out, lse) pairs."""
    g = num_q_heads // num_kv_heads
    ql = dequantize(q8_local, q_descale, query_requests(plan), g)
    req_new = token_requests(cu_seqlens_new)
    req_cache = token_requests(cu_cache)
    kn = dequantize(k8_new, k_descale, req_new, 1)
    vn = dequantize(v8_new, v_descale, req_new, 1)
    kc = dequantize(k8_cached, k_descale, req_cache, 1)
    vc = dequantize(v8_cached, v_descale, req_cache, 1)
    return rank_share(ql, kn, vn, kc, vc, cu_cache, plan, dcp_size, dcp_rank, block_size,
                      num_q_heads, num_kv_heads, scale, query_ids=query_ids)


def rank_share_resplit_fp8(q8_local, k8_local, v8_local, k8_new, v8_new, cu_seqlens_new,
                           k8_cached, v8_cached, cu_cache, ctx_lens, plan: np.ndarray,
                           q_descale, k_descale, v_descale, dcp_size: int, dcp_rank: int,
                           block_size: int, num_q_heads: int, num_kv_heads: int, scale: float,
                           query_ids=None):
    """The re-split rank share (pcp_oracle.rank_share_resplit) of dequantized
    FP8 inputs. ``k8_local`` / ``v8_local`` are the rows' own tokens in the
    rank-local order of the queries, so they take the queries' requests; a
    token written to the cache keeps its request's descales (reading R13)."""
    g = num_q_heads // num_kv_heads
    req_q = query_requests(plan)
    req_new = token_requests(cu_seqlens_new)
    req_cache = token_requests(cu_cache)
    return rank_share_resplit(
        dequantize(q8_local, q_descale, req_q, g), dequantize(k8_local, k_descale, req_q, 1),
        dequantize(v8_local, v_descale, req_q, 1), dequantize(k8_new, k_descale, req_new, 1),
        dequantize(v8_new, v_descale, req_new, 1), cu_seqlens_new,
        dequantize(k8_cached, k_descale, req_cache, 1),
        dequantize(v8_cached, v_descale, req_cache, 1), cu_cache, ctx_lens, plan, dcp_size,
        dcp_rank, block_size, num_q_heads, num_kv_heads, scale, query_ids=query_ids)
