// gfx950 C-ABI entry points of the attention passes with FP8 (E4M3) Q, K and
// V and per-(request, KV head) descales.
//
// "[MRv2] FlashAttention PCP support for GQA on MRv2" (vLLM PR #49564),
// review thread on the context-attention call: the FP8 descales of the varlen
// attention call are shaped (sequences, KV heads); the pages' benchmarks run
// FP8 checkpoints (Hy3-FP8, Qwen3-30B-A3B-FP8). Reading: a descale is indexed
// by (request, KV head); a query of head h uses its KV head h / (Hq / Hkv);
// every key and value of a request, new or cached, uses the request's K and
// V descales of its KV head.
//
// The kernels are the bf16 ones (pcp_attn_fwd.h) with E4M3 tiles: QK^T runs
// on v_mfma_f32_32x32x64_f8f6f4 straight from the codes, with q_descale *
// k_descale folded into the softmax scale; V^T is widened to bf16 (exactly)
// as it is read and PV stays a bf16 MFMA with P in bf16, v_descale applied
// to O at the end. Rounding P to E4M3 as well would double the PV rate but
// puts errors of several 1e-2 on short rows, beyond the output tolerance.

#include "pcp_attn_fwd.h"

namespace {

// Descale tables must be given (and 4-byte aligned) whenever a row may name a
// request; Q/K/V are read 16 bytes at a time.
int check_fp8(const void* q, const void* k, const void* v, const void* kc, const void* vc,
              const float* qd, const float* kd, const float* vd) {
  if (!qd || !kd || !vd) return PCP_EINVAL;
  if (((uintptr_t)qd | (uintptr_t)kd | (uintptr_t)vd) & 3) return PCP_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)kc | (uintptr_t)vc) & 15)
    return PCP_EINVAL;
  return PCP_OK;
}

}  // namespace

extern "C" int pcp_attn_prefill_fp8(const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v,
                                    const pcp_row_t* rows, int num_rows, int total_q,
                                    int total_k, int max_q_len, int num_reqs, int num_q_heads,
                                    int num_kv_heads, int head_dim, float softmax_scale,
                                    const float* q_descale, const float* k_descale,
                                    const float* v_descale, pcp_bf16_t* out, float* lse,
                                    const int32_t* unit_order, int num_units,
                                    hipStream_t stream) {
  if (num_rows < 0 || total_q < 0 || total_k < 0 || max_q_len < 0 || num_reqs < 0)
    return PCP_EINVAL;
  if (unit_order != nullptr && num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim, softmax_scale);
  if (rc != PCP_OK) return rc;
  if (num_rows == 0 || max_q_len == 0 || total_q == 0) return PCP_OK;
  if (!q || !rows || !out || !lse || num_reqs < 1) return PCP_EINVAL;
  if (total_k > 0 && (!k || !v)) return PCP_EINVAL;
  const int rf = check_fp8(q, k, v, nullptr, nullptr, q_descale, k_descale, v_descale);
  if (rf != PCP_OK) return rf;
  // K/V rows are fetched with 32-bit buffer offsets.
  if ((uint64_t)total_k * num_kv_heads * head_dim > 0xFFFFFFFFull) return PCP_EUNSUPPORTED;
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_ds = q_descale;
  a.k_ds = k_descale;
  a.v_ds = v_descale;
  a.rows = rows;
  a.out = out;
  a.lse = lse;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.total_k = total_k;
  a.num_reqs = num_reqs;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale_log2 = softmax_scale * kLog2e;
  a.order = unit_order;
  return dispatch_attn<true>(a, kNewTokens, head_dim, max_q_len, num_units, stream);
}

extern "C" int pcp_attn_context_paged_fp8(
    const pcp_fp8_t* q, const pcp_fp8_t* k_cache, const pcp_fp8_t* v_cache, int num_blocks,
    int block_size, const int32_t* block_tables, int num_reqs, int max_blocks,
    const pcp_row_t* rows, int num_rows, int total_q, int max_q_len, int num_q_heads,
    int num_kv_heads, int head_dim, float softmax_scale, const float* q_descale,
    const float* k_descale, const float* v_descale, pcp_bf16_t* out, float* lse,
    float* workspace, int decode_splits, const int32_t* unit_order, int num_units,
    hipStream_t stream) {
  if (num_rows < 0 || total_q < 0 || max_q_len < 0 || num_blocks < 0 || block_size < 1 ||
      num_reqs < 0 || max_blocks < 0)
    return PCP_EINVAL;
  if (decode_splits < 1 || (decode_splits > 1 && workspace == nullptr)) return PCP_EINVAL;
  if (((uintptr_t)workspace & 15) != 0) return PCP_EINVAL;  // partials are 16-byte stores
  if (decode_splits > kMaxDecodeSplits) return PCP_EUNSUPPORTED;
  if (unit_order != nullptr && num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim, softmax_scale);
  if (rc != PCP_OK) return rc;
  if (num_rows == 0 || max_q_len == 0 || total_q == 0) return PCP_OK;
  if (!q || !rows || !out || !lse || num_reqs < 1) return PCP_EINVAL;
  if (max_blocks > 0 && (!k_cache || !v_cache || !block_tables || num_blocks < 1))
    return PCP_EINVAL;
  const int rf = check_fp8(q, nullptr, nullptr, k_cache, v_cache, q_descale, k_descale,
                           v_descale);
  if (rf != PCP_OK) return rf;
  if ((int64_t)max_blocks * block_size > INT32_MAX) return PCP_EOVERFLOW;
  AttnArgs a = {};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.q_ds = q_descale;
  a.k_ds = k_descale;
  a.v_ds = v_descale;
  a.rows = rows;
  a.block_tables = block_tables;
  a.out = out;
  a.lse = lse;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.num_reqs = num_reqs;
  a.max_blocks = max_blocks;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale_log2 = softmax_scale * kLog2e;
  a.ws = workspace;
  a.dec_splits = decode_splits;
  a.order = unit_order;
  return dispatch_attn<true>(a, kContext, head_dim, max_q_len, num_units, stream);
}

extern "C" int pcp_attn_rank_share_fp8(
    const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v, int total_k,
    const pcp_fp8_t* k_cache, const pcp_fp8_t* v_cache, int num_blocks, int block_size,
    const int32_t* block_tables, int num_reqs, int max_blocks, const pcp_row_t* rows,
    int num_rows, int total_q, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
    float softmax_scale, const float* q_descale, const float* k_descale, const float* v_descale,
    pcp_bf16_t* out, float* lse, float* workspace, int decode_splits, const int32_t* unit_order,
    int num_units, hipStream_t stream) {
  if (num_rows < 0 || total_q < 0 || total_k < 0 || max_q_len < 0 || num_blocks < 0 ||
      block_size < 1 || num_reqs < 0 || max_blocks < 0)
    return PCP_EINVAL;
  if (decode_splits < 1 || (decode_splits > 1 && workspace == nullptr)) return PCP_EINVAL;
  if (((uintptr_t)workspace & 15) != 0) return PCP_EINVAL;
  if (decode_splits > kMaxDecodeSplits) return PCP_EUNSUPPORTED;
  if (unit_order != nullptr && num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim, softmax_scale);
  if (rc != PCP_OK) return rc;
  if (num_rows == 0 || max_q_len == 0 || total_q == 0) return PCP_OK;
  if (!q || !rows || !out || !lse || num_reqs < 1) return PCP_EINVAL;
  if (total_k > 0 && (!k || !v)) return PCP_EINVAL;
  if (max_blocks > 0 && (!k_cache || !v_cache || !block_tables || num_blocks < 1))
    return PCP_EINVAL;
  const int rf = check_fp8(q, k, v, k_cache, v_cache, q_descale, k_descale, v_descale);
  if (rf != PCP_OK) return rf;
  if ((int64_t)max_blocks * block_size > INT32_MAX) return PCP_EOVERFLOW;
  if ((uint64_t)total_k * num_kv_heads * head_dim > 0xFFFFFFFFull) return PCP_EUNSUPPORTED;
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = k_cache;
  a.vc = v_cache;
  a.q_ds = q_descale;
  a.k_ds = k_descale;
  a.v_ds = v_descale;
  a.rows = rows;
  a.block_tables = block_tables;
  a.out = out;
  a.lse = lse;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.total_k = total_k;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.num_reqs = num_reqs;
  a.max_blocks = max_blocks;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale_log2 = softmax_scale * kLog2e;
  a.ws = workspace;
  a.dec_splits = decode_splits;
  a.order = unit_order;
  return dispatch_attn<true>(a, kFused, head_dim, max_q_len, num_units, stream);
}
