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

#include "pcp_attn_call.h"

extern "C" int pcp_attn_prefill_fp8(const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v,
                                    const pcp_row_t* rows, int num_rows, int total_q,
                                    int total_k, int max_q_len, int num_reqs, int num_q_heads,
                                    int num_kv_heads, int head_dim, float softmax_scale,
                                    const float* q_descale, const float* k_descale,
                                    const float* v_descale, pcp_bf16_t* out, float* lse,
                                    const int32_t* unit_order, int num_units,
                                    hipStream_t stream) {
  CallArgs c;
  c.q = q;
  c.k = k;
  c.v = v;
  c.rows = rows;
  c.num_rows = num_rows;
  c.total_q = total_q;
  c.total_k = total_k;
  c.max_q_len = max_q_len;
  c.num_reqs = num_reqs;
  c.hq = num_q_heads;
  c.hkv = num_kv_heads;
  c.head_dim = head_dim;
  c.scale = softmax_scale;
  c.q_ds = q_descale;
  c.k_ds = k_descale;
  c.v_ds = v_descale;
  c.out = out;
  c.lse = lse;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<true>(c, kNewTokens, stream);
}

extern "C" int pcp_attn_context_paged_fp8(
    const pcp_fp8_t* q, const pcp_fp8_t* k_cache, const pcp_fp8_t* v_cache, int num_blocks,
    int block_size, const int32_t* block_tables, int num_reqs, int max_blocks,
    const pcp_row_t* rows, int num_rows, int total_q, int max_q_len, int num_q_heads,
    int num_kv_heads, int head_dim, float softmax_scale, const float* q_descale,
    const float* k_descale, const float* v_descale, pcp_bf16_t* out, float* lse,
    float* workspace, int decode_splits, const int32_t* unit_order, int num_units,
    hipStream_t stream) {
  CallArgs c;
  c.q = q;
  c.kc = k_cache;
  c.vc = v_cache;
  c.num_blocks = num_blocks;
  c.block_size = block_size;
  c.block_tables = block_tables;
  c.num_reqs = num_reqs;
  c.max_blocks = max_blocks;
  c.rows = rows;
  c.num_rows = num_rows;
  c.total_q = total_q;
  c.max_q_len = max_q_len;
  c.hq = num_q_heads;
  c.hkv = num_kv_heads;
  c.head_dim = head_dim;
  c.scale = softmax_scale;
  c.q_ds = q_descale;
  c.k_ds = k_descale;
  c.v_ds = v_descale;
  c.out = out;
  c.lse = lse;
  c.workspace = workspace;
  c.decode_splits = decode_splits;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<true>(c, kContext, stream);
}

extern "C" int pcp_attn_rank_share_fp8(
    const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v, int total_k,
    const pcp_fp8_t* k_cache, const pcp_fp8_t* v_cache, int num_blocks, int block_size,
    const int32_t* block_tables, int num_reqs, int max_blocks, const pcp_row_t* rows,
    int num_rows, int total_q, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
    float softmax_scale, const float* q_descale, const float* k_descale, const float* v_descale,
    pcp_bf16_t* out, float* lse, float* workspace, int decode_splits, const int32_t* unit_order,
    int num_units, hipStream_t stream) {
  CallArgs c;
  c.q = q;
  c.k = k;
  c.v = v;
  c.total_k = total_k;
  c.kc = k_cache;
  c.vc = v_cache;
  c.num_blocks = num_blocks;
  c.block_size = block_size;
  c.block_tables = block_tables;
  c.num_reqs = num_reqs;
  c.max_blocks = max_blocks;
  c.rows = rows;
  c.num_rows = num_rows;
  c.total_q = total_q;
  c.max_q_len = max_q_len;
  c.hq = num_q_heads;
  c.hkv = num_kv_heads;
  c.head_dim = head_dim;
  c.scale = softmax_scale;
  c.q_ds = q_descale;
  c.k_ds = k_descale;
  c.v_ds = v_descale;
  c.out = out;
  c.lse = lse;
  c.workspace = workspace;
  c.decode_splits = decode_splits;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<true>(c, kFused, stream);
}
