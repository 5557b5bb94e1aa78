// gfx950 C-ABI entry points of the bf16 attention passes and the LSE merge
// kernel. The attention kernel itself is in pcp_attn_fwd.h.

#include "pcp_attn_fwd.h"

namespace {

// ---------------------------------------------------------------- merge

constexpr int kMaxParts = 16;

struct MergeArgs {
  const u16* outs[kMaxParts];
  const float* lses[kMaxParts];
  u16* out;
  float* lse_out;
  int k;
  int total_q;
  int hq;
};

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a) {
  constexpr int TPR = D / 8;      // threads per (query, head), 8 values each
  constexpr int PPB = 256 / TPR;  // (query, head) pairs per block
  const int64_t pair = (int64_t)blockIdx.x * PPB + threadIdx.x / TPR;
  const int e = threadIdx.x % TPR;
  if (pair >= (int64_t)a.total_q * a.hq) return;
  const int qi = (int)(pair / a.hq);
  const int h = (int)(pair - (int64_t)qi * a.hq);
  const size_t lidx = (size_t)h * a.total_q + qi;

  float lv[kMaxParts];
  float mx = kNegInf;
  for (int i = 0; i < a.k; ++i) {
    lv[i] = a.lses[i][lidx];
    mx = fmaxf(mx, lv[i]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  const size_t off = (size_t)pair * D + 8 * e;
  if (mx != kNegInf) {
    for (int i = 0; i < a.k; ++i) {
      const float w = __builtin_amdgcn_exp2f((lv[i] - mx) * kLog2e);
      wsum += w;
      if (w != 0.f) {
        const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(a.outs[i] + off);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(w, (float)x[c], acc[c]);
      }
    }
  }
  const float inv = mx != kNegInf ? 1.0f / wsum : 0.f;
  bf16x8_t y;
#pragma unroll
  for (int c = 0; c < 8; ++c) y[c] = (__bf16)(acc[c] * inv);
  *reinterpret_cast<bf16x8_t*>(a.out + off) = y;
  if (e == 0) a.lse_out[lidx] = mx != kNegInf ? mx + __builtin_amdgcn_logf(wsum) * kLn2 : kNegInf;
}

}  // namespace

extern "C" int pcp_attn_prefill(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                                const pcp_row_t* rows, int num_rows, int total_q, int total_k,
                                int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                                float softmax_scale, pcp_bf16_t* out, float* lse,
                                const int32_t* unit_order, int num_units, hipStream_t stream) {
  if (num_rows < 0 || total_q < 0 || total_k < 0 || max_q_len < 0) return PCP_EINVAL;
  if (unit_order != nullptr && num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim, softmax_scale);
  if (rc != PCP_OK) return rc;
  if (num_rows == 0 || max_q_len == 0 || total_q == 0) return PCP_OK;
  if (!q || !rows || !out || !lse) return PCP_EINVAL;
  if (total_k > 0 && (!k || !v)) return PCP_EINVAL;
  // K/V rows are fetched with 32-bit buffer offsets.
  if ((uint64_t)total_k * num_kv_heads * head_dim * 2 > 0xFFFFFFFFull) return PCP_EUNSUPPORTED;
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.rows = rows;
  a.out = out;
  a.lse = lse;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.total_k = total_k;
  a.hq = num_q_heads;
  a.hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.scale_log2 = softmax_scale * kLog2e;
  a.order = unit_order;
  return dispatch_attn<false>(a, kNewTokens, head_dim, max_q_len, num_units, stream);
}

extern "C" int pcp_attn_context_paged(const pcp_bf16_t* q, const pcp_bf16_t* k_cache,
                                      const pcp_bf16_t* v_cache, int num_blocks, int block_size,
                                      const int32_t* block_tables, int num_reqs, int max_blocks,
                                      const pcp_row_t* rows, int num_rows, int total_q,
                                      int max_q_len, int num_q_heads, int num_kv_heads,
                                      int head_dim, float softmax_scale, pcp_bf16_t* out,
                                      float* lse, float* workspace, int decode_splits,
                                      const int32_t* unit_order, int num_units,
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
  if (!q || !rows || !out || !lse) return PCP_EINVAL;
  if (max_blocks > 0 && (!k_cache || !v_cache || !block_tables || num_blocks < 1 || num_reqs < 1))
    return PCP_EINVAL;
  if ((int64_t)max_blocks * block_size > INT32_MAX) return PCP_EOVERFLOW;
  AttnArgs a = {};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
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
  return dispatch_attn<false>(a, kContext, head_dim, max_q_len, num_units, stream);
}

extern "C" int pcp_attn_rank_share(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                                   int total_k, const pcp_bf16_t* k_cache,
                                   const pcp_bf16_t* v_cache, int num_blocks, int block_size,
                                   const int32_t* block_tables, int num_reqs, int max_blocks,
                                   const pcp_row_t* rows, int num_rows, int total_q, int max_q_len,
                                   int num_q_heads, int num_kv_heads, int head_dim,
                                   float softmax_scale, pcp_bf16_t* out, float* lse,
                                   float* workspace, int decode_splits, const int32_t* unit_order,
                                   int num_units, hipStream_t stream) {
  if (num_rows < 0 || total_q < 0 || total_k < 0 || max_q_len < 0 || num_blocks < 0 ||
      block_size < 1 || num_reqs < 0 || max_blocks < 0)
    return PCP_EINVAL;
  if (decode_splits < 1 || (decode_splits > 1 && workspace == nullptr)) return PCP_EINVAL;
  if (((uintptr_t)workspace & 15) != 0) return PCP_EINVAL;  // partials are 16-byte stores
  if (decode_splits > kMaxDecodeSplits) return PCP_EUNSUPPORTED;
  if (unit_order != nullptr && num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(num_q_heads, num_kv_heads, head_dim, softmax_scale);
  if (rc != PCP_OK) return rc;
  if (num_rows == 0 || max_q_len == 0 || total_q == 0) return PCP_OK;
  if (!q || !rows || !out || !lse) return PCP_EINVAL;
  if (total_k > 0 && (!k || !v)) return PCP_EINVAL;
  if (max_blocks > 0 && (!k_cache || !v_cache || !block_tables || num_blocks < 1 || num_reqs < 1))
    return PCP_EINVAL;
  if ((int64_t)max_blocks * block_size > INT32_MAX) return PCP_EOVERFLOW;
  // new-token K/V rows are fetched with 32-bit buffer offsets
  if ((uint64_t)total_k * num_kv_heads * head_dim * 2 > 0xFFFFFFFFull) return PCP_EUNSUPPORTED;
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = k_cache;
  a.vc = v_cache;
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
  return dispatch_attn<false>(a, kFused, head_dim, max_q_len, num_units, stream);
}

extern "C" size_t pcp_context_workspace_bytes(int num_rows, int num_q_heads, int head_dim,
                                              int decode_splits) {
  if (num_rows < 0 || num_q_heads < 1 || decode_splits < 1 || !supported_dim(head_dim)) return 0;
  if (decode_splits == 1) return 0;
  return (size_t)num_rows * num_q_heads * decode_splits * (head_dim + 1) * sizeof(float);
}

extern "C" int lse_merge(int k, const pcp_bf16_t* const* outs, const float* const* lses,
                         int total_q, int num_q_heads, int head_dim, pcp_bf16_t* out,
                         float* lse_out, hipStream_t stream) {
  if (k < 1 || total_q < 0 || num_q_heads < 1 || !outs || !lses) return PCP_EINVAL;
  if (k > kMaxParts) return PCP_EUNSUPPORTED;
  if (!supported_dim(head_dim)) return PCP_EUNSUPPORTED;
  if (total_q == 0) return PCP_OK;
  if (!out || !lse_out) return PCP_EINVAL;
  MergeArgs a = {};
  for (int i = 0; i < k; ++i) {
    if (!outs[i] || !lses[i]) return PCP_EINVAL;
    a.outs[i] = outs[i];
    a.lses[i] = lses[i];
  }
  a.out = out;
  a.lse_out = lse_out;
  a.k = k;
  a.total_q = total_q;
  a.hq = num_q_heads;
  const int64_t pairs = (int64_t)total_q * num_q_heads;
  const int ppb = 256 / (head_dim / 8);
  const int64_t blocks = (pairs + ppb - 1) / ppb;
  if (blocks > INT32_MAX) return PCP_EOVERFLOW;
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL(lse_merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      break;
    case 128:
      hipLaunchKernelGGL(lse_merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(lse_merge_kernel<256>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      break;
  }
  return hipGetLastError() == hipSuccess ? PCP_OK : PCP_EHIP;
}
