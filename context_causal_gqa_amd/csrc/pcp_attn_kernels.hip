// gfx950 C-ABI entry points of the bf16 attention passes and the LSE merge
// kernel. The attention kernel itself is in pcp_attn_fwd.h.

#include <mutex>

#include "pcp_attn_call.h"

namespace {

// ---------------------------------------------------------------- merge

constexpr int kMaxParts = 16;
#ifndef PCP_MERGE_NV
#define PCP_MERGE_NV 1  // 16-byte chunks of each partial per thread
#endif

struct MergeArgs {
  const u16* outs[kMaxParts];
  const float* lses[kMaxParts];
  u16* out;
  float* lse_out;
  int k;
  int total_q;
  int hq;
};

// One (query, head) pair per D / (8 NV) threads, NV chunks of 8 bf16 values
// (16 bytes) of each partial per thread; a pair's threads sit in one wave,
// so every lane has read lses[0] before lane 0 writes lse_out (which may
// alias it). With K > 0 (exactly K partials) all LSEs are read first and then
// all non-empty partials' outputs, so the loads of a thread are in flight
// together; K = 0 takes k from the arguments.
template <int D, int K>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeArgs a) {
  constexpr int NV = PCP_MERGE_NV;
  constexpr int TPR = D / (8 * NV);  // threads per pair
  constexpr int PPB = 256 / TPR;     // pairs per workgroup
  const int64_t pair = (int64_t)blockIdx.x * PPB + threadIdx.x / TPR;
  const int e = threadIdx.x % TPR;
  if (pair >= (int64_t)a.total_q * a.hq) return;
  const int qi = (int)(pair / a.hq);
  const int h = (int)(pair - (int64_t)qi * a.hq);
  const size_t lidx = (size_t)h * a.total_q + qi;
  const size_t off = (size_t)pair * D + 8 * NV * e;
  constexpr int KU = K > 0 ? K : kMaxParts;
  const int k = K > 0 ? K : a.k;

  float lv[KU];
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < KU; ++i) {
    if (K == 0 && i >= k) break;
    lv[i] = a.lses[i][lidx];
    mx = fmaxf(mx, lv[i]);
  }
  float acc[8 * NV];
#pragma unroll
  for (int c = 0; c < 8 * NV; ++c) acc[c] = 0.f;
  float wsum = 0.f;
  if (mx != kNegInf) {
    if constexpr (K > 0) {
      float w[K];
      bf16x8_t x[K][NV];
#pragma unroll
      for (int i = 0; i < K; ++i) {
        w[i] = __builtin_amdgcn_exp2f((lv[i] - mx) * kLog2e);
        wsum += w[i];
#pragma unroll
        for (int v = 0; v < NV; ++v)
          x[i][v] = w[i] != 0.f ? *reinterpret_cast<const bf16x8_t*>(a.outs[i] + off + 8 * v)
                                : bf16x8_t{};
      }
#pragma unroll
      for (int i = 0; i < K; ++i) {
#pragma unroll
        for (int c = 0; c < 8 * NV; ++c) acc[c] = fmaf(w[i], (float)x[i][c >> 3][c & 7], acc[c]);
      }
    } else {
      for (int i = 0; i < k; ++i) {
        const float w = __builtin_amdgcn_exp2f((lv[i] - mx) * kLog2e);
        wsum += w;
        if (w != 0.f) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(a.outs[i] + off + 8 * v);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[8 * v + c] = fmaf(w, (float)x[c], acc[8 * v + c]);
          }
        }
      }
    }
  }
  const float inv = mx != kNegInf ? 1.0f / wsum : 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    bf16x8_t y;
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = (__bf16)(acc[8 * v + c] * inv);
    *reinterpret_cast<bf16x8_t*>(a.out + off + 8 * v) = y;
  }
  if (e == 0) a.lse_out[lidx] = mx != kNegInf ? mx + __builtin_amdgcn_logf(wsum) * kLn2 : kNegInf;
}

template <int D>
void launch_merge(const MergeArgs& a, unsigned blocks, hipStream_t stream) {
  switch (a.k) {
    case 2: hipLaunchKernelGGL((lse_merge_kernel<D, 2>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((lse_merge_kernel<D, 3>), dim3(blocks), dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((lse_merge_kernel<D, 4>), dim3(blocks), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((lse_merge_kernel<D, 0>), dim3(blocks), dim3(256), 0, stream, a); break;
  }
}

}  // namespace

extern "C" int pcp_attn_prefill(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                                const pcp_row_t* rows, int num_rows, int total_q, int total_k,
                                int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                                float softmax_scale, pcp_bf16_t* out, float* lse,
                                const int32_t* unit_order, int num_units, hipStream_t stream) {
  CallArgs c;
  c.q = q;
  c.k = k;
  c.v = v;
  c.rows = rows;
  c.num_rows = num_rows;
  c.total_q = total_q;
  c.total_k = total_k;
  c.max_q_len = max_q_len;
  c.hq = num_q_heads;
  c.hkv = num_kv_heads;
  c.head_dim = head_dim;
  c.scale = softmax_scale;
  c.out = out;
  c.lse = lse;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<false>(c, kNewTokens, stream);
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
  c.out = out;
  c.lse = lse;
  c.workspace = workspace;
  c.decode_splits = decode_splits;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<false>(c, kContext, stream);
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
  c.out = out;
  c.lse = lse;
  c.workspace = workspace;
  c.decode_splits = decode_splits;
  c.order = unit_order;
  c.num_units = num_units;
  return attn_call<false>(c, kFused, stream);
}

// ---------------------------------------------------------- no-allocation variant

// Scratch of pcp_attn_rank_share_noalloc: the split-decode partials go to
// this file-scope array instead of a caller workspace. Each device holds its
// own copy (at its own address) until the process ends.
static __device__ __align__(256) float scratch[PCP_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
float* scratch_addr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of `scratch` on the current device. In host code the array's
// name stands for a host-side shadow, not device memory, so the address is
// looked up with hipGetSymbolAddress once per device (with that device
// current) and kept; kernels and copies use only this address.
int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PCP_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PCP_EHIP;
    scratch_addr[dev] = static_cast<float*>(p);
  }
  *out = scratch_addr[dev];
  return PCP_OK;
}

}  // namespace

extern "C" int pcp_attn_rank_share_noalloc(
    const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v, int total_k,
    const pcp_bf16_t* k_cache, const pcp_bf16_t* v_cache, int num_blocks, int block_size,
    const int32_t* block_tables, int num_reqs, int max_blocks, const pcp_row_t* rows, int num_rows,
    int total_q, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
    float softmax_scale, pcp_bf16_t* out, float* lse, int decode_splits,
    const int32_t* unit_order, int num_units, hipStream_t stream) {
  float* ws = nullptr;
  if (decode_splits > 1) {
    // the partials must fit the fixed array (sizes in 64 bits); every other
    // argument is checked by pcp_attn_rank_share
    if (decode_splits > pcp_geom::kMaxDecodeSplits) return PCP_EUNSUPPORTED;
    if (num_rows < 0 || num_q_heads < 1) return PCP_EINVAL;
    if (!supported_dim(head_dim)) return PCP_EUNSUPPORTED;
    const uint64_t need = (uint64_t)num_rows * num_q_heads * decode_splits * (head_dim + 1) *
                          sizeof(float);
    if (need > PCP_NOALLOC_SCRATCH_BYTES) return PCP_ESCRATCH;
    const int rc = scratch_on_current_device(&ws);
    if (rc != PCP_OK) return rc;
  }
  return pcp_attn_rank_share(q, k, v, total_k, k_cache, v_cache, num_blocks, block_size,
                             block_tables, num_reqs, max_blocks, rows, num_rows, total_q,
                             max_q_len, num_q_heads, num_kv_heads, head_dim, softmax_scale, out,
                             lse, ws, decode_splits, unit_order, num_units, stream);
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
  const int ppb = 256 / (head_dim / (8 * PCP_MERGE_NV));
  const int64_t blocks = (pairs + ppb - 1) / ppb;
  if (blocks > INT32_MAX) return PCP_EOVERFLOW;
  switch (head_dim) {
    case 64: launch_merge<64>(a, (unsigned)blocks, stream); break;
    case 128: launch_merge<128>(a, (unsigned)blocks, stream); break;
    default: launch_merge<256>(a, (unsigned)blocks, stream); break;
  }
  return hipGetLastError() == hipSuccess ? PCP_OK : PCP_EHIP;
}
