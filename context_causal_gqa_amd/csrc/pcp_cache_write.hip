// gfx950 kernel and C-ABI launcher of the paged KV-cache write that precedes
// attention on the re-split path.
//
// "[MRv2][PCP] Carry the row plan in attention metadata; fix mixed
// prefill+decode crash" (fork PR #2), comment on commit 97aad2056e: the
// gathered slot mapping masks every token a rank must not write to a
// negative slot, and the cache writer skips negative slots; "What made it
// removable": the write is ordered before attention, so earlier chunks' new
// tokens are ordinary cached context when the rows attend.
//
// A token's K (and V) row is Hkv * d values (bf16, or E4M3 codes for the
// FP8 cache), contiguous both in the token-major source and at its slot of
// the [num_blocks, block_size, Hkv, d] cache, so the write is a scatter of
// 16-byte chunks: each thread moves one 16-byte chunk of K and the same chunk
// of V per step of a grid-stride loop; consecutive threads take consecutive
// chunks of a row, so loads and stores are coalesced. HBM-bound: 2 * 2 * Hkv
// * d * (bytes per value) per written token.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pcp_attn.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4_t* __restrict__ k, const u32x4_t* __restrict__ v,
    const int64_t* __restrict__ slots, uint32_t num_chunks, uint32_t chunks_per_token,
    int64_t num_slots, u32x4_t* __restrict__ k_cache, u32x4_t* __restrict__ v_cache) {
  // 32-bit chunk indices (the launcher checks they fit); 64-bit addresses
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < num_chunks; i += stride) {
    const uint32_t tok = i / chunks_per_token;
    const uint32_t c = i - tok * chunks_per_token;
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;  // masked (or outside the pool)
    const int64_t dst = slot * chunks_per_token + c;
    k_cache[dst] = k[i];
    v_cache[dst] = v[i];
  }
}

}  // namespace

namespace {

int launch_write(const void* k, const void* v, const int64_t* slot_mapping, int num_tokens,
                 int num_kv_heads, int head_dim, int elem_bytes, void* k_cache, void* v_cache,
                 int num_blocks, int block_size, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 0 || block_size < 1) return PCP_EINVAL;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PCP_EUNSUPPORTED;
  if (num_tokens == 0) return PCP_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PCP_EINVAL;
  // 16-byte chunks: the rows must be 16-byte aligned
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15)
    return PCP_EINVAL;
  // 64-bit sizes: no caller value wraps them
  const int64_t chunks_per_token = (int64_t)num_kv_heads * head_dim * elem_bytes / 16;
  const int64_t num_chunks = (int64_t)num_tokens * chunks_per_token;
  // 32-bit chunk indices: i + stride stays below 2^32
  if (num_chunks > (int64_t)0xFFFFFFFFu - 65536 * 256) return PCP_EUNSUPPORTED;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const int64_t want = (num_chunks + 255) / 256;
  // One chunk per thread up to 2^24 chunks (at most 256 workgroups per CU):
  // measured 5-10% faster than 8 workgroups per CU looping over the chunks
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(k), reinterpret_cast<const u32x4_t*>(v),
                     slot_mapping, (uint32_t)num_chunks, (uint32_t)chunks_per_token, num_slots,
                     reinterpret_cast<u32x4_t*>(k_cache), reinterpret_cast<u32x4_t*>(v_cache));
  return hipGetLastError() == hipSuccess ? PCP_OK : PCP_EHIP;
}

}  // namespace

extern "C" int pcp_kv_cache_write(const pcp_bf16_t* k, const pcp_bf16_t* v,
                                  const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                  int head_dim, pcp_bf16_t* k_cache, pcp_bf16_t* v_cache,
                                  int num_blocks, int block_size, hipStream_t stream) {
  return launch_write(k, v, slot_mapping, num_tokens, num_kv_heads, head_dim, 2, k_cache,
                      v_cache, num_blocks, block_size, stream);
}

extern "C" int pcp_kv_cache_write_fp8(const pcp_fp8_t* k, const pcp_fp8_t* v,
                                      const int64_t* slot_mapping, int num_tokens,
                                      int num_kv_heads, int head_dim, pcp_fp8_t* k_cache,
                                      pcp_fp8_t* v_cache, int num_blocks, int block_size,
                                      hipStream_t stream) {
  return launch_write(k, v, slot_mapping, num_tokens, num_kv_heads, head_dim, 1, k_cache,
                      v_cache, num_blocks, block_size, stream);
}
