// Host side of the attention entry points of libpcpattn (internal header):
// one argument record and one validate-then-launch function shared by the
// bf16 and FP8 C-ABI calls, so that every call checks its arguments in the
// same order and reports every error before anything is enqueued.
#ifndef PCP_ATTN_CALL_H
#define PCP_ATTN_CALL_H

#include "pcp_attn_fwd.h"

namespace {

// Arguments of one attention entry point (bf16 or FP8; pointers are Q/K/V
// elements of either type). Fields a pass does not use stay zero.
struct CallArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const void* kc = nullptr;
  const void* vc = nullptr;
  const float* q_ds = nullptr;
  const float* k_ds = nullptr;
  const float* v_ds = nullptr;
  const pcp_row_t* rows = nullptr;
  const int32_t* block_tables = nullptr;
  pcp_bf16_t* out = nullptr;
  float* lse = nullptr;
  float* workspace = nullptr;
  const int32_t* order = nullptr;
  int num_rows = 0, total_q = 0, total_k = 0, max_q_len = 0;
  int num_blocks = 0, block_size = 1, num_reqs = 0, max_blocks = 0;
  int hq = 0, hkv = 0, head_dim = 0, decode_splits = 1, num_units = 0;
  float scale = 0.f;
};

// Validate (every error is returned before anything is enqueued) and launch
// one pass. The checks run in one order for every entry point.
template <bool FP8>
int attn_call(const CallArgs& c, Pass pass, hipStream_t stream) {
  const bool has_new = pass != kContext;
  const bool has_ctx = pass != kNewTokens;
  constexpr int elem = FP8 ? 1 : 2;
  if (c.num_rows < 0 || c.total_q < 0 || c.max_q_len < 0) return PCP_EINVAL;
  if (has_new && c.total_k < 0) return PCP_EINVAL;
  if ((has_ctx || FP8) && c.num_reqs < 0) return PCP_EINVAL;
  if (has_ctx && (c.num_blocks < 0 || c.block_size < 1 || c.max_blocks < 0)) return PCP_EINVAL;
  if (has_ctx) {
    if (c.decode_splits < 1 || (c.decode_splits > 1 && c.workspace == nullptr)) return PCP_EINVAL;
    if (((uintptr_t)c.workspace & 15) != 0) return PCP_EINVAL;  // partials are 16-byte stores
    if (c.decode_splits > kMaxDecodeSplits) return PCP_EUNSUPPORTED;
  }
  if (c.order != nullptr && c.num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(c.hq, c.hkv, c.head_dim, c.scale);
  if (rc != PCP_OK) return rc;
  if (c.num_rows == 0 || c.max_q_len == 0 || c.total_q == 0) return PCP_OK;
  if (!c.q || !c.rows || !c.out || !c.lse) return PCP_EINVAL;
  if (FP8 && c.num_reqs < 1) return PCP_EINVAL;  // rows index the descale tables
  if (has_new && c.total_k > 0 && (!c.k || !c.v)) return PCP_EINVAL;
  if (has_ctx && c.max_blocks > 0 &&
      (!c.kc || !c.vc || !c.block_tables || c.num_blocks < 1 || c.num_reqs < 1))
    return PCP_EINVAL;
  if constexpr (FP8) {
    // descale tables given and 4-byte aligned; codes read 16 bytes at a time
    if (!c.q_ds || !c.k_ds || !c.v_ds) return PCP_EINVAL;
    if (((uintptr_t)c.q_ds | (uintptr_t)c.k_ds | (uintptr_t)c.v_ds) & 3) return PCP_EINVAL;
    if (((uintptr_t)c.q | (uintptr_t)c.k | (uintptr_t)c.v | (uintptr_t)c.kc | (uintptr_t)c.vc) &
        15)
      return PCP_EINVAL;
  }
  if (has_ctx && (int64_t)c.max_blocks * c.block_size > INT32_MAX) return PCP_EOVERFLOW;
  // new-token K/V rows are fetched with 32-bit buffer offsets
  if (has_new && (uint64_t)c.total_k * c.hkv * c.head_dim * elem > 0xFFFFFFFFull)
    return PCP_EUNSUPPORTED;
  AttnArgs a = {};
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.kc = c.kc;
  a.vc = c.vc;
  a.q_ds = c.q_ds;
  a.k_ds = c.k_ds;
  a.v_ds = c.v_ds;
  a.rows = c.rows;
  a.block_tables = c.block_tables;
  a.out = c.out;
  a.lse = c.lse;
  a.num_rows = c.num_rows;
  a.total_q = c.total_q;
  a.total_k = has_new ? c.total_k : 0;
  a.num_blocks = has_ctx ? c.num_blocks : 0;
  a.block_size = has_ctx ? c.block_size : 0;
  a.num_reqs = c.num_reqs;
  a.max_blocks = has_ctx ? c.max_blocks : 0;
  a.hq = c.hq;
  a.hkv = c.hkv;
  a.group = c.hq / c.hkv;
  a.scale_log2 = c.scale * kLog2e;
  a.ws = has_ctx ? c.workspace : nullptr;
  a.dec_splits = has_ctx ? c.decode_splits : 1;
  a.order = c.order;
  return dispatch_attn<FP8>(a, pass, c.head_dim, c.max_q_len, c.num_units, stream);
}

}  // namespace

#endif  // PCP_ATTN_CALL_H
