// Argument checks of the attention entry points of libpcpattn (internal
// header, host code only): the argument record every bf16 and FP8 call fills
// and the one function that validates it, so that every call checks its
// arguments in the same order and reports every error before anything is
// enqueued. It holds no device code, so the same checks also build with a
// plain host compiler (the CPU sanitizer test of the host code does).
#ifndef PCP_ATTN_CHECK_H
#define PCP_ATTN_CHECK_H

#include <stdint.h>

#include <cmath>

#include "pcp_attn.h"
#include "pcp_geometry.h"

namespace pcp_check {

enum Pass { kNewTokens, kContext, kFused };

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

inline int check_heads(int hq, int hkv, int d, float scale) {
  if (hq < 1 || hkv < 1) return PCP_EINVAL;
  if (hq % hkv != 0) return PCP_EINVAL;
  if (!pcp_geom::supported_dim(d)) return PCP_EUNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return PCP_EINVAL;
  return PCP_OK;
}

// Work units of one launch (rows x head groups x query-tile slots), in 64
// bits so that no caller value can wrap it.
inline int64_t unit_count(const CallArgs& c, Pass pass) {
  const int group = c.hq / c.hkv;
  const int hg = pcp_geom::heads_per_group(group);
  const int64_t qt =
      pcp_geom::q_tiles(c.max_q_len, hg, pass != kNewTokens, c.decode_splits);
  return (int64_t)c.num_rows * c.hkv * (group / hg) * qt;
}

// Returned by validate() when the arguments are valid and the call has no
// work (no rows or no queries): the entry point returns PCP_OK at once.
constexpr int kNothingToDo = 1;

// PCP_OK: launch. kNothingToDo: valid, nothing to launch. Negative: the
// call's error code.
inline int validate(const CallArgs& c, Pass pass, bool fp8) {
  const bool has_new = pass != kContext;
  const bool has_ctx = pass != kNewTokens;
  const int elem = fp8 ? 1 : 2;
  if (c.num_rows < 0 || c.total_q < 0 || c.max_q_len < 0) return PCP_EINVAL;
  if (has_new && c.total_k < 0) return PCP_EINVAL;
  if ((has_ctx || fp8) && c.num_reqs < 0) return PCP_EINVAL;
  if (has_ctx && (c.num_blocks < 0 || c.block_size < 1 || c.max_blocks < 0)) return PCP_EINVAL;
  if (has_ctx) {
    if (c.decode_splits < 1 || (c.decode_splits > 1 && c.workspace == nullptr)) return PCP_EINVAL;
    if (((uintptr_t)c.workspace & 15) != 0) return PCP_EINVAL;  // partials are 16-byte stores
    if (c.decode_splits > pcp_geom::kMaxDecodeSplits) return PCP_EUNSUPPORTED;
  }
  if (c.order != nullptr && c.num_units < 0) return PCP_EINVAL;
  const int rc = check_heads(c.hq, c.hkv, c.head_dim, c.scale);
  if (rc != PCP_OK) return rc;
  if (c.num_rows == 0 || c.max_q_len == 0 || c.total_q == 0) return kNothingToDo;
  if (!c.q || !c.rows || !c.out || !c.lse) return PCP_EINVAL;
  if (fp8 && c.num_reqs < 1) return PCP_EINVAL;  // rows index the descale tables
  if (has_new && c.total_k > 0 && (!c.k || !c.v)) return PCP_EINVAL;
  if (has_ctx && c.max_blocks > 0 &&
      (!c.kc || !c.vc || !c.block_tables || c.num_blocks < 1 || c.num_reqs < 1))
    return PCP_EINVAL;
  if (fp8) {
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
  // one workgroup per unit, unit ids in int32
  if (unit_count(c, pass) > INT32_MAX) return PCP_EOVERFLOW;
  return PCP_OK;
}

}  // namespace pcp_check

#endif  // PCP_ATTN_CHECK_H
