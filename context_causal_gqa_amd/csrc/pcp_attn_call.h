// Host side of the attention entry points of libpcpattn (internal header):
// validate the argument record (pcp_attn_check.h) and launch one pass, shared
// by the bf16 and FP8 C-ABI calls.
#ifndef PCP_ATTN_CALL_H
#define PCP_ATTN_CALL_H

#include "pcp_attn_check.h"
#include "pcp_attn_fwd.h"

namespace {

using pcp_check::CallArgs;

// Validate (every error is returned before anything is enqueued) and launch
// one pass.
template <bool FP8>
int attn_call(const CallArgs& c, Pass pass, hipStream_t stream) {
  const bool has_new = pass != kContext;
  const bool has_ctx = pass != kNewTokens;
  const int rc = pcp_check::validate(c, pass, FP8);
  if (rc == pcp_check::kNothingToDo) return PCP_OK;
  if (rc != PCP_OK) return rc;
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
