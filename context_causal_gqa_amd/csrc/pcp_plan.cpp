// Host side of the C ABI: the rank-local row plan and error strings.
//
// Row plan: "[MRv2][PCP] Carry the row plan in attention metadata; fix mixed
// prefill+decode crash" (fork PR #2), sections "Two things that fell out of
// (1)" (up to two rows per prefilling request, per-row context lengths) and
// "What made it removable" (DualChunkSwap gives each PCP rank a different
// row set; cached context of a row is what precedes it), plus the comment on
// commit 97aad2056e (decode rows are replicated on every PCP rank).

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "pcp_attn.h"

namespace {

// Tokens of a cached prefix of `cached` tokens that DCP rank `rank` holds when
// block j lives on rank j mod dcp: whole blocks, minus the missing tail of the
// global last block if that block is this rank's.
int64_t local_cached_tokens(int64_t cached, int dcp, int rank, int bs) {
  if (cached <= 0) return 0;
  const int64_t nblk = (cached + bs - 1) / bs;
  if (rank >= nblk) return 0;
  const int64_t owned = (nblk - 1 - rank) / dcp + 1;  // blocks rank, rank+dcp, ... < nblk
  int64_t tokens = owned * bs;
  const int64_t last = nblk - 1;
  if (last % dcp == rank) tokens -= nblk * bs - cached;
  return tokens;
}

bool debug_enabled() {
  const char* v = getenv("PCP_ATTN_DEBUG");
  return v != nullptr && v[0] != '\0' && v[0] != '0';
}

}  // namespace

extern "C" const char* pcp_strerror(int code) {
  switch (code) {
    case PCP_OK: return "ok";
    case PCP_EINVAL: return "invalid argument";
    case PCP_EUNSUPPORTED: return "unsupported configuration";
    case PCP_EHIP: return "HIP runtime error";
    case PCP_EOVERFLOW: return "size does not fit 32-bit plan fields";
    case PCP_ESCRATCH: return "call needs more scratch than the library's fixed scratch array";
    default: return code > 0 ? "count" : "unknown error";
  }
}

namespace {

// The rank-local plan. resplit: rows of the re-split path -- a prefill row's
// context is everything before its first query and its new-token keys are
// its own tokens (k_start = q_start in the rank-local K/V buffer).
int build_plan(int num_reqs, const int32_t* cu_seqlens_new, const int32_t* ctx_lens,
               int pcp_size, int pcp_rank, int dcp_size, int dcp_rank, int block_size,
               bool resplit, pcp_row_t* rows, int capacity) {
  if (num_reqs < 0 || pcp_size < 1 || pcp_rank < 0 || pcp_rank >= pcp_size || dcp_size < 1 ||
      dcp_rank < 0 || dcp_rank >= dcp_size || block_size < 1 || capacity < 0)
    return PCP_EINVAL;
  if (num_reqs > 0 && (cu_seqlens_new == nullptr || ctx_lens == nullptr)) return PCP_EINVAL;
  if (capacity > 0 && rows == nullptr) return PCP_EINVAL;
  if (num_reqs > 0 && cu_seqlens_new[0] < 0) return PCP_EINVAL;
  for (int b = 0; b < num_reqs; ++b) {
    if (cu_seqlens_new[b + 1] < cu_seqlens_new[b] || ctx_lens[b] < 0) return PCP_EINVAL;
  }

  const int64_t n_chunks = 2 * static_cast<int64_t>(pcp_size);
  const bool dbg = debug_enabled();
  int64_t count = 0;
  int64_t q_start = 0;
  auto emit = [&](const pcp_row_t& r) {
    if (count < capacity) rows[count] = r;
    if (dbg)
      fprintf(stderr,
              "[pcp_attn] row %lld req %d kind %d q_start %d q_len %d pos %d k_start %d k_len %d "
              "ctx %d ctx_local %d\n",
              (long long)count, r.req, r.kind, r.q_start, r.q_len, r.pos_start, r.k_start, r.k_len,
              r.ctx_len, r.ctx_len_local);
    ++count;
  };
  for (int b = 0; b < num_reqs; ++b) {
    const int64_t k_start = cu_seqlens_new[b];
    const int64_t n_new = static_cast<int64_t>(cu_seqlens_new[b + 1]) - k_start;
    const int64_t ctx = ctx_lens[b];
    if (n_new == 0) continue;
    if (n_new == 1) {
      // Decode row: the token's K/V was written to the cache before attention.
      const int64_t cached = ctx + 1;
      const int64_t local = local_cached_tokens(cached, dcp_size, dcp_rank, block_size);
      if (cached > INT32_MAX || q_start + 1 > INT32_MAX) return PCP_EOVERFLOW;
      pcp_row_t r = {b, PCP_ROW_DECODE, (int32_t)q_start, 1, (int32_t)ctx,
                     (int32_t)(resplit ? q_start : k_start), 0, (int32_t)cached, (int32_t)local};
      emit(r);
      q_start += 1;
      continue;
    }
    const int64_t base = n_new / n_chunks;
    const int64_t rem = n_new % n_chunks;
    const int64_t local = local_cached_tokens(ctx, dcp_size, dcp_rank, block_size);
    const int64_t chunk_ids[2] = {pcp_rank, n_chunks - 1 - pcp_rank};
    for (int side = 0; side < 2; ++side) {
      const int64_t c = chunk_ids[side];
      const int64_t lo = c * base + (c < rem ? c : rem);
      const int64_t len = base + (c < rem ? 1 : 0);
      if (len == 0) continue;
      const int64_t hi = lo + len;
      if (ctx + hi > INT32_MAX || q_start + len > INT32_MAX) return PCP_EOVERFLOW;
      pcp_row_t r = {b,
                     side == 0 ? PCP_ROW_HEAD : PCP_ROW_TAIL,
                     (int32_t)q_start,
                     (int32_t)len,
                     (int32_t)(ctx + lo),
                     (int32_t)k_start,
                     (int32_t)hi,
                     (int32_t)ctx,
                     (int32_t)local};
      if (resplit) {  // context [0, pos_start) from the cache; own tokens as keys
        r.k_start = (int32_t)q_start;
        r.k_len = (int32_t)len;
        r.ctx_len = (int32_t)(ctx + lo);
        r.ctx_len_local = (int32_t)local_cached_tokens(ctx + lo, dcp_size, dcp_rank, block_size);
      }
      emit(r);
      q_start += len;
    }
  }
  if (count > INT32_MAX) return PCP_EOVERFLOW;
  return static_cast<int>(count);
}

}  // namespace

extern "C" int pcp_plan_rows(int num_reqs, const int32_t* cu_seqlens_new, const int32_t* ctx_lens,
                             int pcp_size, int pcp_rank, int dcp_size, int dcp_rank,
                             int block_size, pcp_row_t* rows, int capacity) {
  return build_plan(num_reqs, cu_seqlens_new, ctx_lens, pcp_size, pcp_rank, dcp_size, dcp_rank,
                    block_size, false, rows, capacity);
}

extern "C" int pcp_plan_rows_resplit(int num_reqs, const int32_t* cu_seqlens_new,
                                     const int32_t* ctx_lens, int pcp_size, int pcp_rank,
                                     int dcp_size, int dcp_rank, int block_size, pcp_row_t* rows,
                                     int capacity) {
  return build_plan(num_reqs, cu_seqlens_new, ctx_lens, pcp_size, pcp_rank, dcp_size, dcp_rank,
                    block_size, true, rows, capacity);
}

// Cache slot of every new token (natural order) that this DCP rank writes, or
// -1: token i of request b sits at position p = ctx_lens[b] + i of logical
// block j = p / block_size, which DCP rank j mod dcp_size owns.
extern "C" int pcp_slot_mapping(int num_reqs, const int32_t* cu_seqlens_new,
                                const int32_t* ctx_lens, const int32_t* block_table,
                                int max_blocks, int dcp_size, int dcp_rank, int block_size,
                                int64_t* slots, int capacity) {
  if (num_reqs < 0 || max_blocks < 0 || dcp_size < 1 || dcp_rank < 0 || dcp_rank >= dcp_size ||
      block_size < 1 || capacity < 0)
    return PCP_EINVAL;
  if (num_reqs > 0 && (cu_seqlens_new == nullptr || ctx_lens == nullptr)) return PCP_EINVAL;
  if (capacity > 0 && slots == nullptr) return PCP_EINVAL;
  if (num_reqs > 0 && cu_seqlens_new[0] < 0) return PCP_EINVAL;
  for (int b = 0; b < num_reqs; ++b)
    if (cu_seqlens_new[b + 1] < cu_seqlens_new[b] || ctx_lens[b] < 0) return PCP_EINVAL;
  const int64_t total = num_reqs > 0 ? (int64_t)cu_seqlens_new[num_reqs] - cu_seqlens_new[0] : 0;
  if (total > INT32_MAX) return PCP_EOVERFLOW;
  for (int b = 0; b < num_reqs; ++b) {
    const int64_t n_new = (int64_t)cu_seqlens_new[b + 1] - cu_seqlens_new[b];
    for (int64_t i = 0; i < n_new; ++i) {
      const int64_t p = (int64_t)ctx_lens[b] + i;
      const int64_t j = p / block_size;
      int64_t slot = -1;
      if (j % dcp_size == dcp_rank) {
        if (j >= max_blocks || block_table == nullptr) return PCP_EINVAL;  // table too short
        const int32_t pb = block_table[(int64_t)b * max_blocks + j];
        if (pb < 0) return PCP_EINVAL;
        slot = (int64_t)pb * block_size + p % block_size;
      }
      const int64_t e = (int64_t)cu_seqlens_new[b] - cu_seqlens_new[0] + i;
      if (e < capacity) slots[e] = slot;
    }
  }
  return (int)total;
}
