/*
 * pcp_attn.h -- one prefill-context-parallel (PCP) rank's share of causal
 * grouped-query attention on one MI355X (gfx950).
 *
 * The calls follow the computation described on three pull-request pages
 * about context-parallel prefill in vLLM:
 *   [P1] "Feat/pcp qwen36 hybrid" (vllm-plugin-FL PR #299)
 *   [P2] "[MRv2] FlashAttention PCP support for GQA on MRv2" (vLLM PR #49564)
 *   [P3] "[MRv2][PCP] Carry the row plan in attention metadata; fix mixed
 *        prefill+decode crash" (fork PR #2)
 *
 * Conventions shared by every call:
 *   - Return value: 0 on success, a negative PCP_E* code on error (see
 *     pcp_strerror), or a documented non-negative count. No exception or
 *     abort crosses this boundary.
 *   - Every pointer is owned by the caller, scratch memory included (see
 *     pcp_context_workspace_bytes). Nothing is allocated, freed or cached
 *     inside the library, and calls are safe from several host threads. The
 *     one exception is pcp_attn_rank_share_noalloc, which keeps its scratch
 *     in a fixed per-device array of the library (see there).
 *   - Device calls are enqueued on the caller's stream and return without
 *     synchronising; errors found on the host are reported before anything
 *     is enqueued. No call reads device memory back to the host (the host
 *     passes every size that shapes a launch).
 *   - Device calls enqueue kernel launches only (no memset, copy or
 *     allocation), so they can be captured into a HIP graph and replayed;
 *     pcp_attn_rank_share_noalloc looks its scratch address up on its first
 *     call on a device, which belongs outside a capture.
 *   - bf16 data is passed as uint16_t bit patterns (pcp_bf16_t).
 *   - LSE is the natural logarithm of the softmax denominator, float32,
 *     laid out [num_q_heads, total_q]; an empty key set gives out = 0 and
 *     LSE = -inf.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef PCP_ATTN_H
#define PCP_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pcp_bf16_t;
typedef uint8_t pcp_fp8_t; /* an OCP E4M3 ("fn") code: bias 7, no infinities, max 448 */

enum {
  PCP_OK = 0,
  PCP_EINVAL = -1,       /* a null pointer, a negative size, inconsistent shapes or ranks */
  PCP_EUNSUPPORTED = -2, /* well-formed but not built: head_dim, group size, too many partials */
  PCP_EHIP = -3,         /* the HIP runtime refused a launch */
  PCP_EOVERFLOW = -4,    /* a size or offset does not fit the 32-bit fields of the plan */
  PCP_ESCRATCH = -5      /* pcp_attn_rank_share_noalloc: the call's partials exceed
                            PCP_NOALLOC_SCRATCH_BYTES */
};

/* Row kinds. */
enum { PCP_ROW_HEAD = 0, PCP_ROW_TAIL = 1, PCP_ROW_DECODE = 2 };

/*
 * One row of the rank-local plan: a contiguous run of one request's query
 * tokens held by this rank ([P3] section "Two things that fell out of (1)":
 * up to two rows per prefilling request, each with its own context length).
 *
 *   req            request index in the batch
 *   kind           PCP_ROW_HEAD / PCP_ROW_TAIL (the two zigzag chunks of a
 *                  prefill) or PCP_ROW_DECODE (a request with one new token)
 *   q_start        first row of this row's queries in the rank-local Q / out
 *                  buffers (running sum of q_len in plan order)
 *   q_len          number of queries (m)
 *   pos_start      absolute position of the first query (cached + offset)
 *   k_start        first row of the request's new-token K/V in the
 *                  all-gathered K/V buffers
 *   k_len          new-token keys seen by the row's last query (n); query t
 *                  sees new keys 0 .. n - m + t (end-aligned causal mask,
 *                  [P1] section Changes). 0 for decode rows.
 *   ctx_len        cached tokens every query of the row sees
 *   ctx_len_local  the part of them held by this decode-context-parallel
 *                  (DCP) rank
 */
typedef struct pcp_row {
  int32_t req;
  int32_t kind;
  int32_t q_start;
  int32_t q_len;
  int32_t pos_start;
  int32_t k_start;
  int32_t k_len;
  int32_t ctx_len;
  int32_t ctx_len_local;
} pcp_row_t;

/* Human-readable name of a return code (static storage, never NULL). */
const char* pcp_strerror(int code);

/*
 * pcp_plan_rows -- build this rank's row plan on the host.
 *
 * Zigzag (DualChunkSwap) split ([P3] "What made it removable": each PCP rank
 * owns a different row set): the new tokens of request b,
 * n_b = cu_seqlens_new[b+1] - cu_seqlens_new[b], are cut into 2P chunks
 * (P = pcp_size); chunk c holds floor(n_b / 2P) + (c < n_b mod 2P) tokens.
 * Rank r takes chunk r (head) then chunk 2P-1-r (tail), skipping empty
 * chunks. A request with n_b == 1 is a decode row, present on every rank
 * ([P3] comment on commit 97aad2056e: decode rows are replicated across PCP
 * ranks); its own K/V is already in the paged cache, so its context is
 * ctx_lens[b] + 1 tokens and its k_len is 0. Requests with n_b == 0 give no
 * row. Cached block j of a request lives on DCP rank j mod dcp_size; that
 * decides ctx_len_local.
 *
 * Arguments (all host memory):
 *   num_reqs         B >= 0
 *   cu_seqlens_new   [B+1] non-decreasing, cu_seqlens_new[0] >= 0
 *   ctx_lens         [B] cached tokens before each request's new tokens, >= 0
 *   pcp_size, pcp_rank   P >= 1, 0 <= pcp_rank < P
 *   dcp_size, dcp_rank   D >= 1, 0 <= dcp_rank < D
 *   block_size       tokens per KV-cache block, >= 1
 *   rows             [capacity] output; may be NULL when capacity == 0
 *   capacity         rows the caller provided
 *
 * Returns the number of rows R the plan needs (>= 0) and writes
 * min(R, capacity) of them; when R > capacity nothing past rows[capacity-1]
 * is touched and the caller may call again with a larger buffer (a plan
 * never silently overflows a buffer sized for requests: [P3], the 8-vs-14
 * crash). R <= 2 * (prefilling requests) + (decode requests).
 * Returns PCP_EINVAL for bad arguments, PCP_EOVERFLOW when an offset does
 * not fit int32.
 */
int pcp_plan_rows(int num_reqs, const int32_t* cu_seqlens_new, const int32_t* ctx_lens,
                  int pcp_size, int pcp_rank, int dcp_size, int dcp_rank, int block_size,
                  pcp_row_t* rows, int capacity);

/*
 * pcp_plan_rows_resplit -- the row plan of the re-split path ([P3] "What
 * made it removable": once the new tokens are in the cache, each row is
 * [0, row_start) from the cache plus its own new tokens, local).
 *
 * Same arguments, rows and contract as pcp_plan_rows; the fields differ for
 * prefill rows only:
 *   k_start        = q_start: the row's own K/V sit in the rank-local K/V
 *                    buffer in the same order as its queries
 *   k_len          = q_len: query t sees own keys 0..t (square causal)
 *   ctx_len        = pos_start: every position before the row's first query
 *                    (cached prefix and earlier chunks' new tokens)
 *   ctx_len_local  this DCP rank's part of those (block j on rank j mod D)
 * Decode rows are as in pcp_plan_rows, with k_start = q_start.
 * The paged cache must already hold the new tokens: see pcp_slot_mapping and
 * pcp_kv_cache_write. The rows go to pcp_attn_rank_share (or to
 * pcp_attn_context_paged plus pcp_attn_prefill over the rank-local K/V).
 */
int pcp_plan_rows_resplit(int num_reqs, const int32_t* cu_seqlens_new, const int32_t* ctx_lens,
                          int pcp_size, int pcp_rank, int dcp_size, int dcp_rank,
                          int block_size, pcp_row_t* rows, int capacity);

/*
 * pcp_slot_mapping -- where this DCP rank writes each new token in its paged
 * cache ([P3] comment on commit 97aad2056e: the gathered slot mapping masks
 * every entry a rank must not write; the writer skips negative slots).
 *
 * New token i of request b sits at position p = ctx_lens[b] + i, in logical
 * block j = p / block_size, owned by DCP rank j mod dcp_size. For the owner,
 * slots[t] = block_table[b * max_blocks + j] * block_size + p % block_size;
 * for every other rank slots[t] = -1. t counts new tokens in batch order from
 * cu_seqlens_new[0].
 *
 *   cu_seqlens_new, ctx_lens   host, as in pcp_plan_rows
 *   block_table   host [num_reqs, max_blocks] int32: the request's logical
 *                 blocks (all of them, before DCP sharding) -> pool blocks
 *   slots         host [capacity] int64 output; may be NULL when capacity == 0
 *
 * Returns the number of new tokens N and writes min(N, capacity) slots.
 * PCP_EINVAL for bad arguments or when an owned block is missing from the
 * table (index >= max_blocks or a negative entry).
 */
int pcp_slot_mapping(int num_reqs, const int32_t* cu_seqlens_new, const int32_t* ctx_lens,
                     const int32_t* block_table, int max_blocks, int dcp_size, int dcp_rank,
                     int block_size, int64_t* slots, int capacity);

/*
 * pcp_kv_cache_write -- write new tokens' K and V into the paged cache
 * before attention ([P3] "What made it removable": the write is ordered
 * before attention).
 *
 *   k, v           device [num_tokens, num_kv_heads, head_dim] bf16, 16-byte aligned
 *   slot_mapping   device [num_tokens] int64, e.g. from pcp_slot_mapping;
 *                  token t goes to slot s = block * block_size + offset;
 *                  negative slots (and slots >= num_blocks * block_size) are
 *                  skipped
 *   k_cache, v_cache  device [num_blocks, block_size, num_kv_heads, head_dim]
 *                  bf16, 16-byte aligned
 *   head_dim       64, 128 or 256
 * Two tokens mapped to one slot race (the pages' mappings never do).
 * Errors: PCP_EINVAL, PCP_EUNSUPPORTED (also when num_tokens * num_kv_heads
 * * head_dim / 8 does not fit 32-bit chunk indices, about 64 GiB per
 * tensor), PCP_EHIP.
 */
int pcp_kv_cache_write(const pcp_bf16_t* k, const pcp_bf16_t* v, const int64_t* slot_mapping,
                       int num_tokens, int num_kv_heads, int head_dim, pcp_bf16_t* k_cache,
                       pcp_bf16_t* v_cache, int num_blocks, int block_size, hipStream_t stream);

/*
 * pcp_kv_cache_write_fp8 -- the same write for an FP8 cache: k, v and the
 * caches hold E4M3 codes (one byte per value, 16-byte aligned). The codes
 * are copied as they are: the cache keeps the descales of the FP8 attention
 * calls (a written token takes its request's k_descale / v_descale).
 * Arguments and errors as in pcp_kv_cache_write.
 */
int pcp_kv_cache_write_fp8(const pcp_fp8_t* k, const pcp_fp8_t* v, const int64_t* slot_mapping,
                           int num_tokens, int num_kv_heads, int head_dim, pcp_fp8_t* k_cache,
                           pcp_fp8_t* v_cache, int num_blocks, int block_size,
                           hipStream_t stream);

/*
 * pcp_attn_prefill -- the new-token pass: every plan row's queries attend
 * over their request's new-token keys with end-aligned causal masking
 * ([P1] section Changes: K/V all-gather then end-aligned causal attention).
 * Query t of a row sees keys row.k_start + j for 0 <= j <= k_len - q_len + t.
 * Decode rows (k_len == 0) get out = 0, LSE = -inf.
 *
 *   q        device [total_q, num_q_heads, head_dim] bf16, row-major
 *   k, v     device [total_k, num_kv_heads, head_dim] bf16, row-major
 *   rows     device [num_rows] plan rows (for example from pcp_plan_rows)
 *   max_q_len  >= every row's q_len (sizes the launch)
 *   head_dim   64, 128 or 256; num_q_heads % num_kv_heads == 0
 *   softmax_scale  multiplies q.k before the softmax (usually 1/sqrt(d))
 *   out      device [total_q, num_q_heads, head_dim] bf16
 *   lse      device [num_q_heads, total_q] float32
 *
 * Only rows of the plan are written; query rows not covered by the plan
 * (padding) are left untouched ([P2] review: compute over real rows only).
 * A row whose fields fall outside [0, total_q) / [0, total_k) is skipped
 * without any memory access outside the buffers.
 *   unit_order, num_units  optional launch order: NULL (built-in order) or a
 *            device array of num_units entries written by pcp_attn_schedule
 *            (pass 0) for the same rows, max_q_len, heads and head_dim.
 *            Entries out of range, or -1, launch a workgroup that does nothing;
 *            a unit left out of the order leaves its outputs unwritten.
 *
 * num_rows == 0 is a valid no-op. Errors: PCP_EINVAL, PCP_EUNSUPPORTED
 * (also when k or v exceeds 4 GiB: rows are fetched with 32-bit offsets),
 * PCP_EHIP.
 */
int pcp_attn_prefill(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                     const pcp_row_t* rows, int num_rows, int total_q, int total_k,
                     int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                     float softmax_scale, pcp_bf16_t* out, float* lse,
                     const int32_t* unit_order, int num_units, hipStream_t stream);

/*
 * pcp_attn_context_paged -- the context pass: every plan row's queries
 * attend, without a mask, over the row's ctx_len_local cached tokens held by
 * this DCP rank ([P2] overview: attention over the sharded cached prefix
 * returning (out, lse)). Decode rows are served here in the same launch.
 * Local cached token i of request row.req is slot i % block_size of pool
 * block block_tables[row.req * max_blocks + i / block_size].
 * A row with ctx_len_local == 0 writes out = 0, LSE = -inf; it is never
 * skipped ([P3] "Two traps": an early return that skipped context attention
 * gave fluent, wrong output).
 *
 *   q               device [total_q, num_q_heads, head_dim] bf16
 *   k_cache,v_cache device [num_blocks, block_size, num_kv_heads, head_dim] bf16
 *   block_tables    device [num_reqs, max_blocks] int32, this rank's local
 *                   logical block -> pool block; entries past a row's
 *                   ctx_len_local are never read
 *   rows            device [num_rows]; row.req < num_reqs and
 *                   row.ctx_len_local <= max_blocks * block_size
 *   max_q_len       >= every row's q_len
 *   out, lse        as in pcp_attn_prefill
 *
 *   workspace       device float32 scratch of
 *                   pcp_context_workspace_bytes(num_rows, num_q_heads, head_dim,
 *                   decode_splits) bytes, 16-byte aligned; may be NULL when
 *                   decode_splits == 1. Its contents on entry do not matter
 *                   and are meaningless afterwards; two calls in flight at
 *                   once must not share it.
 *   decode_splits   1 .. 256. A decode row (q_len == 1, k_len == 0: one
 *                   query against a long cached context) is cut into this
 *                   many ranges of whole key tiles processed by separate
 *                   workgroups; each range's (out, lse) goes to the workspace
 *                   and a second kernel on the same stream combines them with
 *                   the lse_merge arithmetic. This fills the GPU when a batch
 *                   is mostly decode rows; other rows are unaffected.
 *   unit_order, num_units  as in pcp_attn_prefill, from pcp_attn_schedule
 *                   (pass 1) with the same decode_splits.
 *
 * k_cache, v_cache and block_tables may be NULL when max_blocks == 0. Out of
 * range block-table entries are clamped into the pool (the values are then
 * meaningless, but nothing outside the pool is read).
 * Errors: PCP_EINVAL (also decode_splits < 1, or > 1 with a NULL workspace),
 * PCP_EUNSUPPORTED (head_dim, group size, decode_splits > 256), PCP_EHIP.
 */
int pcp_attn_context_paged(const pcp_bf16_t* q, const pcp_bf16_t* k_cache,
                           const pcp_bf16_t* v_cache, int num_blocks, int block_size,
                           const int32_t* block_tables, int num_reqs, int max_blocks,
                           const pcp_row_t* rows, int num_rows, int total_q, int max_q_len,
                           int num_q_heads, int num_kv_heads, int head_dim,
                           float softmax_scale, pcp_bf16_t* out, float* lse,
                           float* workspace, int decode_splits, const int32_t* unit_order,
                           int num_units, hipStream_t stream);

/*
 * pcp_attn_rank_share -- the whole rank share in one launch: each work unit
 * streams the row's cached-context tiles of this DCP rank (as in
 * pcp_attn_context_paged) and then its new-token tiles (as in
 * pcp_attn_prefill, end-aligned causal) through one online softmax, and
 * writes the merged (out, LSE).
 *
 * This is the result of pcp_attn_context_paged and pcp_attn_prefill followed
 * by lse_merge of the two ([P2] overview: sharded cached-prefix attention
 * plus the prefill attention, merged by LSE; [P1] section Changes): a
 * softmax over the union of two disjoint key sets equals the LSE merge of
 * the softmaxes over each (up to rounding order). The partial outputs, their
 * re-read and the merge pass are not needed.
 *
 *   q, k, v, total_k          as in pcp_attn_prefill
 *   k_cache ... max_blocks    as in pcp_attn_context_paged
 *   rows, num_rows, total_q, max_q_len, heads, head_dim, softmax_scale,
 *   out, lse                  as in both
 *   workspace, decode_splits  as in pcp_attn_context_paged (decode rows have
 *                             no new-token keys, so their key-range partials
 *                             are the whole result once combined)
 *   unit_order, num_units     from pcp_attn_schedule (pass 2)
 *
 * Errors: the union of both calls' errors.
 */
int pcp_attn_rank_share(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                        int total_k, const pcp_bf16_t* k_cache, const pcp_bf16_t* v_cache,
                        int num_blocks, int block_size, const int32_t* block_tables,
                        int num_reqs, int max_blocks, const pcp_row_t* rows, int num_rows,
                        int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                        int head_dim, float softmax_scale, pcp_bf16_t* out, float* lse,
                        float* workspace, int decode_splits, const int32_t* unit_order,
                        int num_units, hipStream_t stream);

/* Size of the scratch array of pcp_attn_rank_share_noalloc, per device. */
#define PCP_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * pcp_attn_rank_share_noalloc -- pcp_attn_rank_share for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same launch, arguments and result,
 * without the workspace argument. The split-decode partials go to a scratch
 * array inside the library instead, PCP_NOALLOC_SCRATCH_BYTES (16 MiB) per
 * device, which each device the library runs on keeps until the process
 * ends; its address is looked up on the first call on a device (with that
 * device current). The call itself allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 *
 * The partials need num_rows * num_q_heads * decode_splits * (head_dim + 1)
 * * 4 bytes (pcp_context_workspace_bytes); a larger need returns
 * PCP_ESCRATCH and enqueues nothing (decode_splits == 1 needs none). The
 * array needs no clearing: every partial the combine reads is written by
 * the same call first. Every call on one device shares that device's array,
 * so two calls that overlap on one device (other streams, other host
 * threads) race and give wrong results; calls ordered on one stream do not.
 * The stream must belong to the current device.
 *
 * Errors: those of pcp_attn_rank_share, PCP_ESCRATCH, and PCP_EHIP when the
 * scratch address cannot be looked up.
 */
int pcp_attn_rank_share_noalloc(const pcp_bf16_t* q, const pcp_bf16_t* k, const pcp_bf16_t* v,
                                int total_k, const pcp_bf16_t* k_cache,
                                const pcp_bf16_t* v_cache, int num_blocks, int block_size,
                                const int32_t* block_tables, int num_reqs, int max_blocks,
                                const pcp_row_t* rows, int num_rows, int total_q, int max_q_len,
                                int num_q_heads, int num_kv_heads, int head_dim,
                                float softmax_scale, pcp_bf16_t* out, float* lse,
                                int decode_splits, const int32_t* unit_order, int num_units,
                                hipStream_t stream);

/*
 * FP8 variants of the three attention calls: Q, K and V are E4M3 codes with
 * descales ([P2] review thread on the context-attention call: the FP8
 * descales handed to the varlen attention call are shaped (sequences, KV
 * heads); the [P2] benchmarks run FP8 checkpoints).
 *
 * A value is its code times a descale indexed by (request, KV head):
 * query head h of request b reads q * q_descale[b * num_kv_heads + h / G]
 * (G = num_q_heads / num_kv_heads); every key and value of request b, new or
 * cached, of KV head j is k * k_descale[b * num_kv_heads + j] and
 * v * v_descale[b * num_kv_heads + j]. The result is the bf16 call's result
 * on those values (out bf16, LSE float32, same layouts); a per-layer scale
 * is the case of a constant table.
 *
 *   q, k, v, k_cache, v_cache   device, as in the bf16 calls with one byte
 *                               per element; 16-byte aligned
 *   q_descale, k_descale, v_descale   device float32 [num_reqs, num_kv_heads]
 *   num_reqs (pcp_attn_prefill_fp8)   rows of the descale tables; every
 *                               row's req must be below it
 *   other arguments             as in pcp_attn_prefill,
 *                               pcp_attn_context_paged, pcp_attn_rank_share;
 *                               unit_order from pcp_attn_schedule (the work
 *                               units are the same)
 *
 * Every descale a row uses must be finite and > 0 (an FP8 checkpoint's
 * scales are): the kernels fold q_descale * k_descale into the softmax scale
 * after taking each tile's row max of the unscaled scores, so a negative
 * product turns that max into a min and a zero one meets a masked key
 * (-inf * 0); either makes the output non-finite. The calls do not read the
 * tables on the host (they are device memory) and cannot reject such values.
 *
 * Errors: those of the bf16 call, and PCP_EINVAL for a missing or
 * misaligned descale table or a misaligned Q/K/V buffer. Rows naming a
 * request outside [0, num_reqs) are skipped, as in the context pass.
 */
int pcp_attn_prefill_fp8(const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v,
                         const pcp_row_t* rows, int num_rows, int total_q, int total_k,
                         int max_q_len, int num_reqs, int num_q_heads, int num_kv_heads,
                         int head_dim, float softmax_scale, const float* q_descale,
                         const float* k_descale, const float* v_descale, pcp_bf16_t* out,
                         float* lse, const int32_t* unit_order, int num_units,
                         hipStream_t stream);

int pcp_attn_context_paged_fp8(const pcp_fp8_t* q, const pcp_fp8_t* k_cache,
                               const pcp_fp8_t* v_cache, int num_blocks, int block_size,
                               const int32_t* block_tables, int num_reqs, int max_blocks,
                               const pcp_row_t* rows, int num_rows, int total_q, int max_q_len,
                               int num_q_heads, int num_kv_heads, int head_dim,
                               float softmax_scale, const float* q_descale,
                               const float* k_descale, const float* v_descale, pcp_bf16_t* out,
                               float* lse, float* workspace, int decode_splits,
                               const int32_t* unit_order, int num_units, hipStream_t stream);

int pcp_attn_rank_share_fp8(const pcp_fp8_t* q, const pcp_fp8_t* k, const pcp_fp8_t* v,
                            int total_k, const pcp_fp8_t* k_cache, const pcp_fp8_t* v_cache,
                            int num_blocks, int block_size, const int32_t* block_tables,
                            int num_reqs, int max_blocks, const pcp_row_t* rows, int num_rows,
                            int total_q, int max_q_len, int num_q_heads, int num_kv_heads,
                            int head_dim, float softmax_scale, const float* q_descale,
                            const float* k_descale, const float* v_descale, pcp_bf16_t* out,
                            float* lse, float* workspace, int decode_splits,
                            const int32_t* unit_order, int num_units, hipStream_t stream);

/*
 * pcp_context_workspace_bytes -- size of the workspace pcp_attn_context_paged
 * or pcp_attn_rank_share needs for these arguments: num_rows * num_q_heads * decode_splits *
 * (head_dim + 1) * 4 bytes, or 0 when decode_splits == 1 or an argument is
 * invalid (negative, or an unsupported head_dim). Host only.
 */
size_t pcp_context_workspace_bytes(int num_rows, int num_q_heads, int head_dim,
                                   int decode_splits);

/*
 * pcp_choose_decode_splits -- the decode_splits to pass to
 * pcp_attn_context_paged (fused == 0) or pcp_attn_rank_share (fused != 0)
 * for this plan: how many key ranges each decode row is cut into ([P2]
 * overview and [P3] comment on commit 97aad2056e: decode rows of a mixed
 * batch go through the same context attention; the ranges' partials are
 * combined by the LSE merge of [P2]'s benchmark notes).
 *
 * A decode row (q_len == 1, k_len <= 0) is one workgroup per KV head
 * streaming its cached context, and one workgroup fills a compute unit. The
 * rule, for MI355X's 256 compute units:
 *   - 1 when the plan has no decode row with cached keys, or when the launch
 *     already has 512 workgroups with work: (decode rows + the sum over the
 *     other rows with keys in the pass of ceil(q_len / 128)) * num_kv_heads.
 *     Splitting would then only add per-workgroup latency and a combine pass.
 *   - otherwise the longest decode row is cut so that each range holds no
 *     more keys than one compute unit's even share of all decode keys
 *     (sum of ctx_len_local * num_kv_heads / 256), and no fewer than about
 *     256 keys: ceil(longest / max(share, 256)), at most 256.
 *
 *   rows          host [num_rows], the plan the attention call will get
 *   num_kv_heads  >= 1
 *   fused         0: a context pass (rows count with cached keys); else a
 *                 fused launch (rows count with cached or new-token keys)
 *
 * Returns the split count (1 .. 256), or PCP_EINVAL (num_rows < 0,
 * num_kv_heads < 1, rows NULL with num_rows > 0). Host only.
 */
int pcp_choose_decode_splits(const pcp_row_t* rows, int num_rows, int num_kv_heads, int fused);

/*
 * pcp_attn_schedule -- launch order of the work units of one attention call,
 * built on the host from the plan.
 *
 * The attention calls split their work into units of (row, KV head's group
 * of query heads, query tile, or key range of a split one-query row). Units
 * differ in length: the end-aligned causal mask ([P1] section Changes) gives
 * a row's query tiles from k_len - q_len + BQ up to k_len keys, and a mixed
 * batch mixes rows of very different lengths ([P3] "Two things that fell out
 * of (1)"). Launching them longest first keeps all compute units busy to the
 * end. MI355X deals workgroups to its 8 XCDs round-robin, each with its own
 * L2: the order keeps runs of neighbouring query tiles of one row and head
 * group, which read overlapping K/V, on one XCD, balances the XCDs' work and
 * sorts each XCD's units longest first. When a model of the dispatch finds
 * that order less than 1% faster than the kernels' built-in one (typical for
 * a single long prompt), the built-in order is returned instead. When the
 * call's K/V exceeds the 256 MB Infinity Cache and
 * every (request, KV head) group of units is at most 1/32 of the work, whole
 * groups are placed on XCDs instead, longest first, each group's units
 * together and longest first, so that a group's keys are read from HBM once
 * per group rather than once per XCD.
 *
 *   pass           0 for pcp_attn_prefill, 1 for pcp_attn_context_paged,
 *                  2 for pcp_attn_rank_share
 *   rows           host [num_rows], the rows the attention call will get
 *   max_q_len, num_q_heads, num_kv_heads, head_dim
 *                  as the attention call will get them
 *   decode_splits  as the attention call will get it (passes 1 and 2;
 *                  pass 0 ignores it but it must be >= 1)
 *   kv_elem_bytes  bytes per K/V element of the attention call: 2 (bf16) or
 *                  1 (E4M3); it sizes the call's K/V footprint
 *   order          host [capacity] output; may be NULL when capacity == 0
 *
 * Returns the number of entries N (-1 entries included) and writes
 * min(N, capacity) of them; call again with a larger buffer when
 * N > capacity. Errors: PCP_EINVAL (bad sizes, a row's q_len outside
 * [0, max_q_len], inconsistent heads, kv_elem_bytes not 1 or 2),
 * PCP_EUNSUPPORTED (head_dim),
 * PCP_EOVERFLOW. Host only; the result depends only on the arguments.
 */
int pcp_attn_schedule(int pass, const pcp_row_t* rows, int num_rows, int max_q_len,
                      int num_q_heads, int num_kv_heads, int head_dim, int decode_splits,
                      int kv_elem_bytes, int32_t* order, int capacity);

/*
 * lse_merge -- combine k partial results over disjoint key sets into the
 * result over their union ([P2] Qwen3-30B-A3B-FP8 benchmark: LSE combine of
 * DCP partials; [P3] "What made it removable": the LSE combine over ranks).
 * For each (query, head): M = max_i lse_i; w_i = exp(lse_i - M);
 * lse = M + log(sum_i w_i); out = sum_i w_i * out_i / sum_i w_i, in float32.
 * All lse_i == -inf gives out = 0, lse = -inf.
 *
 *   k        1 <= k <= 16 partials
 *   outs     host array [k] of device pointers, each [total_q, num_q_heads, head_dim] bf16
 *   lses     host array [k] of device pointers, each [num_q_heads, total_q] float32
 *   out      device [total_q, num_q_heads, head_dim] bf16; may alias outs[0]
 *   lse_out  device [num_q_heads, total_q] float32; may alias lses[0]
 *   head_dim 64, 128 or 256
 */
int lse_merge(int k, const pcp_bf16_t* const* outs, const float* const* lses, int total_q,
              int num_q_heads, int head_dim, pcp_bf16_t* out, float* lse_out,
              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PCP_ATTN_H */
