// Attention kernel of libpcpattn (internal header): the flash-attention
// style kernel template for one PCP rank's share of causal GQA attention --
// the end-aligned causal new-token pass, the paged context pass over this DCP
// rank's cache shard (decode rows included) and both fused in one launch --
// with its tile geometry, the split-decode combine and the launch dispatch.
// The bf16 and the FP8 entry points instantiate it in their own translation
// units.
//
// Method: "Feat/pcp qwen36 hybrid" (vllm-plugin-FL PR #299), section Changes
// (local query rows against all-gathered K/V, end-aligned causal mask);
// "[MRv2] FlashAttention PCP support for GQA on MRv2" (vLLM PR #49564),
// overview (attention over the sharded cached prefix returning (out, lse),
// mixed prefill + decode batches), its Qwen3-30B-A3B-FP8 benchmark notes
// (LSE combine of DCP partials) and the FP8 descales of its context-attention
// call. The kernel is a flash-attention style single pass with an online
// softmax (Dao, FlashAttention-2, 2023), designed for CDNA4 as follows.
//
// Work unit: one workgroup of 8 waves takes BQ = 256/HG consecutive queries
// of one row for HG query heads that share one KV head (GQA packing), so all
// 8 waves consume the same K/V tile. Each wave owns 32 queries of one head.
//
// Per key tile of BN keys (K and V row-major in LDS, filled straight from
// global memory by buffer loads into LDS, through a ring of 3 stages with one
// barrier per tile and two tiles of loads in flight):
//   S^T = K Q^T      bf16: v_mfma_f32_32x32x16_bf16; E4M3: 32x32x64_f8f6f4.
//                    A = K rows from LDS (ds_read_b128), B = Q^T held in
//                    registers for the whole unit. In the accumulator layout
//                    each lane owns one query (lane % 32) and 16 keys, so the
//                    softmax row max/sum are 16 in-lane ops plus one exchange
//                    between the wave's two 32-lane halves.
//   P^T = exp2(S^T * scale*log2e - m)   (online softmax, stale-max rescaling:
//                    the reference max only moves when a tile's max exceeds
//                    it by more than 2^8, which keeps P <= 256 and makes the
//                    O rescale rare; exact, no approximation). P is bf16.
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, B = P^T straight from the S^T
//                    accumulators (no data movement: the key order inside a
//                    16-key step is permuted identically on both operands).
//                    A = V^T: bf16 V is read with ds_read_b64_tr_b16 (4 keys
//                    of one d column per lane and read); E4M3 V with
//                    ds_read_b64_tr_b8 (8 keys) and widened to bf16 exactly.
// FP8: the Q and K descales of the unit's (request, KV head) fold into the
// softmax scale, the V descale into the final normalisation.
// LDS swizzles (gfx950 LDS: 64 banks of 4 bytes, so a 16-byte slot index
// mod 16 names its bank group): K slots are XORed so that the 16 keys one
// ds_read_b128 cycle touches hit 16 bank groups; V slots so that the keys x
// slots one transposed-read cycle touches are distinct (see Attn::swz_k and
// Attn::swz_v).

#ifndef PCP_ATTN_FWD_H
#define PCP_ATTN_FWD_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "pcp_attn.h"
#include "pcp_attn_check.h"
#include "pcp_geometry.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x4_t lds_i32x4_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

// Tuning knobs (the defaults are the measured best on MI355X).
#ifndef PCP_STAGES
#define PCP_STAGES 3  // LDS ring depth: 2 (two barriers per tile), 3 or 4 (one barrier
                      // per tile, 2 or 3 tiles of loads in flight)
#endif
#ifndef PCP_SCHED_QK
#define PCP_SCHED_QK 1  // 1: pin the QK order to (K read, MFMA) pairs KPREF reads ahead
#endif
#ifndef PCP_SCHED_PV
#define PCP_SCHED_PV 1  // 1: pin the PV order to (MFMA, 2 V^T reads) pairs VPREF ahead
#endif
#ifndef PCP_KPREF
#define PCP_KPREF 3  // K operand fragments read ahead of their MFMA
#endif
#ifndef PCP_VPREF
#define PCP_VPREF 3  // V operand fragments read ahead of their MFMA
#endif
#ifndef PCP_PERMLANE
#define PCP_PERMLANE 1  // 1: exchange the two 32-lane halves with v_permlane32_swap (VALU)
#endif
#ifndef PCP_LAUNDER_MIN_D
#define PCP_LAUNDER_MIN_D 256  // head dims from which the LDS operand offsets are recomputed
                               // every tile (fewer registers, more VALU); below it they stay
                               // in registers across the loop
#endif
#ifndef PCP_DECODE_PACK
#define PCP_DECODE_PACK 1  // 1: a decode row's heads share wave 0's query slots
#endif
#ifndef PCP_SKIP_MASKED
#define PCP_SKIP_MASKED 1  // 1: a wave skips new-token tiles past its queries' causal bound
#endif
#ifndef PCP_DECODE_16
#define PCP_DECODE_16 1  // 1: decode units of a context pass run on 16x16 MFMAs (heads in 16 columns)
#endif

constexpr int kWaves = pcp_geom::kWaves;
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves per workgroup");
constexpr int kThreads = kWaves * 64;
constexpr int kStages = PCP_STAGES;
static_assert(kStages >= 2 && kStages <= 4, "2, 3 or 4 LDS stages");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kRescaleTau = 8.0f;  // log2 units: P stays <= 2^8 between rescales
constexpr float kNegInf = -INFINITY;

struct AttnArgs {
  // Q/K/V elements are bf16, or E4M3 codes in the FP8 kernels.
  const void* q;   // [total_q, hq, D]
  const void* k;   // new-token K/V: [total_k, hkv, D]
  const void* v;
  const void* kc;  // paged cache K/V: [num_blocks, block_size, hkv, D]
  const void* vc;
  // FP8 kernels: descales [num_reqs, hkv] (a value is code * descale of its
  // request and KV head; a query uses its head's KV head).
  const float* q_ds;
  const float* k_ds;
  const float* v_ds;
  const pcp_row_t* rows;
  const int32_t* block_tables;
  u16* out;
  float* lse;
  int num_rows;
  int total_q;
  int total_k;
  int num_blocks;
  int block_size;
  // key / block_size for 0 <= key < 2^31 as (mulhi(key, bs_magic) + key) >>
  // bs_shift (round-up multiplier: Granlund and Montgomery, "Division by
  // invariant integers using multiplication", 1994, section 4), set by the
  // launcher; the kernels divide keys by block_size every tile.
  uint32_t bs_magic;
  uint32_t bs_shift;
  int num_reqs;
  int max_blocks;
  int hq;
  int hkv;
  int group;          // hq / hkv
  int groups_per_kv;  // group / HG
  int q_tiles;        // ceil(max_q_len / BQ)
  int num_units;
  float scale_log2;   // softmax_scale * log2(e)
  // Context pass only: rows with one query are split into dec_splits key
  // ranges whose partials go to ws: out as [num_rows][hq][dec_splits][D]
  // floats, then lse as [num_rows][hq][dec_splits] floats; they are merged
  // afterwards by decode_combine_kernel.
  float* ws;
  int dec_splits;
  // Optional launch order (device, one unit id per workgroup, -1 = none):
  // unit id = (row * groups + group) * q_tiles + q_tile.
  const int32_t* order;
  int has_new;  // the launch also runs the new-token tiles (fused pass)
};

// Workgroups are dealt to the 8 XCDs round-robin by launch index. Remap so
// that each XCD receives runs of kXcdRun consecutive work units (the same row
// and KV head, neighbouring query tiles), which then share K/V in that XCD's
// L2. Units stay in roughly the same launch order, so the longest-first order
// of the unit list survives.
constexpr int kXcds = pcp_geom::kXcds;
constexpr int kXcdRun = pcp_geom::kXcdRun;

__device__ __forceinline__ int xcd_remap(int b, int n) {
  constexpr int W = kXcds * kXcdRun;
  const int full = (n / W) * W;
  if (b >= full) return b;
  const int win = b / W;
  const int within = b - win * W;
  return win * W + (within % kXcds) * kXcdRun + within / kXcds;
}

// Tags of the key phases of a work unit: cached context, new-token keys, and
// the cached context of a decode unit on the 16x16 layout.
struct CtxPhase {
  static constexpr bool ctx = true;
  static constexpr bool dec = false;
};
struct NewPhase {
  static constexpr bool ctx = false;
  static constexpr bool dec = false;
};
struct DecPhase {
  static constexpr bool ctx = true;
  static constexpr bool dec = true;
};

// max / sum of a value over lanes l and l ^ 32: the accumulator layouts keep
// one query's keys in the two 32-lane halves of a wave.
__device__ __forceinline__ float halves_max(float x) {
  if constexpr (PCP_PERMLANE != 0) {
    // v_permlane32_swap with both operands x gives every lane x[lane % 32]
    // and x[32 + lane % 32]: no LDS round trip as with ds_bpermute.
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(x, __shfl_xor(x, 32));
  }
}
__device__ __forceinline__ float halves_sum(float x) {
  if constexpr (PCP_PERMLANE != 0) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return x + __shfl_xor(x, 32);
  }
}

// max / sum over lanes l, l ^ 16, l ^ 32 and l ^ 48: the 16x16 accumulator
// layout spreads one column's rows over the four 16-lane groups of a wave.
// v_permlane16_swap with both operands x gives every lane x of its own
// position in the two 16-lane rows of its pair, as permlane32_swap does for
// the two halves.
__device__ __forceinline__ float quad_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return halves_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

__device__ __forceinline__ void block_barrier() {
  // s_barrier without the workgroup-scope fences of __syncthreads(): those
  // would force every outstanding global_load_lds (the next tile) to finish.
  // The memory clobber keeps the compiler from moving LDS accesses across.
  asm volatile("s_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ uint32_t div_block(uint32_t key, const AttnArgs& a) {
  return (__umulhi(key, a.bs_magic) + key) >> a.bs_shift;
}

// The K or the V buffer descriptor of a chunk, or `none` when the tile is
// past the last one (chosen by value: selecting between the variables as
// lvalues can leave them in scratch memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pick_rsrc(bool live, bool v,
                                                            __amdgpu_buffer_rsrc_t vr,
                                                            __amdgpu_buffer_rsrc_t kr,
                                                            __amdgpu_buffer_rsrc_t none) {
  return live ? (v ? vr : kr) : none;
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

// Q^T operand fragment of one QK^T MFMA: 8 bf16, or 32 E4M3 codes.
template <bool FP8>
struct Frag {
  typedef bf16x8_t type;
};
template <>
struct Frag<true> {
  typedef i32x8_t type;
};

// Tile geometry; EB = bytes per Q/K/V element (2: bf16, 1: E4M3).
template <int D, int BN, int HG, int EB>
struct Attn {
  static constexpr int BQ = 32 * kWaves / HG;  // queries per workgroup
  static_assert(HG <= kWaves, "each wave holds one head");
  static constexpr int RB = D * EB;            // bytes per key row
  static constexpr int NQC = EB == 2 ? D / 16 : D / 64;  // d steps of QK^T (one MFMA each)
  static constexpr int NDB = D / 32;           // 32-wide d blocks of O^T
  static constexpr int NJ = BN / 32;           // 32-key S^T accumulators per tile
  static constexpr int NKC = BN / 16;          // 16-key steps of PV
  static constexpr int KCH = BN * RB / 1024;   // 1 KB chunks of the K tile (same for V)
  static constexpr int CPW = 2 * KCH / kWaves; // chunks each wave loads per tile
  static constexpr int RPC = 1024 / RB;        // key rows per 1 KB chunk
  static constexpr int SPR = RB / 16;          // 16-byte slots per key row
  static constexpr int STAGE = 2 * BN * RB;    // bytes per stage (K then V)
  // 16x16x32 layout of decode units (bf16): QK^T steps of 32 d, 16-key S^T
  // blocks, 32-key PV steps, 16-wide d blocks of O^T.
  static constexpr int NC16 = EB == 2 ? D / 32 : D / 128;  // E4M3: 16x16x128 QK^T steps
  static constexpr int NB16 = BN / 16;
  static constexpr int NKS16 = BN / 32;
  static constexpr int NDB16 = D / 16;
  static_assert((2 * KCH) % kWaves == 0, "tile must split evenly over waves");
  static_assert(SPR >= (EB == 2 ? 8 : 4), "swizzles need 8 (bf16) or 4 (E4M3) slots per row");
  // XOR applied to the 16-byte slot index of key row r within a tile. K: the
  // 16 rows one ds_read_b128 cycle touches land in 16 bank groups (rows that
  // share a 256-byte bank sweep are told apart by their position in it).
  static __device__ __forceinline__ int swz_k(int r) {
    return SPR >= 16 ? (r & 15) : ((r >> (SPR == 8 ? 1 : 2)) & (SPR - 1));
  }
  // V, bf16 (ds_read_b64_tr_b16): 4 keys x 4 slots per cycle are distinct.
  // V, E4M3 (ds_read_b64_tr_b8): the 8 keys one 32-lane half reads (bits 0,
  // 1 and 3 of the key vary) x 2 slots; an even XOR keeps each slot's low bit.
  static __device__ __forceinline__ int swz_v(int r) {
    if constexpr (EB == 2) {
      return SPR >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
    } else if constexpr (SPR >= 16) {
      return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
    } else if constexpr (SPR == 8) {
      return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    } else {
      return 2 * ((r >> 3) & 1);
    }
  }
  // V of a decode unit, bf16: one transposed-read cycle (32 lanes) touches 8
  // consecutive keys x 2 adjacent slots; an even XOR that differs over those
  // 8 keys (rows of 256 bytes and more), or over their row pairs (128-byte
  // rows, whose odd rows start half a bank sweep later), keeps the 16 cells
  // in 16 bank groups.
  // E4M3 (ds_read_b64_tr_b8): a 32-lane half reads 16 keys, r and r + 16 for
  // r in 8 consecutive keys, one whole slot each; the XOR differs over them
  // (256-byte rows) or over each parity class (128-byte rows).
  static __device__ __forceinline__ int swz_vd(int r) {
    if constexpr (EB == 2) {
      return SPR >= 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
    } else {
      return SPR >= 16 ? ((r & 7) | (((r >> 4) & 1) << 3)) : (((r >> 1) & 3) | (((r >> 4) & 1) << 2));
    }
  }
};

// MODE 0: new-token pass (contiguous K/V). MODE 1: context pass, block_size a
// multiple of the key rows per 1 KB chunk (block ids fetched per chunk with
// scalar loads). MODE 2: context pass, any block_size (per-lane lookups).
// MODE 3 / 4: both passes fused in one unit (context tiles as in MODE 1 / 2,
// then the new-token tiles), one softmax state, the merged result written.
// FP8: Q/K/V are E4M3 codes with per-(request, KV head) descales.
// The launch bound (kThreads per workgroup, one workgroup per CU) puts
// kWaves / 4 waves on each SIMD and caps a wave's registers accordingly; the
// waves-per-EU hint does not change the code's speed (a (2, 2) hint at eight
// waves measured the same).
template <int D, int BN, int HG, int MODE, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8 / kWaves, 8 / kWaves)))
void attn_fwd_kernel(const AttnArgs a) {
  constexpr bool HAS_CTX = MODE != 0;              // paged cached-context tiles
  constexpr bool HAS_NEW = MODE == 0 || MODE >= 3;  // contiguous new-token tiles
  constexpr int EB = FP8 ? 1 : 2;                   // bytes per Q/K/V element
  using C = Attn<D, BN, HG, EB>;
  // Separate objects per stage: the compiler then tells the stage being read
  // from the stages being filled and keeps the prefetch outstanding.
  __shared__ __attribute__((aligned(16))) char smem0[C::STAGE];
  __shared__ __attribute__((aligned(16))) char smem1[C::STAGE];
  __shared__ __attribute__((aligned(16))) char smem2[kStages >= 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char smem3[kStages >= 4 ? C::STAGE : 16];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work unit: (row, group of HG heads, query tile)
  const int groups_total = a.hkv * a.groups_per_kv;
  int row_id, grp, qtile;
  if (a.order != nullptr) {  // host-made schedule
    const int uid = a.order[blockIdx.x];
    if (uid < 0 || uid >= a.num_units) return;
    qtile = uid % a.q_tiles;
    const int rest = uid / a.q_tiles;
    grp = rest % groups_total;
    row_id = rest / groups_total;
  } else {  // rows in reverse plan order, query tiles last to first, runs per XCD
    const int u = xcd_remap(blockIdx.x, a.num_units);
    const int qt_rev = u % a.q_tiles;
    const int rest = u / a.q_tiles;
    grp = rest % groups_total;
    row_id = a.num_rows - 1 - rest / groups_total;
    qtile = a.q_tiles - 1 - qt_rev;
  }
  const pcp_row_t row = a.rows[row_id];
  // A decode row (one query, no new-token keys) may be split over its
  // cached keys: the query-tile slot then numbers the split.
  const bool split = HAS_CTX && a.dec_splits > 1 && row.q_len == 1 && row.k_len <= 0;
  const int split_id = split ? qtile : 0;
  if (split && split_id >= a.dec_splits) return;
  const int q0 = split ? 0 : qtile * C::BQ;
  if (row.q_len <= q0) return;
  if (row.q_start < 0 || row.q_start > a.total_q - row.q_len) return;

  // Keys of the unit: nctx cached ones (context tiles first), then nnew new
  // ones up to the causal bound of the unit's last query.
  int nctx = 0, nnew = 0;
  if (HAS_CTX || FP8) {  // the request indexes the block table / the descales
    if (row.req < 0 || row.req >= a.num_reqs) return;
  }
  if constexpr (HAS_CTX) {
    nctx = row.ctx_len_local;
    if (nctx < 0 || (int64_t)nctx > (int64_t)a.max_blocks * a.block_size) return;
  }
  if constexpr (HAS_NEW) {
    if (row.k_start < 0 || row.k_len < 0 || row.k_start > a.total_k - row.k_len) return;
    const int t_last = min(q0 + C::BQ, row.q_len) - 1;
    nnew = max(0, min(row.k_len, row.k_len - row.q_len + t_last + 1));
  }
  const int ctx_tiles = (nctx + BN - 1) / BN;
  const int nkeys = nctx + nnew;

  const int kvh = grp / a.groups_per_kv;
  const int head0 = kvh * a.group + (grp % a.groups_per_kv) * HG;
  // A decode row (one query, no new-token keys) packs the unit's HG heads
  // into the query slots of wave 0 (slot l32 < HG is head head0 + l32), so
  // one wave's MFMAs serve all of them; the other waves only load tiles.
  // Otherwise each wave holds 32 queries of one head.
  // Decode units of a context pass run on the 16x16 layout (16x16x32 bf16;
  // E4M3 QK^T on 16x16x128, d >= 128), whose 16 query columns (lane % 16)
  // hold the heads. Not in the fused launch: at
  // d = 256 its new-token loop uses all 256 registers, and the extra code
  // path there moves register spills into that loop.
  const bool pack = PCP_DECODE_PACK != 0 && HAS_CTX && row.q_len == 1 && row.k_len <= 0;
  constexpr bool kDec16 = PCP_DECODE_16 != 0 && PCP_DECODE_PACK != 0 &&
                         (MODE == 1 || MODE == 2) && (!FP8 || D >= 128);
  const bool dec16 = kDec16 && pack;
  const int qcol = dec16 ? (lane & 15) : l32;
  const int head = pack ? head0 + min(qcol, HG - 1) : head0 + (wave % HG);
  const int t0 = pack ? 0 : q0 + 32 * (wave / HG);
  const bool wave_active = pack ? wave == 0 : t0 < row.q_len;
  const int t = pack ? 0 : t0 + l32;
  const bool q_valid = pack ? qcol < HG : t < row.q_len;

  // Softmax scale (log2 units) and output factor of the unit: FP8 folds the
  // Q and K descales into the first and the V descale into the second.
  float scale_log2 = a.scale_log2;
  float out_scale = 1.0f;
  if constexpr (FP8) {
    const int di = row.req * a.hkv + kvh;
    scale_log2 *= a.q_ds[di] * a.k_ds[di];
    out_scale = a.v_ds[di];
  }

  // ---- Q^T operand, held for the whole unit: lane owns query t; bf16
  // d = 16c + 8hh + [0,8), E4M3 d = 64c + 32hh + [0,32) (the K fragments
  // take the same d of their key, so the d order inside a step is the same
  // on both operands and the product is the full dot product).
  typename Frag<FP8>::type qf[C::NQC];
  if (q_valid && nkeys > 0 && !dec16) {  // no keys: the output is (0, -inf), Q is not needed
    if constexpr (FP8) {
      const uint8_t* qp =
          (const uint8_t*)a.q + ((size_t)(row.q_start + t) * a.hq + head) * D + 32 * hh;
#pragma unroll
      for (int c = 0; c < C::NQC; ++c) {
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(qp + 64 * c);
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(qp + 64 * c + 16);
        qf[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    } else {
      const u16* qp = (const u16*)a.q + ((size_t)(row.q_start + t) * a.hq + head) * D + 8 * hh;
#pragma unroll
      for (int c = 0; c < C::NQC; ++c) qf[c] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * c);
    }
  } else {
#pragma unroll
    for (int c = 0; c < C::NQC; ++c) qf[c] = typename Frag<FP8>::type{};
  }

  const size_t key_stride = (size_t)a.hkv * D;  // elements
  const int32_t* btab = HAS_CTX ? a.block_tables + (size_t)row.req * a.max_blocks : nullptr;

  // Per-lane constants of the tile loads: chunk ci (K chunks first, then V)
  // covers key rows cc * RPC .. and this lane fetches row r, logical slot ls,
  // stored at physical slot ps (the swizzle is applied on the global side
  // because global/buffer loads into LDS write 16 consecutive bytes per lane).
  int lrow[C::CPW];
  int lslot[C::CPW];
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) {
    const int ci = wave * C::CPW + i;
    const bool isv = ci >= C::KCH;
    const int cc = isv ? ci - C::KCH : ci;
    const int r = cc * C::RPC + lane / C::SPR;
    const int ps = lane % C::SPR;
    lrow[i] = r;
    lslot[i] = ps ^ (isv ? (dec16 ? C::swz_vd(r) : C::swz_v(r)) : C::swz_k(r));
  }

  // New-token pass: K/V rows of the request are contiguous; buffer loads with
  // 32-bit offsets from the row's first key (reads past the buffer return 0,
  // reads past nkeys inside it return finite keys that the mask removes).
  __amdgpu_buffer_rsrc_t krsrc, vrsrc;
  uint32_t lane_off[C::CPW];
  if constexpr (HAS_NEW) {
    const size_t first = ((size_t)row.k_start * key_stride + (size_t)kvh * D) * EB;
    const char* kb = (const char*)a.k + first;
    const char* vb = (const char*)a.v + first;
    const uint64_t left = ((uint64_t)(a.total_k - row.k_start) * key_stride - (uint64_t)kvh * D) * EB;
    const int nrec = (int)(left > 0xFFFFFFFFull ? 0xFFFFFFFFull : left);
    krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, nrec, 0x00020000);
    vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, nrec, 0x00020000);
  }
  // Byte offset of each chunk's lane from the tile's first row: rows are
  // key_stride elements apart in the new-token K/V and within a cache block.
  if constexpr (HAS_NEW || MODE == 1 || MODE == 3) {
#pragma unroll
    for (int i = 0; i < C::CPW; ++i)
      lane_off[i] = (uint32_t)lrow[i] * (uint32_t)(key_stride * EB) + (uint32_t)lslot[i] * 16u;
  }

  // Fill one stage with the K and V rows of a tile.
  // Context pass, block_size a multiple of RPC: the RPC keys of one chunk
  // instruction lie in one cache block, so the block id is wave-uniform. It
  // is fetched with a scalar load one tile ahead (scalar loads do not share
  // the vector memory counter, so fetching it never waits for the K/V tiles
  // in flight) and the block base rides in the instruction's SGPR address.
  constexpr bool uniform_blocks = MODE == 1 || MODE == 3;
  // Uniform blocks: one buffer descriptor per pool over this KV head's rows
  // (the launcher takes this path only for pools under 4 GiB, so 32-bit
  // offsets reach every block); a chunk's block enters as the scalar offset
  // block * block_bytes, its rows as per-lane offsets within the block.
  __amdgpu_buffer_rsrc_t kpool, vpool;
  const uint32_t block_bytes = (uint32_t)((size_t)a.block_size * key_stride * EB);
  if constexpr (uniform_blocks) {
    const uint64_t head_off = (uint64_t)kvh * D * EB;
    const uint64_t pool = (uint64_t)a.num_blocks * block_bytes;
    const int nrec = (int)(uint32_t)(pool - head_off);
    kpool = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.kc + head_off), (short)0,
                                              nrec, 0x00020000);
    vpool = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.vc + head_off), (short)0,
                                              nrec, 0x00020000);
  }
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const_i32_ptr btab_s = (const_i32_ptr)btab;
  int bt_next[C::CPW];       // pool block of each chunk of the next tile to issue (as read)
  uint32_t lb_next[C::CPW];  // and its logical block
  // The ids are loaded back to back and clamped only where the tile is
  // issued, after the next barrier: a clamp here would wait for each load in
  // turn, and the wait there overlaps the wait for the current tile.
  // A wave's chunks are CPW * RPC consecutive rows of the tile from row r0, a
  // multiple of CPW * RPC. When block_size is a multiple of that too, they
  // lie in one cache block, and a full tile needs one block id per wave: the
  // chunks then differ only by their lanes' row offsets (lane_off), as in the
  // new-token tiles. The last, partial tile clamps its keys chunk by chunk.
  // Compiled where a wave spans at most 16 rows, so that 16-key blocks (and
  // any multiple) qualify; elsewhere the extra path only costs registers.
  constexpr bool kOneBlock = C::CPW * C::RPC <= 16;
  const bool wave_blocks = kOneBlock && a.block_size % (C::CPW * C::RPC) == 0;
  const int r0 = ((wave * C::CPW) % C::KCH) * C::RPC;
  auto one_block = [&](int tile) { return wave_blocks && (tile + 1) * BN <= nctx; };
  auto fetch_blocks = [&](int tile) {
    if (kOneBlock && one_block(tile)) {
      const uint32_t lb = __builtin_amdgcn_readfirstlane(div_block((uint32_t)(tile * BN + r0), a));
      const int bt = btab_s[lb];
#pragma unroll
      for (int i = 0; i < C::CPW; ++i) {
        lb_next[i] = lb;
        bt_next[i] = bt;
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) {
      const int ci = wave * C::CPW + i;
      const int cc = ci >= C::KCH ? ci - C::KCH : ci;
      const int key0 = min(tile * BN + cc * C::RPC, nctx - 1);
      const uint32_t lb = __builtin_amdgcn_readfirstlane(div_block((uint32_t)key0, a));
      lb_next[i] = lb;
      bt_next[i] = btab_s[lb];
    }
  };

  // Tiles are numbered within their phase (CtxPhase: cached context of this
  // DCP rank, NewPhase: new-token keys).
  // A tile past the last one (live false) is issued with a descriptor of no
  // records: the loads read nothing and write zeros to the stage (see run).
  const __amdgpu_buffer_rsrc_t no_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.q, (short)0, 0, 0x00020000);
  auto issue = [&](auto phase, char* stage, int tile, bool live = true) {
    constexpr bool ctx = decltype(phase)::ctx;
    const int tile_base = tile * BN;
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) {
      const int ci = wave * C::CPW + i;  // wave-uniform
      const bool isv = ci >= C::KCH;
      const int cc = isv ? ci - C::KCH : ci;
      char* dst = stage + (isv ? BN * C::RB : 0) + cc * 1024;
      if constexpr (ctx) {
        // keys past nctx are clamped to the last valid key (finite, masked)
        const int key = min(tile_base + lrow[i], nctx - 1);
        if constexpr (uniform_blocks) {
          // The RPC rows of the chunk lie in one block (block_size is a
          // multiple of RPC). Buffer loads into LDS count in vmcnt only,
          // whereas global_load_lds would also hold lgkmcnt and serialise
          // every LDS operand wait behind the tile loads in flight.
          const int slot = key - (int)(lb_next[i] * (uint32_t)a.block_size);
          const uint32_t boff = (uint32_t)(EB * slot * (int)key_stride + 16 * lslot[i]);
          const uint32_t soff = (uint32_t)min(max(bt_next[i], 0), a.num_blocks - 1) * block_bytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(pick_rsrc(live, isv, vpool, kpool, no_rsrc),
                                                   (lds_void_t*)(dst), 16, boff, soff, 0, 0);
        } else {
          const int lb = (int)div_block((uint32_t)key, a);
          const int slot = key - lb * a.block_size;
          int pb = btab[lb];
          pb = min(max(pb, 0), a.num_blocks - 1);
          const size_t off = ((size_t)pb * a.block_size + slot) * key_stride + (size_t)kvh * D;
          const char* src = (const char*)(isv ? a.vc : a.kc) + off * EB + lslot[i] * 16;
          __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst), 16, 0, 0);
        }
      } else {
        const uint32_t voff = (uint32_t)tile_base * (uint32_t)(key_stride * EB) + lane_off[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pick_rsrc(live, isv, vrsrc, krsrc, no_rsrc),
                                                 (lds_void_t*)(dst), 16, voff, 0, 0, 0);
      }
    }
  };
  // Block ids of context tile t for the paged loads (uniform blocks). They are
  // fetched after a tile's LDS reads have drained and before the barrier that
  // precedes their use: a scalar load in flight during the MFMA/LDS work would
  // make every LDS wait a full lgkmcnt(0) (scalar loads return out of order).
  auto prefetch_ids = [&](auto phase, int t, int tend) {
    if constexpr (decltype(phase)::ctx && uniform_blocks) {
      if (t < tend) fetch_blocks(t);
    }
  };

  f32x16_t o[C::NDB];
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) o[b] = f32x16_t{};
  float m_run = kNegInf;  // reference max, log2 units (scaled)
  float l_lane = 0.f;     // this lane's share of the softmax denominator

  // Per-lane LDS byte offsets of the two operand reads. The slot XOR of a
  // key row depends only on the lane here, so an offset is a lane base plus
  // (compile-time step offset XOR a lane constant) plus an immediate.
  //   K: row 32j + l32, slot 2c + hh              -> byte 16 * ((2c + hh) ^ swz_k)
  //   V (transposed read): row 16kc + 8q + 4hh + (i16 >> 2),
  //      slot 4b + 2dh + ((i16 & 3) >> 1), +8 bytes when i16 is odd
  // E4M3:
  //   K: row 32j + l32, slots 4c + 2hh + u (u = 0, 1), two ds_read_b128 per
  //      MFMA; the XOR splits into its bits 0..1 (in the two lane bases) and
  //      the bits above (XORed onto the step offset 64c).
  //   V (ds_read_b64_tr_b8: in each 16-lane group, result lane i's byte e
  //      comes from source lane 2e + (i >> 3), byte i & 7): source lane s
  //      of group (hh, dh) points at key 8(e >> 2) + 4hh + (e & 3), e = s >> 1,
  //      of the 16-key step, d 32b + 16dh + 8(s & 1). Result lane (hh, l32)
  //      then holds keys 8(e >> 2) + 4hh + (e & 3), e = 0..7, of d column
  //      32b + l32: the keys P^T's operand holds in the same positions.
  const uint32_t krow = (uint32_t)(l32 * C::RB);
  const uint32_t kx = (uint32_t)(16 * (hh ^ C::swz_k(l32)));
  const int gk = C::swz_k(l32);
  const uint32_t kb0 = krow + (uint32_t)(16 * ((2 * hh) ^ (gk & 3)));
  const uint32_t kb1 = krow + (uint32_t)(16 * ((2 * hh + 1) ^ (gk & 3)));
  const uint32_t kxh = (uint32_t)(16 * (gk & ~3));
  uint32_t vrow_off, vx;
  {
    const int i16 = lane & 15;
    const int dh = (lane >> 4) & 1;
    if constexpr (FP8) {
      const int e = i16 >> 1;
      const int key = 8 * (e >> 2) + 4 * hh + (e & 3);
      vrow_off = (uint32_t)(key * C::RB + 16 * dh + 8 * (i16 & 1));
      vx = (uint32_t)(16 * C::swz_v(key));  // even slot XOR: a multiple of 32 bytes
    } else {
      const int vrow = 4 * hh + (i16 >> 2);
      const int vlo = 2 * dh + ((i16 & 3) >> 1);
      vrow_off = (uint32_t)(vrow * C::RB + 16 * vlo + (i16 & 1) * 8);
      vx = (uint32_t)(16 * C::swz_v(vrow));  // slot XOR, only bits 2..3 of the slot
    }
  }

  // Phase 1, E4M3: S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (both operands
  // E4M3, no block scales), 64 d per MFMA.
  auto qk8 = [&](const char* stage, f32x16_t (&s)[C::NJ]) {
    if constexpr (FP8) {
      uint32_t kxh_t = kxh;
      if constexpr (D >= PCP_LAUNDER_MIN_D) asm volatile("" : "+v"(kxh_t));
      const lds_char_t* sK = (const lds_char_t*)(stage);
      constexpr int NK = C::NQC * C::NJ;
      constexpr int KP = PCP_KPREF < NK ? PCP_KPREF : NK;
      auto kload = [&](int idx) -> i32x8_t {
        const int c = idx / C::NJ, j = idx % C::NJ;
        const uint32_t step = ((uint32_t)(64 * c) ^ kxh_t) + (uint32_t)(j * 32 * C::RB);
        const i32x4_t lo = *(const lds_i32x4_t*)(sK + kb0 + step);
        const i32x4_t hi = *(const lds_i32x4_t*)(sK + kb1 + step);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) s[j] = f32x16_t{};
      i32x8_t kbuf[KP + 1];
#pragma unroll
      for (int i = 0; i < KP; ++i) kbuf[i] = kload(i);
#pragma unroll
      for (int idx = 0; idx < NK; ++idx) {
        if (idx + KP < NK) kbuf[(idx + KP) % (KP + 1)] = kload(idx + KP);
        const int c = idx / C::NJ, j = idx % C::NJ;
        s[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kbuf[idx % (KP + 1)], qf[c], s[j], 0,
                                                               0, 0, 0, 0, 0);
      }
      if constexpr (PCP_SCHED_QK != 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KP, 0);
#pragma unroll
        for (int i = 0; i < NK - KP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KP, 0);
      }
    }
  };

  // Phase 1: S^T = K Q^T, K fragments read PCP_KPREF steps ahead of their MFMA.
  auto qk = [&](const char* stage, f32x16_t (&s)[C::NJ]) {
    if constexpr (FP8) {
      qk8(stage, s);
    } else {
      // At d = 256 the per-step XOR offsets are recomputed each tile (one
      // v_xor + add per read) instead of held in registers across the loop;
      // smaller head dims have the registers and keep them (~1% faster).
      uint32_t kx_t = kx;
      if constexpr (D >= PCP_LAUNDER_MIN_D) asm volatile("" : "+v"(kx_t));
      const lds_char_t* sK = (const lds_char_t*)(stage);
      constexpr int NK = C::NQC * C::NJ;
      constexpr int KP = PCP_KPREF < NK ? PCP_KPREF : NK;
      auto kload = [&](int idx) -> bf16x8_t {
        const int c = idx / C::NJ, j = idx % C::NJ;
        // (2c + hh) ^ x over the low 4 slot bits: 32 * (c & 7) ^ (16 * (hh ^ x))
        const uint32_t off = krow + ((uint32_t)(32 * (c & 7)) ^ kx_t) +
                             (uint32_t)(256 * (c >> 3) + j * 32 * C::RB);
        return *(const __attribute__((address_space(3))) bf16x8_t*)(sK + off);
      };
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) s[j] = f32x16_t{};
      bf16x8_t kbuf[KP + 1];
#pragma unroll
      for (int i = 0; i < KP; ++i) kbuf[i] = kload(i);
#pragma unroll
      for (int idx = 0; idx < NK; ++idx) {
        if (idx + KP < NK) kbuf[(idx + KP) % (KP + 1)] = kload(idx + KP);
        const int c = idx / C::NJ, j = idx % C::NJ;
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kbuf[idx % (KP + 1)], qf[c], s[j], 0, 0, 0);
      }
      if constexpr (PCP_SCHED_QK != 0) {
        // KP reads first, then (MFMA, read) pairs, then the last KP MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, KP, 0);
#pragma unroll
        for (int i = 0; i < NK - KP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KP, 0);
      }
    }
  };

  // Phase 2: mask, online softmax with stale-max rescaling, P^T as bf16.
  auto softmax = [&](auto phase, f32x16_t (&s)[C::NJ], int tile, bf16x8_t (&pf)[C::NKC]) {
    // Mask: context tiles end at nctx; new-token tiles at the causal bound
    // of this lane's query (and nnew).
    constexpr bool ctx = decltype(phase)::ctx;
    const int tile_base = tile * BN;
    int full_end;  // keys below this are visible to every query of the wave
    if constexpr (ctx) {
      full_end = nctx;
    } else {
      full_end = min(nnew, row.k_len - row.q_len + t0 + 1);
    }
    if (tile_base + BN > full_end) {
      int kb;
      if constexpr (ctx) {
        kb = nctx - 1;
      } else {
        kb = min(nnew - 1, row.k_len - row.q_len + t);
      }
      kb -= tile_base + 4 * hh;
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * j + 8 * (i >> 2) + (i & 3);
          if (key > kb) s[j][i] = kNegInf;
        }
      }
    }

    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[j][i]);
    }
    mx = halves_max(mx);
    const float mnew = mx * scale_log2;
    const bool need = mnew > m_run + kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
      m_run = need ? mnew : m_run;
      l_lane *= alpha;
#pragma unroll
      for (int b = 0; b < C::NDB; ++b) o[b] *= alpha;
    }
    const float negm = (m_run == kNegInf) ? 0.f : -m_run;
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j][i], scale_log2, negm));
        lsum += p;
        pf[2 * j + (i >> 3)][i & 7] = (__bf16)p;
      }
    }
    l_lane += lsum;
  };

  // Phase 3, E4M3: V^T read with ds_read_b64_tr_b8 (8 keys of one d column
  // per lane) and widened to bf16 (exact: every E4M3 value is a bf16 value),
  // so O^T += V^T P^T stays a bf16 MFMA with P kept in bf16.
  auto pv8 = [&](const char* stage, const bf16x8_t (&pf)[C::NKC]) {
    if constexpr (FP8) {
      uint32_t vx_t = vx;
      if constexpr (D >= PCP_LAUNDER_MIN_D) asm volatile("" : "+v"(vx_t));
      const lds_char_t* sV = (const lds_char_t*)(stage + BN * C::RB);
      constexpr int NV = C::NKC * C::NDB;
      constexpr int VP = PCP_VPREF < NV ? PCP_VPREF : NV;
      auto vload = [&](int idx) -> i32x2_t {
        const int kc = idx / C::NDB, b = idx % C::NDB;
        const uint32_t off = vrow_off + ((uint32_t)(32 * b) ^ vx_t) + (uint32_t)(16 * kc * C::RB);
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(sV + off));
      };
      auto widen = [](i32x2_t r) -> bf16x8_t {
        const bf16x2_t e01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[0], 1.0f, false);
        const bf16x2_t e23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[0], 1.0f, true);
        const bf16x2_t e45 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[1], 1.0f, false);
        const bf16x2_t e67 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[1], 1.0f, true);
        const bf16x4_t lo = __builtin_shufflevector(e01, e23, 0, 1, 2, 3);
        const bf16x4_t hi = __builtin_shufflevector(e45, e67, 0, 1, 2, 3);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      i32x2_t vbuf[VP + 1];
#pragma unroll
      for (int i = 0; i < VP; ++i) vbuf[i] = vload(i);
#pragma unroll
      for (int idx = 0; idx < NV; ++idx) {
        if (idx + VP < NV) vbuf[(idx + VP) % (VP + 1)] = vload(idx + VP);
        const int kc = idx / C::NDB, b = idx % C::NDB;
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen(vbuf[idx % (VP + 1)]), pf[kc], o[b], 0,
                                                       0, 0);
      }
      if constexpr (PCP_SCHED_PV != 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, VP, 0);
#pragma unroll
        for (int i = 0; i < NV - VP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, VP, 0);
      }
    }
  };

  // Phase 3: O^T += V^T P^T, V fragments read PCP_VPREF steps ahead of their MFMA.
  auto pv = [&](const char* stage, const bf16x8_t (&pf)[C::NKC]) {
    if constexpr (FP8) {
      pv8(stage, pf);
    } else {
      uint32_t vx_t = vx;
      if constexpr (D >= PCP_LAUNDER_MIN_D) asm volatile("" : "+v"(vx_t));
      const lds_char_t* sV = (const lds_char_t*)(stage + BN * C::RB);
      constexpr int NV = C::NKC * C::NDB;
      constexpr int VP = PCP_VPREF < NV ? PCP_VPREF : NV;
      auto vload = [&](int idx) -> bf16x8_t {
        const int kc = idx / C::NDB, b = idx % C::NDB;
        // slot (4b + vlo) ^ swz_v: the XOR only touches bits 2..3, i.e. b & 3
        const uint32_t off = vrow_off + ((uint32_t)(64 * (b & 3)) ^ vx_t) +
                             (uint32_t)(256 * (b >> 2) + 16 * kc * C::RB);
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(sV + off));
        const bf16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(sV + off + 8 * C::RB));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t vbuf[VP + 1];
#pragma unroll
      for (int i = 0; i < VP; ++i) vbuf[i] = vload(i);
#pragma unroll
      for (int idx = 0; idx < NV; ++idx) {
        if (idx + VP < NV) vbuf[(idx + VP) % (VP + 1)] = vload(idx + VP);
        const int kc = idx / C::NDB, b = idx % C::NDB;
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vbuf[idx % (VP + 1)], pf[kc], o[b], 0, 0, 0);
      }
      if constexpr (PCP_SCHED_PV != 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VP, 0);
#pragma unroll
        for (int i = 0; i < NV - VP; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, VP, 0);
      }
    }
  };

  // New-token tiles past the causal bound of the wave's last query are fully
  // masked for it (a unit of several query blocks, HG < kWaves, runs up to the
  // bound of its last query): the wave skips them and only takes part in the
  // loads and barriers. Context tiles are visible to every query. Not at
  // d = 256, where the extra state tips the loop into spilling a load offset.
  constexpr bool kSkipMasked = PCP_SKIP_MASKED != 0 && HG < kWaves && D <= 128;
  const int wave_new_end =
      kSkipMasked ? min(nnew, row.k_len - row.q_len + min(t0 + 32, row.q_len)) : 0;
  auto visible = [&](auto phase, int tile) -> bool {
    if constexpr (decltype(phase)::ctx || !kSkipMasked) {
      return true;
    } else {
      return tile * BN < wave_new_end;
    }
  };

  auto compute = [&](auto phase, const char* stage, int tile) {
    f32x16_t s[C::NJ];
    bf16x8_t pf[C::NKC];
    qk(stage, s);
    softmax(phase, s, tile, pf);
    pv(stage, pf);
  };

  // Stream tiles [tfirst, tend) of one phase through the LDS ring; comp
  // consumes a tile.
  auto run = [&](auto phase, int tfirst, int tend, auto&& comp) {
    prefetch_ids(phase, tfirst, tend);
    if constexpr (kStages >= 3) {
      // Ring of kStages stages, one barrier per tile: when every wave has
      // passed the barrier of tile j, all reads of tile j-1 are done, so its
      // stage is refilled with tile j + kStages - 1 (kStages - 1 tiles of
      // loads in flight).
      constexpr int AHEAD = kStages - 1;
      if constexpr (kStages == 3 && (!decltype(phase)::ctx || uniform_blocks)) {
        // Buffer-load tiles: every step issues one tile, a tile past tend
        // with a descriptor of no records (it reads nothing), and the loop
        // runs whole rounds of the three stages (one or two steps past the
        // last tile). Each step then waits alike for its own tile, and every
        // path through the loop issues the same loads into the same stages,
        // which keeps the compiler's own wait before a stage's first read
        // from covering the loads still in flight (with a refill issued on
        // some paths only, or the loop left between stages, it waited for
        // all of them in one of the three steps).
        if (tfirst >= tend) return;
        auto ustep = [&](const char* cur, char* refill, int tile) {
          wait_vmcnt<C::CPW>();  // this tile landed; the next one may be in flight
          block_barrier();
          if constexpr (decltype(phase)::ctx) wait_lgkm0();  // block ids of the refill
          issue(phase, refill, tile + AHEAD, tile + AHEAD < tend);
          if (tile < tend && wave_active && visible(phase, tile)) comp(phase, cur, tile);
          wait_lgkm0();
          prefetch_ids(phase, tile + AHEAD + 1, tend);
        };
        issue(phase, smem0, tfirst, true);
        prefetch_ids(phase, tfirst + 1, tend);
        issue(phase, smem1, tfirst + 1, tfirst + 1 < tend);
        prefetch_ids(phase, tfirst + 2, tend);
        int tile = tfirst;
        do {
          ustep(smem0, smem2, tile);
          ustep(smem1, smem0, tile + 1);
          ustep(smem2, smem1, tile + 2);
          tile += 3;
        } while (tile < tend);
        return;
      }
      auto step = [&](const char* cur, char* refill, int tile) {
        // wait for tile `tile`; the tiles issued after it may stay in flight
        const int later = min(AHEAD - 1, tend - 1 - tile);
        if (later >= 2) {
          wait_vmcnt<2 * C::CPW>();
        } else if (later == 1) {
          wait_vmcnt<C::CPW>();
        } else {
          wait_vmcnt<0>();
        }
        block_barrier();
        // the block ids fetched during the last tile are due now (both
        // branches below then start with no scalar load pending)
        if constexpr (decltype(phase)::ctx && uniform_blocks) wait_lgkm0();
        if (tile + AHEAD < tend) issue(phase, refill, tile + AHEAD);
        if (wave_active && visible(phase, tile)) comp(phase, cur, tile);
        wait_lgkm0();
        prefetch_ids(phase, tile + AHEAD + 1, tend);
      };
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) {
        char* st = i == 0 ? smem0 : (i == 1 ? smem1 : smem2);
        if (tfirst + i < tend) issue(phase, st, tfirst + i);
        prefetch_ids(phase, tfirst + i + 1, tend);
      }
      if constexpr (kStages == 3) {
        for (int tile = tfirst; tile < tend; tile += 3) {
          step(smem0, smem2, tile);
          if (tile + 1 >= tend) break;
          step(smem1, smem0, tile + 1);
          if (tile + 2 >= tend) break;
          step(smem2, smem1, tile + 2);
        }
      } else {
        for (int tile = tfirst; tile < tend; tile += 4) {
          step(smem0, smem3, tile);
          if (tile + 1 >= tend) break;
          step(smem1, smem0, tile + 1);
          if (tile + 2 >= tend) break;
          step(smem2, smem1, tile + 2);
          if (tile + 3 >= tend) break;
          step(smem3, smem2, tile + 3);
        }
      }
    } else {
      // Two stages: load tile j+1 while tile j is consumed; a second barrier
      // frees the stage before it is refilled.
      auto step = [&](const char* cur, char* next, int tile) {
        if (tile + 1 < tend) {
          issue(phase, next, tile + 1);
          wait_vmcnt<C::CPW>();
        } else {
          wait_vmcnt<0>();
        }
        block_barrier();
        if (wave_active && visible(phase, tile)) comp(phase, cur, tile);
        wait_lgkm0();
        prefetch_ids(phase, tile + 2, tend);
        block_barrier();
      };
      if (tfirst < tend) issue(phase, smem0, tfirst);
      prefetch_ids(phase, tfirst + 1, tend);
      for (int tile = tfirst; tile < tend; tile += 2) {
        step(smem0, smem1, tile);
        if (tile + 1 >= tend) break;
        step(smem1, smem0, tile + 1);
      }
    }
  };

  // Context tiles first (a split decode row takes its range of them), then
  // the new-token tiles; one online softmax runs through both.
  const int new_tiles = (nnew + BN - 1) / BN;
  if constexpr (HAS_CTX) {
    int cfirst = 0, cend = ctx_tiles;
    if (split) {
      const int per = (ctx_tiles + a.dec_splits - 1) / a.dec_splits;
      cfirst = min(split_id * per, ctx_tiles);
      cend = min(ctx_tiles, cfirst + per);
    }
    if constexpr (kDec16) {
      if (dec16) {
        // Decode unit, 16x16 layout: lane (n, g), n = lane % 16, g = lane / 16.
        //   S^T = K Q^T: A = K row 16jb + n of the tile, B = Q^T of head column
        //     n, both with d 32c + 8g + [0, 8) of step c (E4M3: 128c + 32g +
        //     [0, 32)); the accumulator of block jb then holds keys 16jb + 4g + e
        //     (e < 4) of column n.
        //   O^T += V^T P^T in 32-key steps ks (16x16x32 bf16): element i of
        //     P^T's lane (n, g) is key 32ks + 16(i >> 2) + 4g + (i & 3) (the
        //     accumulators of blocks 2ks and 2ks + 1 as they stand); V^T's lane
        //     (m, g) takes the same keys of d column 16b + m from transposed
        //     reads (E4M3: one read of all 8 keys, widened to bf16).
        const int g = lane >> 4;
        typedef typename Frag<FP8>::type qd_t;
        qd_t qd[C::NC16];
        if (q_valid && nkeys > 0) {
          if constexpr (FP8) {
            const uint8_t* qp =
                (const uint8_t*)a.q + ((size_t)row.q_start * a.hq + head) * D + 32 * g;
#pragma unroll
            for (int c = 0; c < C::NC16; ++c) {
              const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(qp + 128 * c);
              const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(qp + 128 * c + 16);
              qd[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          } else {
            const u16* qp = (const u16*)a.q + ((size_t)row.q_start * a.hq + head) * D + 8 * g;
#pragma unroll
            for (int c = 0; c < C::NC16; ++c)
              qd[c] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * c);
          }
        } else {
#pragma unroll
          for (int c = 0; c < C::NC16; ++c) qd[c] = qd_t{};
        }
        f32x4_t od[C::NDB16];
#pragma unroll
        for (int b = 0; b < C::NDB16; ++b) od[b] = f32x4_t{};
        // K: row n of a 16-key block. bf16: slot (4c + g) ^ swz_k(n) = lane base
        // + (64c XOR the slot XOR's bits 2..3). E4M3: slots (8c + 2g + u) ^
        // swz_k(n), u = 0, 1 = lane base u + (128c XOR the XOR's bit 3).
        const int sk = C::swz_k(lane & 15);
        const uint32_t krow_d = (uint32_t)((lane & 15) * C::RB);
        const uint32_t kd_base = krow_d + (uint32_t)(FP8 ? 16 * ((2 * g) ^ (sk & 7))
                                                        : 16 * (g ^ (sk & 3)));
        const uint32_t kd_base1 = krow_d + (uint32_t)(16 * ((2 * g + 1) ^ (sk & 7)));
        const uint32_t kdx = (uint32_t)(FP8 ? 16 * (sk & ~7) : 16 * (sk & ~3));
        // V, bf16 (ds_read_b64_tr_b16): source lane s = lane % 16 of group g
        // points at key 4g + (s >> 2), d 16b + 4(s & 3) (slot 2b + ((s & 3) >>
        // 1), 8 bytes further when s is odd); result lane m then holds the 4
        // keys of d column 16b + m. The even slot XOR only touches bits 1..3 of
        // 2b. E4M3 (ds_read_b64_tr_b8: result lane i's byte e comes from source
        // lane 2e + (i >> 3), byte i & 7): source lane s points at key
        // 16(e >> 2) + 4g + (e & 3), e = s >> 1, d 16b + 8(s & 1), i.e. slot b
        // XOR swz_vd, 8 bytes further when s is odd.
        const int s16 = lane & 15;
        int vkey;
        uint32_t vd_base;
        if constexpr (FP8) {
          const int e = s16 >> 1;
          vkey = 16 * (e >> 2) + 4 * g + (e & 3);
          vd_base = (uint32_t)(vkey * C::RB + 8 * (s16 & 1));
        } else {
          vkey = 4 * g + (s16 >> 2);
          vd_base = (uint32_t)(vkey * C::RB + 16 * ((s16 & 3) >> 1) + 8 * (s16 & 1));
        }
        const uint32_t vdx = (uint32_t)(16 * C::swz_vd(vkey));

        auto qk_dec = [&](const char* stage, f32x4_t (&sc)[C::NB16]) {
          const lds_char_t* sK = (const lds_char_t*)(stage);
          constexpr int NK = C::NC16 * C::NB16;
          constexpr int KP = PCP_KPREF < NK ? PCP_KPREF : NK;
          auto kload = [&](int idx) -> qd_t {
            const int c = idx / C::NB16, jb = idx % C::NB16;
            if constexpr (FP8) {
              const uint32_t step = ((uint32_t)(128 * c) ^ kdx) + (uint32_t)(16 * jb * C::RB);
              const i32x4_t lo = *(const lds_i32x4_t*)(sK + kd_base + step);
              const i32x4_t hi = *(const lds_i32x4_t*)(sK + kd_base1 + step);
              return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
              const uint32_t off =
                  kd_base + ((uint32_t)(64 * c) ^ kdx) + (uint32_t)(16 * jb * C::RB);
              return *(const __attribute__((address_space(3))) bf16x8_t*)(sK + off);
            }
          };
#pragma unroll
          for (int jb = 0; jb < C::NB16; ++jb) sc[jb] = f32x4_t{};
          qd_t kbuf[KP + 1];
#pragma unroll
          for (int i = 0; i < KP; ++i) kbuf[i] = kload(i);
#pragma unroll
          for (int idx = 0; idx < NK; ++idx) {
            if (idx + KP < NK) kbuf[(idx + KP) % (KP + 1)] = kload(idx + KP);
            const int c = idx / C::NB16, jb = idx % C::NB16;
            if constexpr (FP8) {
              sc[jb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  kbuf[idx % (KP + 1)], qd[c], sc[jb], 0, 0, 0, 0, 0, 0);
            } else {
              sc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbuf[idx % (KP + 1)], qd[c], sc[jb],
                                                               0, 0, 0);
            }
          }
        };
        auto softmax_dec = [&](f32x4_t (&sc)[C::NB16], int tile, bf16x8_t (&pf)[C::NKS16]) {
          const int tile_base = tile * BN;
          if (tile_base + BN > nctx) {
            const int kb = nctx - 1 - tile_base - 4 * g;
#pragma unroll
            for (int jb = 0; jb < C::NB16; ++jb) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (16 * jb + e > kb) sc[jb][e] = kNegInf;
            }
          }
          float mx = kNegInf;
#pragma unroll
          for (int jb = 0; jb < C::NB16; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[jb][e]);
          }
          mx = quad_max(mx);
          const float mnew = mx * scale_log2;
          const bool need = mnew > m_run + kRescaleTau;
          if (__builtin_amdgcn_ballot_w64(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
            m_run = need ? mnew : m_run;
            l_lane *= alpha;
#pragma unroll
            for (int b = 0; b < C::NDB16; ++b) od[b] *= alpha;
          }
          const float negm = (m_run == kNegInf) ? 0.f : -m_run;
          float lsum = 0.f;
#pragma unroll
          for (int jb = 0; jb < C::NB16; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sc[jb][e], scale_log2, negm));
              lsum += p;
              pf[jb >> 1][4 * (jb & 1) + e] = (__bf16)p;
            }
          }
          l_lane += lsum;
        };
        auto pv_dec = [&](const char* stage, const bf16x8_t (&pf)[C::NKS16]) {
          const lds_char_t* sV = (const lds_char_t*)(stage + BN * C::RB);
          constexpr int NV = C::NKS16 * C::NDB16;
          constexpr int VP = PCP_VPREF < NV ? PCP_VPREF : NV;
          auto vload = [&](int idx) -> bf16x8_t {
            const int ks = idx / C::NDB16, b = idx % C::NDB16;
            if constexpr (FP8) {
              const uint32_t off = vd_base + ((uint32_t)(16 * b) ^ vdx) + (uint32_t)(32 * ks * C::RB);
              const i32x2_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(sV + off));
              const bf16x2_t e01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[0], 1.0f, false);
              const bf16x2_t e23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[0], 1.0f, true);
              const bf16x2_t e45 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[1], 1.0f, false);
              const bf16x2_t e67 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)r[1], 1.0f, true);
              const bf16x4_t lo = __builtin_shufflevector(e01, e23, 0, 1, 2, 3);
              const bf16x4_t hi = __builtin_shufflevector(e45, e67, 0, 1, 2, 3);
              return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
              const uint32_t off = vd_base + ((uint32_t)(32 * (b & 7)) ^ vdx) +
                                   (uint32_t)(256 * (b >> 3) + 32 * ks * C::RB);
              const bf16x4_t lo =
                  __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(sV + off));
              const bf16x4_t hi =
                  __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(sV + off + 16 * C::RB));
              return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          };
          bf16x8_t vbuf[VP + 1];
#pragma unroll
          for (int i = 0; i < VP; ++i) vbuf[i] = vload(i);
#pragma unroll
          for (int idx = 0; idx < NV; ++idx) {
            if (idx + VP < NV) vbuf[(idx + VP) % (VP + 1)] = vload(idx + VP);
            const int ks = idx / C::NDB16, b = idx % C::NDB16;
            od[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vbuf[idx % (VP + 1)], pf[ks], od[b], 0, 0,
                                                            0);
          }
        };
        auto compute_dec = [&](auto, const char* stage, int tile) {
          f32x4_t sc[C::NB16];
          bf16x8_t pf[C::NKS16];
          qk_dec(stage, sc);
          softmax_dec(sc, tile, pf);
          pv_dec(stage, pf);
        };
        run(DecPhase{}, cfirst, cend, compute_dec);

        if (!wave_active) return;
        const float l_tot = quad_sum(l_lane);
        if (!q_valid) return;
        const bool has = l_tot > 0.f;
        const float inv = has ? out_scale / l_tot : 0.f;
        const float lse_v = has ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
        if (split) {
          const size_t part = ((size_t)row_id * a.hq + head) * a.dec_splits + split_id;
          float* wp = a.ws + part * D + 4 * g;
#pragma unroll
          for (int b = 0; b < C::NDB16; ++b) *reinterpret_cast<f32x4_t*>(wp + 16 * b) = od[b] * inv;
          if (g == 0) a.ws[(size_t)a.num_rows * a.hq * a.dec_splits * D + part] = lse_v;
          return;
        }
        u16* op = a.out + ((size_t)row.q_start * a.hq + head) * D + 4 * g;
#pragma unroll
        for (int b = 0; b < C::NDB16; ++b) {
          bf16x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(od[b][e] * inv);
          *reinterpret_cast<bf16x4_t*>(op + 16 * b) = w;
        }
        if (g == 0) a.lse[(size_t)head * a.total_q + row.q_start] = lse_v;
        return;
      }
    }
    run(CtxPhase{}, cfirst, cend, compute);
    // every wave is done with the ring before the new-token tiles refill it
    if (HAS_NEW && cfirst < cend && new_tiles > 0) block_barrier();
    wait_lgkm0();  // no scalar load left pending into the new-token tiles
  }
  if constexpr (HAS_NEW) run(NewPhase{}, 0, new_tiles, compute);

  // d <= 128: the output tile leaves through LDS (below), in the stages of
  // the ring, once every wave's loads into them have landed and every wave
  // is done reading them.
  constexpr bool kStageOut = D <= 128;
  if constexpr (kStageOut) {
    wait_vmcnt<0>();
    block_barrier();
  }
  if (!wave_active) return;
  const float l_tot = halves_sum(l_lane);
  if (!kStageOut && !q_valid) return;
  const bool has = l_tot > 0.f;
  const float inv = has ? out_scale / l_tot : 0.f;
  const float lse_v = has ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
  if (split) {  // partial of one key range: fp32 out and lse to the workspace
    if (!q_valid) return;
    const size_t part = ((size_t)row_id * a.hq + head) * a.dec_splits + split_id;
    float* wp = a.ws + part * D + 4 * hh;
#pragma unroll
    for (int b = 0; b < C::NDB; ++b) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[b][4 * g4 + e] * inv;
        *reinterpret_cast<f32x4_t*>(wp + 32 * b + 8 * g4) = w;
      }
    }
    if (hh == 0) a.ws[(size_t)a.num_rows * a.hq * a.dec_splits * D + part] = lse_v;
    return;
  }
  if constexpr (kStageOut) {
    // Lane (l32, hh) holds, of its slot's output row, d = 32b + 8g4 + 4hh +
    // [0, 4). Written as rows of D bf16 into this wave's part of the stages
    // (16-byte slots XORed with the row), then read back 16 bytes per lane,
    // D / 8 lanes to a row, each row goes out in one contiguous store
    // instead of 8-byte pieces of 64 rows per instruction. A slot is a
    // query (a packed decode row: a head).
    constexpr int SL = D / 8;        // 16-byte slots per row
    constexpr int RPI = 64 / SL;     // rows per read instruction
    char* region = (wave < 4 ? smem0 : smem1) + (wave & 3) * (32 * D * 2);
    static_assert(4 * 32 * D * 2 <= C::STAGE, "four waves' output tiles fit one stage");
#pragma unroll
    for (int b = 0; b < C::NDB; ++b) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][4 * g4 + e] * inv);
        const int slot = (4 * b + g4) ^ (l32 & (SL - 1));
        *(lds_bf16x4_t*)(region + l32 * (2 * D) + 16 * slot + 8 * hh) = w;
      }
    }
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int r = k * RPI + lane / SL;
      const int sl = lane % SL;
      const i32x4_t v = *(const lds_i32x4_t*)(region + r * (2 * D) + 16 * (sl ^ (r & (SL - 1))));
      const bool valid = pack ? r < HG : t0 + r < row.q_len;
      const size_t orow = pack ? (size_t)row.q_start * a.hq + head0 + r
                               : (size_t)(row.q_start + t0 + r) * a.hq + head;
      if (valid) *reinterpret_cast<i32x4_t*>(a.out + orow * D + 8 * sl) = v;
    }
    if (hh == 0 && q_valid) a.lse[(size_t)head * a.total_q + row.q_start + t] = lse_v;
    return;
  }
  u16* op = a.out + ((size_t)(row.q_start + t) * a.hq + head) * D + 4 * hh;
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][4 * g4 + e] * inv);
      *reinterpret_cast<bf16x4_t*>(op + 32 * b + 8 * g4) = w;
    }
  }
  if (hh == 0) a.lse[(size_t)head * a.total_q + row.q_start + t] = lse_v;
}

// Merge the key-range partials of every split one-query row of a context
// pass: one wave per (row, head), the same LSE combine as lse_merge.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const AttnArgs a) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= a.num_rows * a.hq) return;
  const int row_id = pair / a.hq;
  const int head = pair - row_id * a.hq;
  const pcp_row_t row = a.rows[row_id];
  // only split rows, and not the ones the attention kernel skipped
  if (row.q_len != 1 || row.k_len > 0 || row.q_start < 0 || row.q_start >= a.total_q) return;
  if (row.req < 0 || row.req >= a.num_reqs || row.ctx_len_local < 0 ||
      (int64_t)row.ctx_len_local > (int64_t)a.max_blocks * a.block_size)
    return;
  if (a.has_new && (row.k_start < 0 || row.k_len < 0 || row.k_start > a.total_k - row.k_len))
    return;
  const size_t part0 = ((size_t)row_id * a.hq + head) * a.dec_splits;
  const float* wp = a.ws + part0 * D;
  const float* wl = a.ws + (size_t)a.num_rows * a.hq * a.dec_splits * D + part0;
  const int S = a.dec_splits;
  // Each lane holds PER consecutive d values. The splits are taken U at a
  // time, and every load of a group (the LSEs, which every lane reads, and
  // the partial outputs, all written by the attention kernel, empty ranges
  // as (0, -inf)) is issued before any is used, so a group costs one memory
  // round trip. A running max carries over from group to group; with S <= U
  // it is the max of all the LSEs and the sums are those of a plain
  // max-then-sum pass.
  constexpr int PER = D / 64;
  constexpr int U = 16;
  typedef float fper_t __attribute__((ext_vector_type(PER)));
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  float mx = kNegInf;
  for (int s0 = 0; s0 < S; s0 += U) {
    float lw[U];
    fper_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      lw[u] = s < S ? wl[s] : kNegInf;
      x[u] = s < S ? *reinterpret_cast<const fper_t*>(wp + (size_t)s * D + PER * lane) : fper_t{};
    }
    float gm = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) gm = fmaxf(gm, lw[u]);
    const float mnew = fmaxf(mx, gm);
    if (mnew == kNegInf) continue;  // every range so far empty
    if (mnew != mx) {               // rescale what the earlier groups summed
      const float r = __builtin_amdgcn_exp2f((mx - mnew) * kLog2e);
      wsum *= r;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] *= r;
      mx = mnew;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = __builtin_amdgcn_exp2f((lw[u] - mx) * kLog2e);
      wsum += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, x[u][e], acc[e]);
    }
  }
  const float inv = mx != kNegInf ? 1.0f / wsum : 0.f;
  u16* op = a.out + ((size_t)row.q_start * a.hq + head) * D + PER * lane;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const __bf16 y = (__bf16)(acc[e] * inv);
    op[e] = __builtin_bit_cast(u16, y);
  }
  if (lane == 0)
    a.lse[(size_t)head * a.total_q + row.q_start] =
        mx != kNegInf ? mx + __builtin_amdgcn_logf(wsum) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------- launchers

using pcp_geom::heads_per_group;
using pcp_geom::supported_dim;

template <int D, int BN, int HG, int MODE, bool FP8>
int launch_attn(AttnArgs args, int max_q_len, int num_ordered, hipStream_t stream) {
  using C = Attn<D, BN, HG, FP8 ? 1 : 2>;
  static_assert(C::BQ == pcp_geom::block_q(HG) && BN == pcp_geom::block_n(D, FP8 ? 1 : 2),
                "geometry");
  args.groups_per_kv = args.group / HG;
  args.has_new = MODE == 0 || MODE >= 3;
  const int64_t qt = pcp_geom::q_tiles(max_q_len, HG, MODE != 0, args.dec_splits);
  const int64_t units = (int64_t)args.num_rows * args.hkv * args.groups_per_kv * qt;
  if (qt > INT32_MAX || units > INT32_MAX) return PCP_EOVERFLOW;
  args.q_tiles = (int)qt;
  args.num_units = (int)units;
  const int grid = args.order != nullptr ? num_ordered : (int)units;
  if (units == 0 || grid == 0) return PCP_OK;
  hipLaunchKernelGGL((attn_fwd_kernel<D, BN, HG, MODE, FP8>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, args);
  if (hipGetLastError() != hipSuccess) return PCP_EHIP;
  if (MODE != 0 && args.dec_splits > 1) {
    const int64_t pairs = (int64_t)args.num_rows * args.hq;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0,
                       stream, args);
    if (hipGetLastError() != hipSuccess) return PCP_EHIP;
  }
  return PCP_OK;
}

template <int D, int MODE, bool FP8>
int dispatch_group(const AttnArgs& args, int max_q_len, int n_ord, hipStream_t stream) {
  constexpr int BN = pcp_geom::block_n(D, FP8 ? 1 : 2);
  switch (heads_per_group(args.group)) {
    case 8:
      if constexpr (kWaves >= 8)
        return launch_attn<D, BN, 8, MODE, FP8>(args, max_q_len, n_ord, stream);
      return PCP_EUNSUPPORTED;
    case 4: return launch_attn<D, BN, 4, MODE, FP8>(args, max_q_len, n_ord, stream);
    case 2: return launch_attn<D, BN, 2, MODE, FP8>(args, max_q_len, n_ord, stream);
    default: return launch_attn<D, BN, 1, MODE, FP8>(args, max_q_len, n_ord, stream);
  }
}

using pcp_check::Pass;
using pcp_check::kNewTokens;
using pcp_check::kContext;
using pcp_check::kFused;

// Round-up multiplier of block_size for div_block (key < 2^31).
inline void set_block_divisor(AttnArgs& a) {
  const uint32_t d = a.block_size > 0 ? (uint32_t)a.block_size : 1u;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  a.bs_shift = l;
  a.bs_magic = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
}

template <int D, bool FP8>
int dispatch_mode(AttnArgs args, Pass pass, int max_q_len, int n_ord, hipStream_t stream) {
  set_block_divisor(args);
  // context tiles: block ids per 1 KB chunk (1024 / row bytes key rows) when
  // block_size allows and 32-bit offsets reach the whole pool
  constexpr int elem = FP8 ? 1 : 2;
  constexpr int rpc = 1024 / (D * elem);
  const uint64_t pool_bytes = (uint64_t)args.num_blocks * args.block_size * args.hkv * D * elem;
  const bool uniform = args.block_size % rpc == 0 && pool_bytes <= 0xFFFFFFFFull;
  switch (pass) {
    case kNewTokens: return dispatch_group<D, 0, FP8>(args, max_q_len, n_ord, stream);
    case kContext:
      return uniform ? dispatch_group<D, 1, FP8>(args, max_q_len, n_ord, stream)
                     : dispatch_group<D, 2, FP8>(args, max_q_len, n_ord, stream);
    default:
      return uniform ? dispatch_group<D, 3, FP8>(args, max_q_len, n_ord, stream)
                     : dispatch_group<D, 4, FP8>(args, max_q_len, n_ord, stream);
  }
}

template <bool FP8>
int dispatch_attn(const AttnArgs& args, Pass pass, int d, int max_q_len, int n_ord,
                  hipStream_t stream) {
  switch (d) {
    case 64: return dispatch_mode<64, FP8>(args, pass, max_q_len, n_ord, stream);
    case 128: return dispatch_mode<128, FP8>(args, pass, max_q_len, n_ord, stream);
    case 256: return dispatch_mode<256, FP8>(args, pass, max_q_len, n_ord, stream);
    default: return PCP_EUNSUPPORTED;
  }
}

}  // namespace

#endif  // PCP_ATTN_FWD_H
