// Work-unit geometry of the attention kernels, shared by the kernel
// launchers and the host-side unit scheduler so that both enumerate the same
// units. Internal to libpcpattn.
#ifndef PCP_GEOMETRY_H
#define PCP_GEOMETRY_H

#include <stdint.h>

// Tuning knobs (the defaults are the measured best on MI355X).
#ifndef PCP_BN_D256
#define PCP_BN_D256 32  // keys per tile at d = 256
#endif
#ifndef PCP_BN_SMALL
#define PCP_BN_SMALL 64  // keys per tile at d = 64 and 128
#endif
#ifndef PCP_BN_D256_FP8
#define PCP_BN_D256_FP8 64  // keys per tile at d = 256, E4M3 K/V (half the bytes per key)
#endif
#ifndef PCP_BN_SMALL_FP8
#define PCP_BN_SMALL_FP8 128  // keys per tile at d = 64 and 128, E4M3 K/V
#endif
#ifndef PCP_XCD_RUN
#define PCP_XCD_RUN 4  // consecutive query tiles of one (row, head group) kept on one XCD
#endif
#ifndef PCP_WAVES
#define PCP_WAVES 8  // waves per workgroup: 8 (two per SIMD) or 4 (one per SIMD, 512 registers)
#endif

namespace pcp_geom {

constexpr int kWaves = PCP_WAVES;
constexpr int kXcds = 8;  // MI355X: workgroups are dealt to 8 XCDs round-robin by launch index
constexpr int kXcdRun = PCP_XCD_RUN;

constexpr bool supported_dim(int d) { return d == 64 || d == 128 || d == 256; }

// Keys per tile of bf16 (elem_bytes 2) or E4M3 (1) K/V. Work-unit ids do not
// depend on it, so one unit order serves both element types; the host
// scheduler's cost model counts bf16 tiles.
constexpr int block_n(int d, int elem_bytes = 2) {
  return elem_bytes == 2 ? (d == 256 ? PCP_BN_D256 : PCP_BN_SMALL)
                         : (d == 256 ? PCP_BN_D256_FP8 : PCP_BN_SMALL_FP8);
}

// Query heads sharing one KV head that one workgroup packs (each wave holds
// one head): the largest of 8, 4, 2, 1 dividing the group size.
inline int heads_per_group(int group) {
  for (int hg : {8, 4, 2, 1})
    if (hg <= kWaves && group % hg == 0) return hg;
  return 1;
}

// Queries per workgroup: 32 per wave, HG heads.
constexpr int block_q(int hg) { return 32 * kWaves / hg; }

// Most key ranges a decode row of a context pass is split into.
constexpr int kMaxDecodeSplits = 256;

// Query-tile slots per (row, head group). In the context pass a row with one
// query is split into decode_splits key ranges that use these slots too.
// 64-bit, so that no max_q_len wraps it; callers check the unit count.
inline int64_t q_tiles(int64_t max_q_len, int hg, bool context, int decode_splits) {
  const int64_t bq = block_q(hg);
  int64_t qt = (max_q_len + bq - 1) / bq;
  if (context && decode_splits > qt) qt = decode_splits;
  return qt;
}

}  // namespace pcp_geom

#endif  // PCP_GEOMETRY_H
