// Host side of the C ABI: the launch order of the attention work units.
//
// A work unit of the attention kernels is (row, group of query heads sharing
// one KV head, query tile); its run time is close to proportional to the key
// tiles it streams plus a fixed start-up cost. Units differ a lot in length:
// under the end-aligned causal mask ("Feat/pcp qwen36 hybrid", vllm-plugin-FL
// PR #299, section Changes) a row's last query tile sees k_len keys and its
// first one k_len - q_len + BQ, and mixed batches mix rows of very different
// lengths ("[MRv2][PCP] Carry the row plan in attention metadata; fix mixed
// prefill+decode crash", fork PR #2, section "Two things that fell out of
// (1)"). Launching the units longest first keeps the GPU full until the end
// (longest-processing-time list scheduling).
//
// MI355X deals workgroups to its 8 XCDs round-robin by launch index and each
// XCD has its own L2, so the order is built per XCD:
//   1. units of one (row, head group) are cut into runs of kXcdRun
//      neighbouring query tiles, which read overlapping K/V;
//   2. runs go, longest first, to the XCD with the least work so far;
//   3. each XCD's units are sorted longest first;
//   4. the 8 queues are interleaved (entry 8 i + x is XCD x's i-th unit),
//      shorter queues padded with -1 (a workgroup that exits at once).
// The kernels' built-in order (rows in reverse plan order, query tiles last
// to first, runs of kXcdRun units per XCD) is already close to this for one
// long prompt, where it measures slightly faster. Both orders are therefore
// run through a model of the dispatch (each XCD hands its units in order to
// the first of its CUs to free up) and the built-in one is returned unless
// the longest-first order finishes at least 1% sooner.
//
// Neither keeps the units that read one request's K/V for one KV head
// together. While the launch's K/V fits the 256 MB Infinity Cache that costs
// little; beyond it, those units re-read their keys from HBM on every XCD
// they land on. For such launches, when every (request, KV head) group is
// small next to an XCD's share of the work, whole groups are placed on XCDs
// instead (grouped_order): measured 8% faster for 32 Qwen-shaped 4096-token
// requests and 16% for 64, against 6-12% slower for 8 or 16 requests, whose
// K/V fits the cache.

#include <stdint.h>

#include <algorithm>
#include <functional>
#include <initializer_list>
#include <queue>
#include <vector>

#include "pcp_attn.h"
#include "pcp_geometry.h"

namespace {

constexpr int kUnitStartCost = 2;  // start-up of a unit, in key tiles (Q load, pipeline fill)
constexpr int kCusPerXcd = 32;
constexpr double kMinGain = 0.01;  // prefer the built-in order unless this much faster
constexpr int kPiecesPerXcd = 4;  // K/V groups up to total / (8 * this) are kept whole
constexpr int64_t kMallBytes = 256ll << 20;  // MI355X Infinity Cache (last level before HBM)

// Finish time of an order under the dispatch model, in key tiles.
int64_t model_makespan(const std::vector<int32_t>& order, const std::vector<int32_t>& cost_of) {
  int64_t span = 0;
  for (int x = 0; x < pcp_geom::kXcds; ++x) {
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> cu;
    for (int c = 0; c < kCusPerXcd; ++c) cu.push(0);
    for (size_t e = x; e < order.size(); e += pcp_geom::kXcds) {
      if (order[e] < 0) continue;
      const int64_t t = cu.top() + cost_of[order[e]];
      cu.pop();
      cu.push(t);
    }
    while (cu.size() > 1) cu.pop();
    span = std::max(span, cu.top());
  }
  return span;
}

// The kernels' built-in launch order as unit ids (mirrors attn_fwd_kernel's
// decode when no order is given).
std::vector<int32_t> builtin_order(int num_rows, int groups_total, int qt) {
  const int n = num_rows * groups_total * qt;
  const int w = pcp_geom::kXcds * pcp_geom::kXcdRun;
  const int full = (n / w) * w;
  std::vector<int32_t> order(n);
  for (int b = 0; b < n; ++b) {
    int u = b;
    if (b < full) {
      const int win = b / w, within = b - win * w;
      u = win * w + (within % pcp_geom::kXcds) * pcp_geom::kXcdRun + within / pcp_geom::kXcds;
    }
    const int qt_rev = u % qt, rest = u / qt;
    const int grp = rest % groups_total, row = num_rows - 1 - rest / groups_total;
    order[b] = (row * groups_total + grp) * qt + (qt - 1 - qt_rev);
  }
  return order;
}

struct Unit {
  int32_t id;
  int32_t cost;
  int32_t seq;  // position in the natural enumeration (ties keep it)
  int64_t kv;   // K/V set it reads: request * num_kv_heads + KV head
  int64_t keys;  // keys of that set it reads (a split decode row: the whole row's)
};

// K/V-grouped order: the units reading one request's K/V for one KV head
// are kept together on one XCD and next to each other in its queue, so
// that their shared key tiles stay in that XCD's L2 while they run. Groups
// go longest first to the least loaded XCD; each XCD runs its groups in that
// order, each group's units longest first. Returned empty (not worth it)
// when the launch's K/V (at kv_elem_bytes per element) fits the Infinity
// Cache, where the longest-first order of single units balances the end of
// the launch better, or when a group costs more than total / (8 *
// kPiecesPerXcd), where keeping it whole would unbalance the XCDs.
std::vector<int32_t> grouped_order(const std::vector<Unit>& units, int head_dim,
                                   int kv_elem_bytes) {
  using namespace pcp_geom;
  std::vector<int> by_kv(units.size());
  int64_t total = 0;
  for (size_t u = 0; u < units.size(); ++u) {
    by_kv[u] = (int)u;
    total += units[u].cost;
  }
  std::stable_sort(by_kv.begin(), by_kv.end(),
                   [&](int x, int y) { return units[x].kv < units[y].kv; });
  const int64_t cap = std::max<int64_t>(1, total / (kXcds * kPiecesPerXcd));
  std::vector<std::vector<int>> pieces;  // one per K/V group
  std::vector<int64_t> piece_cost;
  int64_t kv_bytes = 0;
  for (size_t i = 0; i < by_kv.size(); ++i) {
    const int u = by_kv[i];
    if (i == 0 || units[u].kv != units[by_kv[i - 1]].kv) {
      pieces.emplace_back();
      piece_cost.push_back(0);
      int64_t keys = 0;  // the group's footprint: the most keys one of its units reads
      for (size_t j = i; j < by_kv.size() && units[by_kv[j]].kv == units[u].kv; ++j)
        keys = std::max(keys, units[by_kv[j]].keys);
      kv_bytes += keys * head_dim * kv_elem_bytes * 2;  // K and V
    }
    pieces.back().push_back(u);
    piece_cost.back() += units[u].cost;
    if (piece_cost.back() > cap) return {};
  }
  if (kv_bytes <= kMallBytes) return {};
  std::vector<int> by_cost(pieces.size());
  for (size_t i = 0; i < pieces.size(); ++i) by_cost[i] = (int)i;
  std::stable_sort(by_cost.begin(), by_cost.end(),
                   [&](int x, int y) { return piece_cost[x] > piece_cost[y]; });
  std::vector<std::vector<int32_t>> queue(kXcds);
  int64_t load[kXcds] = {};
  for (int i : by_cost) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += piece_cost[i];
    std::vector<int> m = pieces[i];
    std::stable_sort(m.begin(), m.end(), [&](int x, int y) {
      return units[x].cost != units[y].cost ? units[x].cost > units[y].cost
                                            : units[x].seq < units[y].seq;
    });
    for (int u : m) queue[best].push_back(units[u].id);
  }
  size_t longest = 0;
  for (auto& qx : queue) longest = std::max(longest, qx.size());
  std::vector<int32_t> order(longest * kXcds);
  for (size_t e = 0; e < order.size(); ++e) {
    const auto& qx = queue[e % kXcds];
    const size_t i = e / kXcds;
    order[e] = i < qx.size() ? qx[i] : -1;
  }
  return order;
}

}  // namespace

extern "C" int pcp_attn_schedule(int pass, const pcp_row_t* rows, int num_rows, int max_q_len,
                                 int num_q_heads, int num_kv_heads, int head_dim,
                                 int decode_splits, int kv_elem_bytes, int32_t* order,
                                 int capacity) {
  using namespace pcp_geom;
  if (pass < 0 || pass > 2) return PCP_EINVAL;
  if (num_rows < 0 || max_q_len < 0 || capacity < 0 || decode_splits < 1) return PCP_EINVAL;
  if (kv_elem_bytes != 1 && kv_elem_bytes != 2) return PCP_EINVAL;
  if (num_rows > 0 && rows == nullptr) return PCP_EINVAL;
  if (capacity > 0 && order == nullptr) return PCP_EINVAL;
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0) return PCP_EINVAL;
  if (!supported_dim(head_dim)) return PCP_EUNSUPPORTED;
  const bool context = pass != 0;    // context tiles (passes 1 and 2)
  const bool new_tokens = pass != 1;  // new-token tiles (passes 0 and 2)
  const int splits = context ? decode_splits : 1;
  const int group = num_q_heads / num_kv_heads;
  const int hg = heads_per_group(group);
  const int groups_total = num_kv_heads * (group / hg);
  const int bq = block_q(hg);
  const int bn = block_n(head_dim);
  const int64_t qt64 = q_tiles(max_q_len, hg, context, splits);
  for (int r = 0; r < num_rows; ++r)
    if (rows[r].q_len < 0 || rows[r].q_len > max_q_len) return PCP_EINVAL;
  if (qt64 > INT32_MAX || (int64_t)num_rows * groups_total * qt64 > INT32_MAX)
    return PCP_EOVERFLOW;
  const int qt = (int)qt64;

  // Units of every (row, group) in query-tile order last to first, with the
  // key tiles the kernel will stream for each.
  std::vector<Unit> units;
  std::vector<int> run_start;  // index into units of each run's first unit
  int seq = 0;
  for (int r = 0; r < num_rows; ++r) {
    const pcp_row_t& row = rows[r];
    const bool split = context && splits > 1 && row.q_len == 1 && row.k_len <= 0;
    for (int g = 0; g < groups_total; ++g) {
      int in_run = 0;
      for (int q = qt - 1; q >= 0; --q) {
        // 64-bit: the row fields are the caller's and not range-checked here
        int64_t tiles;
        int64_t keys;
        const int64_t ctx = std::max<int64_t>(row.ctx_len_local, 0);
        if (split) {
          if (q >= splits) continue;
          const int64_t all = (ctx + bn - 1) / bn;
          const int64_t per = (all + splits - 1) / splits;
          tiles = std::max<int64_t>(0, std::min<int64_t>(all - q * per, per));
          keys = ctx;
        } else {
          const int64_t q0 = (int64_t)q * bq;
          if (row.q_len <= q0) continue;
          tiles = keys = 0;
          if (context) {
            tiles += (ctx + bn - 1) / bn;
            keys += ctx;
          }
          if (new_tokens) {
            const int64_t t_last = std::min<int64_t>(q0 + bq, row.q_len) - 1;
            const int64_t k_len = row.k_len;
            const int64_t nnew =
                std::max<int64_t>(0, std::min<int64_t>(k_len, k_len - row.q_len + t_last + 1));
            tiles += (nnew + bn - 1) / bn;
            keys += nnew;
          }
        }
        tiles = std::min<int64_t>(tiles, INT32_MAX / 2);  // a cost, not an index
        if (in_run == 0) run_start.push_back((int)units.size());
        in_run = (in_run + 1) % kXcdRun;
        units.push_back({(int32_t)(((int64_t)r * groups_total + g) * qt + q),
                         (int32_t)(tiles + kUnitStartCost), (int32_t)seq++,
                         (int64_t)row.req * num_kv_heads + g / (group / hg), keys});
      }  // runs restart with every (row, group) pair
    }
  }
  if (units.empty()) return 0;

  // Runs, longest first, each to the least loaded XCD.
  const int nruns = (int)run_start.size();
  std::vector<int64_t> run_cost(nruns, 0);
  for (int i = 0; i < nruns; ++i) {
    const int end = i + 1 < nruns ? run_start[i + 1] : (int)units.size();
    for (int u = run_start[i]; u < end; ++u) run_cost[i] += units[u].cost;
  }
  std::vector<int> by_cost(nruns);
  for (int i = 0; i < nruns; ++i) by_cost[i] = i;
  std::stable_sort(by_cost.begin(), by_cost.end(),
                   [&](int x, int y) { return run_cost[x] > run_cost[y]; });
  std::vector<std::vector<Unit>> queue(kXcds);
  int64_t load[kXcds] = {};
  for (int i : by_cost) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += run_cost[i];
    const int end = i + 1 < nruns ? run_start[i + 1] : (int)units.size();
    for (int u = run_start[i]; u < end; ++u) queue[best].push_back(units[u]);
  }

  // Longest first within each XCD, then interleave.
  size_t longest = 0;
  for (auto& qx : queue) {
    std::stable_sort(qx.begin(), qx.end(), [](const Unit& x, const Unit& y) {
      return x.cost != y.cost ? x.cost > y.cost : x.seq < y.seq;
    });
    longest = std::max(longest, qx.size());
  }
  if ((int64_t)longest * kXcds > INT32_MAX) return PCP_EOVERFLOW;
  std::vector<int32_t> lpt(longest * kXcds);
  for (size_t e = 0; e < lpt.size(); ++e) {
    const auto& qx = queue[e % kXcds];
    const size_t i = e / kXcds;
    lpt[e] = i < qx.size() ? qx[i].id : -1;
  }

  // Keep the built-in order unless the model says longest first is faster.
  const int total = num_rows * groups_total * qt;
  std::vector<int32_t> cost_of(total, 0);  // 0: the unit exits at once
  for (const Unit& u : units) cost_of[u.id] = u.cost;
  std::vector<int32_t> builtin = builtin_order(num_rows, groups_total, qt);
  const int64_t t_lpt = model_makespan(lpt, cost_of);
  const int64_t t_builtin = model_makespan(builtin, cost_of);
  const std::vector<int32_t> grouped = grouped_order(units, head_dim, kv_elem_bytes);
  if ((int64_t)grouped.size() > INT32_MAX) return PCP_EOVERFLOW;
  const std::vector<int32_t>& best =
      !grouped.empty() ? grouped
                       : ((double)t_lpt < (1.0 - kMinGain) * (double)t_builtin ? lpt : builtin);
  const int64_t n = (int64_t)best.size();
  const int64_t w = std::min<int64_t>(n, capacity);
  for (int64_t e = 0; e < w; ++e) order[e] = best[e];
  return (int)n;
}

// Key-range splits of the decode rows of one context pass (fused: of one
// pcp_attn_rank_share launch). A decode row is one workgroup per KV head
// streaming its whole cached context, and one workgroup fills a CU.
extern "C" int pcp_choose_decode_splits(const pcp_row_t* rows, int num_rows, int num_kv_heads,
                                        int fused) {
  constexpr int64_t kFillUnits = 512;      // workgroups with work that keep the chip busy
  constexpr int64_t kCus = 256;            // MI355X compute units
  constexpr int64_t kMinKeysPerSplit = 256;
  if (num_rows < 0 || num_kv_heads < 1 || (num_rows > 0 && rows == nullptr)) return PCP_EINVAL;
  int64_t dec_rows = 0, others = 0, sum_keys = 0, longest = 0;
  for (int r = 0; r < num_rows; ++r) {
    const pcp_row_t& row = rows[r];
    if (row.q_len == 1 && row.k_len <= 0) {  // decode row: split candidate
      const int64_t keys = std::max<int64_t>(row.ctx_len_local, 0);
      ++dec_rows;
      sum_keys += keys;
      longest = std::max(longest, keys);
    } else if (row.q_len > 0 && (row.ctx_len_local > 0 || (fused && row.k_len > 0))) {
      others += ((int64_t)row.q_len + 127) / 128;  // at least this many units per KV head
    }
  }
  // Busy enough already (or nothing to split): splitting only adds
  // per-workgroup latency and a combine pass.
  if (dec_rows == 0 || longest <= 0) return 1;
  if ((dec_rows + others) * num_kv_heads >= kFillUnits) return 1;
  // Ranges of the longest row hold no more keys than one CU's even share of
  // all decode keys (sum * KV heads / CUs), and no fewer than about
  // kMinKeysPerSplit: rows of one length then run as a single round of
  // ranges, and rows of mixed lengths keep the longest from finishing last.
  const int64_t total = sum_keys * num_kv_heads;  // share = total / kCus keys
  const int64_t splits = total >= kCus * kMinKeysPerSplit
                             ? (longest * kCus + total - 1) / total
                             : (longest + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
  return (int)std::max<int64_t>(1, std::min<int64_t>(splits, pcp_geom::kMaxDecodeSplits));
}
