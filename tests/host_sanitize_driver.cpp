// Host code of libpcpattn under AddressSanitizer and UndefinedBehaviorSanitizer
// (test infrastructure). tests/test_host_sanitized.py compiles this file
// together with the library's host sources (pcp_plan.cpp, pcp_sched.cpp and
// the attention calls' argument checks in pcp_attn_check.h) with g++
// -fsanitize=address,undefined, feeds it commands on stdin and compares the
// answers with the oracle and with the GPU library's own host entry points.
//
// One command per line, integers separated by spaces; one answer line each:
//   PLAN resplit B P r D rd bs cap cu[B+1] ctx[B]
//        -> "n" then min(n, cap) rows of 9 ints (pcp_plan_rows / _resplit)
//   SLOT B max_blocks D rd bs cap cu[B+1] ctx[B] table[B*max_blocks]
//        -> "n" then min(n, cap) slots                 (pcp_slot_mapping)
//   SCHED pass R max_q_len hq hkv d splits elem cap rows[R*9]
//        -> "n" then min(n, cap) unit ids              (pcp_attn_schedule)
//   SPLITS R hkv fused rows[R*9]
//        -> the split count                     (pcp_choose_decode_splits)
//   CHECK pass fp8 num_rows total_q total_k max_q_len num_blocks block_size
//         num_reqs max_blocks hq hkv d decode_splits num_units scale_x1000
//         ptrs
//        -> the return code of the argument checks; ptrs is a bit mask of
//           the pointers given (bit 0 q, 1 k, 2 v, 3 kc, 4 vc, 5 q_ds,
//           6 k_ds, 7 v_ds, 8 rows, 9 block_tables, 10 out, 11 lse,
//           12 workspace, 13 order); given pointers are 256-byte aligned
//           dummies that are never dereferenced, bit 14 makes them only
//           8-byte aligned.
// Arrays the library writes are heap buffers of exactly `cap` entries, so
// that a write past the capacity is an AddressSanitizer error.

#include <stdint.h>
#include <stdio.h>

#include <iostream>
#include <string>
#include <vector>

#include "pcp_attn.h"
#include "pcp_attn_check.h"

namespace {

std::vector<long long> read_ints(std::istream& in, long long n) {
  std::vector<long long> v(n > 0 ? (size_t)n : 0);  // a negative count reads nothing
  for (auto& x : v) in >> x;
  return v;
}

std::vector<int32_t> as_i32(const std::vector<long long>& v) {
  return std::vector<int32_t>(v.begin(), v.end());
}

std::vector<pcp_row_t> as_rows(const std::vector<long long>& v) {
  std::vector<pcp_row_t> r(v.size() / 9);
  for (size_t i = 0; i < r.size(); ++i) {
    const long long* f = &v[9 * i];
    r[i] = {(int32_t)f[0], (int32_t)f[1], (int32_t)f[2], (int32_t)f[3], (int32_t)f[4],
            (int32_t)f[5], (int32_t)f[6], (int32_t)f[7], (int32_t)f[8]};
  }
  return r;
}

template <class T>
T* heap(long long n) {  // exactly n entries (NULL for none)
  return n > 0 ? new T[n] : nullptr;
}

}  // namespace

int main() {
  std::string cmd;
  while (std::cin >> cmd) {
    if (cmd == "PLAN") {
      const auto h = read_ints(std::cin, 8);
      const int B = (int)h[1], cap = (int)h[7];
      const auto cu = as_i32(read_ints(std::cin, B + 1));
      const auto ctx = as_i32(read_ints(std::cin, B));
      pcp_row_t* rows = heap<pcp_row_t>(cap);
      const int n = (h[0] ? pcp_plan_rows_resplit : pcp_plan_rows)(
          B, cu.empty() ? nullptr : cu.data(), ctx.empty() ? nullptr : ctx.data(), (int)h[2], (int)h[3], (int)h[4], (int)h[5], (int)h[6], rows,
          cap);
      printf("%d\n", n);
      for (int i = 0; i < n && i < cap; ++i)
        printf("%d %d %d %d %d %d %d %d %d\n", rows[i].req, rows[i].kind, rows[i].q_start,
               rows[i].q_len, rows[i].pos_start, rows[i].k_start, rows[i].k_len, rows[i].ctx_len,
               rows[i].ctx_len_local);
      delete[] rows;
    } else if (cmd == "SLOT") {
      const auto h = read_ints(std::cin, 6);
      const int B = (int)h[0], maxb = (int)h[1], cap = (int)h[5];
      const auto cu = as_i32(read_ints(std::cin, B + 1));
      const auto ctx = as_i32(read_ints(std::cin, B));
      const auto table = as_i32(read_ints(std::cin, (long long)B * maxb));
      int64_t* slots = heap<int64_t>(cap);
      const int n = pcp_slot_mapping(B, cu.empty() ? nullptr : cu.data(),
                                     ctx.empty() ? nullptr : ctx.data(),
                                     table.empty() ? nullptr : table.data(),
                                     maxb, (int)h[2], (int)h[3], (int)h[4], slots, cap);
      printf("%d\n", n);
      for (int i = 0; i < n && i < cap; ++i) printf("%lld%c", (long long)slots[i], i + 1 < n && i + 1 < cap ? ' ' : '\n');
      delete[] slots;
    } else if (cmd == "SCHED") {
      const auto h = read_ints(std::cin, 9);
      const int R = (int)h[1], cap = (int)h[8];
      const auto rows = as_rows(read_ints(std::cin, (long long)R * 9));
      int32_t* order = heap<int32_t>(cap);
      const int n = pcp_attn_schedule((int)h[0], rows.empty() ? nullptr : rows.data(), R,
                                      (int)h[2], (int)h[3], (int)h[4], (int)h[5], (int)h[6],
                                      (int)h[7], order, cap);
      printf("%d\n", n);
      for (int i = 0; i < n && i < cap; ++i) printf("%d%c", order[i], i + 1 < n && i + 1 < cap ? ' ' : '\n');
      delete[] order;
    } else if (cmd == "SPLITS") {
      const auto h = read_ints(std::cin, 3);
      const int R = (int)h[0];
      const auto rows = as_rows(read_ints(std::cin, (long long)R * 9));
      pcp_row_t* r = heap<pcp_row_t>(rows.size());  // exactly R rows on the heap
      for (size_t i = 0; i < rows.size(); ++i) r[i] = rows[i];
      printf("%d\n", pcp_choose_decode_splits(r, R, (int)h[1], (int)h[2]));
      delete[] r;
    } else if (cmd == "CHECK") {
      const auto h = read_ints(std::cin, 17);
      pcp_check::CallArgs c;
      const long long ptrs = h[16];
      const uintptr_t base = (ptrs >> 14) & 1 ? 0x10008 : 0x10000;
      auto ptr = [&](int bit) { return (ptrs >> bit) & 1 ? (void*)(base + 0x1000 * bit) : nullptr; };
      c.q = ptr(0);
      c.k = ptr(1);
      c.v = ptr(2);
      c.kc = ptr(3);
      c.vc = ptr(4);
      c.q_ds = (const float*)ptr(5);
      c.k_ds = (const float*)ptr(6);
      c.v_ds = (const float*)ptr(7);
      c.rows = (const pcp_row_t*)ptr(8);
      c.block_tables = (const int32_t*)ptr(9);
      c.out = (pcp_bf16_t*)ptr(10);
      c.lse = (float*)ptr(11);
      c.workspace = (float*)ptr(12);
      c.order = (const int32_t*)ptr(13);
      c.num_rows = (int)h[2];
      c.total_q = (int)h[3];
      c.total_k = (int)h[4];
      c.max_q_len = (int)h[5];
      c.num_blocks = (int)h[6];
      c.block_size = (int)h[7];
      c.num_reqs = (int)h[8];
      c.max_blocks = (int)h[9];
      c.hq = (int)h[10];
      c.hkv = (int)h[11];
      c.head_dim = (int)h[12];
      c.decode_splits = (int)h[13];
      c.num_units = (int)h[14];
      c.scale = (float)h[15] / 1000.f;
      printf("%d\n", pcp_check::validate(c, (pcp_check::Pass)h[0], h[1] != 0));
    } else {
      fprintf(stderr, "unknown command %s\n", cmd.c_str());
      return 2;
    }
  }
  return 0;
}
