// planner_check.cpp -- host driver for the library's planning headers
// (ring_plan.h, tree_plan.h, ring_model.h), built by a CPU test with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer. It reads commands on
// stdin and prints what the headers compute, for the test to compare with
// the oracle's own partition and tree shapes:
//   plan <coll> <count> <nranks> <nchannels> <chunk_bytes> <elem_size>
//       -> one line "c l k lo hi" per chunk (k = -1 for reduce-scatter and
//          all-gather), then "end"
//   tree <nranks>  -> "t r parent kid0 kid1" for both trees, "depth d", "end"
//   model <nranks> <nchannels> <bytes_per_rank>
//       -> the bulk, FLAG, WIDE (1..8 workgroups) and tree predictions, "end"
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <string>

#include "../ring_all_reduce_allreduce_amd/csrc/ring_model.h"
#include "../ring_all_reduce_allreduce_amd/csrc/ring_plan.h"
#include "../ring_all_reduce_allreduce_amd/csrc/tree_plan.h"

using namespace ringsim;

static void plan(int coll, int64_t count, int n, int nch, int64_t chunk_bytes, int64_t esize) {
  const int64_t A = 16 / esize;
  const int64_t chunk = chunk_bytes / esize;
  for (int c = 0; c < nch; ++c) {
    const Range ch = channel_range(count, nch, c, A);
    const int64_t L = ch.hi - ch.lo;
    if (coll == 0) {
      int64_t l = 0;
      for (int64_t off = 0; off < L; off += (int64_t)n * chunk, ++l) {
        const int64_t rem = L - off;
        const int64_t cur = ar_loop_chunk(rem, n, chunk, A);
        for (int k = 0; k < n; ++k) {
          const Range r = ar_chunk(off, rem, cur, k);
          // every workgroup split of the chunk tiles it exactly
          for (int parts = 1; parts <= 16; parts *= 2) {
            int64_t covered = 0;
            for (int w = 0; w < parts; ++w) {
              const Range p = split_part(r.hi - r.lo, parts, w, A);
              if (p.lo != covered && p.hi > p.lo) std::printf("bad split\n");
              covered = p.hi > p.lo ? p.hi : covered;
            }
            if (covered != r.hi - r.lo) std::printf("bad split\n");
          }
          std::printf("%d %lld %d %lld %lld\n", c, (long long)l, k, (long long)(ch.lo + r.lo), (long long)(ch.lo + r.hi));
        }
        // stage j of rank r visits chunk (r + N - 1 - j) mod N
        for (int rk = 0; rk < n; ++rk)
          for (int j = 0; j < 2 * n - 1; ++j)
            if (ring_chunk(rk, n, j) != ((rk + 2 * n - 1 - j) % n)) std::printf("bad chunk id\n");
      }
    } else {
      int64_t l = 0;
      for (int64_t off = 0; off < L; off += chunk, ++l)
        std::printf("%d %lld -1 %lld %lld\n", c, (long long)l, (long long)(ch.lo + off),
                    (long long)(ch.lo + min64(off + chunk, L)));
    }
  }
  std::printf("end\n");
}

static void tree(int n) {
  for (int t = 0; t < 2; ++t)
    for (int r = 0; r < n; ++r) {
      const TreeLinks l = double_tree(n, r, t);
      std::printf("%d %d %d %d %d\n", t, r, l.parent, l.kid[0], l.kid[1]);
    }
  std::printf("depth %d\nend\n", double_tree_depth(n));
}

static void model(int n, int nch, double bytes) {
  const RingModel m;
  std::printf("bulk %.6f\n", bulk_model_us(m, kModelAllReduce, n, bytes));
  for (int proto : {kModelFlag, kModelWide})
    for (int w = 1; w <= 8; w *= 2) {
      const LineShape sh{w, proto == kModelWide ? 12.0 : 8.0, 1024.0, 524288.0, 256};
      std::printf("line %d %d %.6f\n", proto, w, line_model_us(m, kModelAllReduce, n, nch, bytes, proto, sh));
    }
  for (int tc = 1; tc <= 8; tc *= 2)
    std::printf("tree %d %.6f\n", tc, tree_model_us(m, n, double_tree_depth(n), tc, 3072.0, 12.0, bytes, 256));
  std::printf("end\n");
}

// Workgroups per channel of a bulk call, and the longest unit of one
// workgroup's stage at that count and at one workgroup.
static void bulkw(int coll, int64_t count, int n, int nch, int64_t chunk_bytes, int esize, int wpc_max,
                  int64_t slot_bytes, int nslots) {
  const int64_t chunk = chunk_bytes / esize;
  const int w = bulk_call_wpc(count, n, nch, chunk, coll == 0, esize, wpc_max, slot_bytes, nslots);
  const int64_t unit = ring_max_unit_bytes(count, n, nch, chunk, coll == 0, esize, w);
  const int64_t unit1 = ring_max_unit_bytes(count, n, nch, chunk, coll == 0, esize, 1);
  std::printf("%d %lld %lld\nend\n", w, (long long)unit, (long long)unit1);
}

int main() {
  std::string cmd;
  while (std::cin >> cmd) {
    if (cmd == "plan") {
      int coll, n, nch;
      long long count, chunk_bytes, esize;
      std::cin >> coll >> count >> n >> nch >> chunk_bytes >> esize;
      plan(coll, count, n, nch, chunk_bytes, esize);
    } else if (cmd == "tree") {
      int n;
      std::cin >> n;
      tree(n);
    } else if (cmd == "bulkw") {
      int coll, n, nch, esize, wpc_max, nslots;
      long long count, chunk_bytes, slot_bytes;
      std::cin >> coll >> count >> n >> nch >> chunk_bytes >> esize >> wpc_max >> slot_bytes >> nslots;
      bulkw(coll, count, n, nch, chunk_bytes, esize, wpc_max, slot_bytes, nslots);
    } else if (cmd == "model") {
      int n, nch;
      double bytes;
      std::cin >> n >> nch >> bytes;
      model(n, nch, bytes);
    }
    std::fflush(stdout);
  }
  return 0;
}
