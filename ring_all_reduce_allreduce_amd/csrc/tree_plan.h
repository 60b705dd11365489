// tree_plan.h -- shape and partition of the double-binary-tree all-reduce.
// Host and device code both use these helpers, so the launch and the
// kernels agree on every range.
//
// Sources: "NCCL" book (aireadcode.com), ch. 4, ncclGetBtree: a rank's links
// follow from its lowest set bit, rank 0 being the root with a single child;
// ncclGetDtree: a second tree that mirrors the first for an even number of
// ranks and shifts it by one rank for an odd number, the two trees each
// reducing and broadcasting half of the data. Ch. 5, tree.cc: the tree serves
// the all-reduce only.
#pragma once

#include "ring_plan.h"

namespace ringsim {

struct TreeLinks {
  int parent;  // -1 at the root
  int kid[2];  // first and second child, -1 = none
};

// Links of `rank` in the basic binary tree over `nranks` ranks. The lowest
// set bit b of the rank decides everything: the parent clears b and sets the
// bit 2b (or only clears b when that would leave the rank range); the children sit b/2
// below and up to b/2 above, the upper one shrinking to the largest power of
// two that stays in range. Rank 0 takes b = the first power of two >= nranks.
inline TreeLinks basic_tree(int nranks, int rank) {
  int b = 1;
  while (b < nranks && (rank & b) == 0) b <<= 1;
  const int down = b >> 1;
  TreeLinks l{-1, {-1, -1}};
  if (rank == 0) {
    if (nranks > 1) l.kid[1] = down;
    return l;
  }
  const int up = (rank & ~b) | (b << 1);
  l.parent = up < nranks ? up : (rank & ~b);
  if (down > 0) {
    l.kid[0] = rank - down;
    for (int s = down; s > 0; s >>= 1) {
      if (rank + s < nranks) {
        l.kid[1] = rank + s;
        break;
      }
    }
  }
  return l;
}

// Links of `rank` in tree `t` (0 or 1) of the double binary tree. Tree 1
// renames the ranks of tree 0: r plays nranks-1-r for an even count, r-1
// (mod nranks) for an odd one; links are renamed back the same way and keep
// their child slot.
inline TreeLinks double_tree(int nranks, int rank, int t) {
  if (t == 0) return basic_tree(nranks, rank);
  const bool mirror = nranks % 2 == 0;
  const int role = mirror ? nranks - 1 - rank : (rank + nranks - 1) % nranks;
  const TreeLinks l = basic_tree(nranks, role);
  auto back = [&](int x) { return x < 0 ? -1 : (mirror ? nranks - 1 - x : (x + 1) % nranks); };
  return TreeLinks{back(l.parent), {back(l.kid[0]), back(l.kid[1])}};
}

// Edges on the longest root-to-leaf path of either tree.
inline int double_tree_depth(int nranks) {
  int depth = 0;
  for (int t = 0; t < 2; ++t) {
    for (int r = 0; r < nranks; ++r) {
      int d = 0;
      for (int x = r; d <= nranks; ++d) {
        x = double_tree(nranks, x, t).parent;
        if (x < 0) break;
      }
      depth = depth > d ? depth : d;
    }
  }
  return depth;
}

// First element of tree 1's half: half of the count, rounded up to whole
// 16-byte units (as every ring channel boundary is) and clipped to the count.
RP_HD int64_t tree_split(int64_t count, int64_t align) {
  return min64(count, align_up(div_up(count, 2), align));
}

// Elements [lo, hi) of tree `t`, channel `c` of `nchannels`.
RP_HD Range tree_channel_range(int64_t count, int t, int c, int nchannels, int64_t align) {
  const int64_t split = tree_split(count, align);
  const int64_t base = t == 0 ? 0 : split;
  const int64_t len = t == 0 ? split : count - split;
  const Range r = channel_range(len, nchannels, c, align);
  return Range{base + r.lo, base + r.hi};
}

}  // namespace ringsim
