// ring_plan.h -- partition of a collective into channels, loops, chunks and
// workgroup parts. Shared by the host planner (ringsim_debug_plan) and the
// device kernels so that both always walk the same ranges.
//
// Sources: "NCCL" book (aireadcode.com), ch. 2, s. 2.2: a channel takes
// count/nChannels elements; s. 2.3, RingARAlgorithm::getNextSendAddr: a loop
// spans nRanks chunks, the last loop shrinks the chunk to
// alignUp(divUp(remaining, nRanks), 16/elemSize), and at stage s of a loop
// rank r works on chunk (r + nRanks - 1 - s) mod nRanks.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define RP_HD __host__ __device__ __forceinline__
#else
#define RP_HD inline
#endif

namespace ringsim {

struct Range {
  int64_t lo;
  int64_t hi;
};

RP_HD int64_t div_up(int64_t x, int64_t y) { return (x + y - 1) / y; }
RP_HD int64_t align_up(int64_t x, int64_t a) { return div_up(x, a) * a; }
RP_HD int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
RP_HD int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Elements per channel: count / nChannels rounded up to whole 16-byte units,
// so channel boundaries stay vector aligned; trailing channels may be empty.
RP_HD int64_t channel_span(int64_t count, int nchannels, int64_t align) {
  return count > 0 ? align_up(div_up(count, nchannels), align) : 0;
}

RP_HD Range channel_range(int64_t count, int nchannels, int c, int64_t align) {
  const int64_t per = channel_span(count, nchannels, align);
  const int64_t lo = min64((int64_t)c * per, count);
  return Range{lo, min64(lo + per, count)};
}

// All-reduce: chunk size of a loop that has `rem` elements of its channel left.
RP_HD int64_t ar_loop_chunk(int64_t rem, int nranks, int64_t chunk, int64_t align) {
  return rem >= (int64_t)nranks * chunk ? chunk : align_up(div_up(rem, nranks), align);
}

// Chunk k of the loop at channel offset `off` ([off, off+rem) is what is left
// of the channel); relative to the channel start, possibly empty.
RP_HD Range ar_chunk(int64_t off, int64_t rem, int64_t cur, int k) {
  return Range{off + min64((int64_t)k * cur, rem), off + min64((int64_t)(k + 1) * cur, rem)};
}

// Chunk handled by `rank` at all-reduce / reduce-scatter stage `stage`.
RP_HD int ring_chunk(int rank, int nranks, int stage) {
  return (rank + 2 * nranks - 1 - stage) % nranks;
}

// Block handled by `rank` at all-gather stage `stage`: (rank - stage) mod N.
RP_HD int ag_block(int rank, int nranks, int stage) {
  return (rank - stage % nranks + nranks) % nranks;
}

// Part `w` of `parts` of an n-element range, in whole 16-byte units. This
// only divides a chunk among the workgroups of one channel; it does not
// change which chunk (and so which fold order) an element belongs to.
RP_HD Range split_part(int64_t n, int parts, int w, int64_t align) {
  const int64_t sub = align_up(div_up(n, parts), align);
  const int64_t lo = min64((int64_t)w * sub, n);
  return Range{lo, min64(lo + sub, n)};
}

}  // namespace ringsim
