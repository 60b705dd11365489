// ring_model.h -- protocol cost model of the ring collectives on one MI355X.
//
// Form of the model: "NCCL" book (aireadcode.com), ch. 5, ring.cc -- a ring
// collective's latency is nSteps hops of a per-hop latency, its bandwidth term
// is the bytes it moves over the achievable bandwidth (bus bandwidth times
// nRanks / nSteps), and the flag-packed protocols pay for their flags: LL
// half the bandwidth, LL128 a sixteenth.
//
// Bulk protocol: the latency and bandwidth terms overlap (the ring pipelines
// steps while the first chunks are still in flight), so they are combined as
// a 2-norm rather than added:
//
//   t = base + sqrt((hops * hop_latency)^2 + (bytes / bandwidth)^2)
//
// with hops = 2(N-1) for the all-reduce and N-1 for reduce-scatter and
// all-gather and bytes = the HBM bytes of the method; a hop costs ~2.45 us
// and the kernel sustains ~6.9 TB/s.
//
// Line protocols (FLAG, WIDE): a workgroup moves its part of every stage in
// steps of at most one slot, and up to a few MiB its speed is set by steps,
// not bytes. The first step of every stage waits for the neighbour's previous
// stage (a hop); further steps of the same stage find their lines already
// written and cost a step time. Both grow with the lines of a step (lines per
// thread), and both grow when more workgroups than compute units share the
// device. Large messages meet the line protocols' byte rate instead:
//
//   steps_us = crowd * (hops * hop(L) + stages * (steps - 1) * step(L))
//   t = base + sqrt(steps_us^2 + (line_bytes / line_bandwidth)^2)
//
// with L the lines of a workgroup's step, steps the slot steps of one stage
// of one workgroup (all loops), hop(L) = a + b * L / 256, step(L) likewise,
// crowd = 1 + c * (workgroups / CUs - 1) above one workgroup per CU, and
// line_bytes the method bytes with the line format's FIFO factor. The
// constants are fitted to bench.py sweeps on MI355X (4, 8 and 16 ranks with
// as many channels, 1, 2, 4 and 8 workgroups per channel, 4 KiB .. 8 MiB per
// rank); the library evaluates every workgroup count it may launch and takes
// the fastest.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "ring_plan.h"

namespace ringsim {

// ---------------------------------------------------------------------------
// Workgroups of a bulk call
// ---------------------------------------------------------------------------

// Longest unit (bytes) one workgroup of a ring launch moves in one stage with
// `wpc` workgroups per channel; no step is longer. The first loop of channel
// 0 (the longest channel) holds the longest units. `count` is per rank for
// the all-reduce and per block for reduce-scatter and all-gather.
inline int64_t ring_max_unit_bytes(int64_t count, int nranks, int nchannels, int64_t chunk_elems, bool allreduce,
                                   int esize, int wpc) {
  const int64_t A = 16 / esize;
  const int64_t l0 = channel_span(count, nchannels, A);
  const int64_t cur = allreduce ? ar_loop_chunk(l0, nranks, chunk_elems, A) : min64(chunk_elems, l0);
  return align_up(div_up(cur, wpc), A) * esize;
}

// Bulk workgroups per channel of one call, at most `wpc_max` (the
// communicator's count). A call whose stages are short takes fewer: about
// one per kBulkPartBytes of a channel's stage, at least two, and rounded up
// so that channels x workgroups is a multiple of the 8 XCDs (the rank-major
// workgroup ids then put every workgroup of a pipeline on one XCD). A call
// ends with its slowest pipeline, and fewer, fuller pipelines finish sooner:
// 8 ranks x 8 channels at 4 KiB - 512 KiB per rank 31.5-32.7 us with 2
// against 37-39 us with 8; 4 ranks x 4 KiB on one channel 15.7 us with 8
// against 17.1 us with 16. A smaller count is taken only when one
// workgroup's stage still fits half of its FIFO of `nslots` slots.
constexpr int64_t kBulkPartBytes = 4096;
constexpr int kXcds = 8;
inline int bulk_call_wpc(int64_t count, int nranks, int nchannels, int64_t chunk_elems, bool allreduce, int esize,
                         int wpc_max, int64_t slot_bytes, int nslots) {
  int64_t w = std::max<int64_t>(
      2, div_up(ring_max_unit_bytes(count, nranks, nchannels, chunk_elems, allreduce, esize, 1), kBulkPartBytes));
  while (w < wpc_max && ((int64_t)nchannels * w) % kXcds != 0) ++w;
  if (w >= wpc_max) return wpc_max;
  const int64_t unit = ring_max_unit_bytes(count, nranks, nchannels, chunk_elems, allreduce, esize, (int)w);
  if (2 * div_up(unit, slot_bytes) > (int64_t)nslots) return wpc_max;
  return (int)w;
}

enum ModelProto : int { kModelBulk = 0, kModelFlag = 1, kModelWide = 2 };

struct RingModel {
  double base_us = 3.0;
  double bulk_hop_us = 2.45;
  double bulk_gbs = 6900.0;
  // Line protocols, [FLAG, WIDE][a, b]: per hop and per further step,
  // a + b * lines / 256 microseconds.
  double line_base_us = 6.83;
  double line_hop_us[2][2] = {{0.727, 0.400}, {0.822, 0.170}};
  double line_step_us[2][2] = {{0.971, 0.097}, {0.888, 0.095}};
  double line_crowd = 0.368;
  double line_gbs = 4540.0;
  // Double-binary tree (WIDE lines, one line per thread per step): base,
  // per hop a + b * lines / 256, per further step, and how much each grows
  // per workgroup per compute unit beyond the first.
  double tree_base_us = 7.152;
  double tree_hop_us[2] = {0.762, 0.069};
  double tree_step_us = 1.037;
  double tree_hop_crowd = 0.168;
  double tree_step_crowd = 0.41;
};

enum ModelColl : int { kModelAllReduce = 0, kModelReduceScatter = 1, kModelAllGather = 2 };

// FIFO bytes per payload byte of each protocol's slots.
inline double fifo_factor(int proto) { return proto == kModelFlag ? 2.0 : proto == kModelWide ? 4.0 / 3.0 : 1.0; }

// Method bytes of one call with S bytes per rank (all-reduce buffer,
// reduce-scatter input, all-gather output), summed over ranks.
inline double model_bytes(int coll, int nranks, double s, int proto) {
  const double n = nranks;
  const double fifo = (coll == kModelAllReduce ? 4.0 * (n - 1.0) : 2.0 * (n - 1.0)) * s;
  const double user = coll == kModelAllReduce ? 2.0 * n * s : (n + 1.0) * s;
  return user + fifo_factor(proto) * fifo;
}

inline double model_hops(int coll, int nranks) {
  return coll == kModelAllReduce ? 2.0 * (nranks - 1) : (double)(nranks - 1);
}

// Predicted microseconds of a bulk-protocol call.
inline double bulk_model_us(const RingModel& m, int coll, int nranks, double bytes_per_rank) {
  if (nranks <= 1) return m.base_us;
  const double bytes = model_bytes(coll, nranks, bytes_per_rank, kModelBulk);
  return m.base_us + std::hypot(model_hops(coll, nranks) * m.bulk_hop_us, bytes / (m.bulk_gbs * 1e3));
}

// Shape of a line launch: workgroups per channel, payload bytes per line,
// lines per slot, chunk bytes, and the device's compute units.
struct LineShape {
  int wpc;
  double payload;
  double slot_lines;
  double chunk_bytes;
  int cus;
};

// Predicted microseconds of a line-protocol (FLAG or WIDE) call. Every
// collective moves S / (N * C) bytes per stage of one (rank, channel), in
// units of at most one chunk.
inline double line_model_us(const RingModel& m, int coll, int nranks, int nchannels, double bytes_per_rank, int proto,
                            const LineShape& sh) {
  if (nranks <= 1) return m.base_us;
  const int k = proto == kModelWide ? 1 : 0;
  const double stage_bytes = bytes_per_rank / ((double)nranks * nchannels);
  const double unit = std::min(stage_bytes, sh.chunk_bytes);
  const double lines = std::min(std::ceil(unit / sh.wpc / sh.payload), sh.slot_lines);
  const double steps = std::max(1.0, std::ceil(std::ceil(stage_bytes / sh.wpc / sh.payload) / sh.slot_lines));
  const double hops = model_hops(coll, nranks);
  const double wgs = (double)nranks * nchannels * sh.wpc;
  const double crowd = 1.0 + m.line_crowd * std::max(0.0, wgs / sh.cus - 1.0);
  const double hop = m.line_hop_us[k][0] + m.line_hop_us[k][1] * lines / 256.0;
  const double step = m.line_step_us[k][0] + m.line_step_us[k][1] * lines / 256.0;
  const double steps_us = crowd * (hops * hop + (hops + 1.0) * (steps - 1.0) * step);
  const double bytes = model_bytes(coll, nranks, bytes_per_rank, proto);
  return m.line_base_us + std::hypot(steps_us, bytes / (m.line_gbs * 1e3));
}

// Predicted microseconds of a double-binary-tree all-reduce: the reduce
// climbs `depth` hops to each root and the broadcast descends as many, one
// slice of `slice_bytes` per step in lines of `line_payload` bytes; each
// tree's half of the buffer is split over `tree_channels` channels, and the
// 4 x N x tree_channels workgroups (two trees, an up and a down role each)
// share `cus` compute units: beyond one workgroup per unit, hops and steps
// slow down in proportion. Fitted to the tree's own sweeps at 16, 8 and 4
// ranks with one and two workgroups per unit, 1 KiB to 2 MiB per rank
// (within 6%).
inline double tree_model_us(const RingModel& m, int nranks, int depth, int tree_channels, double slice_bytes,
                            double line_payload, double bytes_per_rank, int cus) {
  if (nranks <= 1) return m.base_us;
  const double per_channel = std::ceil(bytes_per_rank / 2.0 / tree_channels);
  const double lines = std::ceil(std::min(per_channel, slice_bytes) / line_payload);
  const double steps = std::max(1.0, std::ceil(per_channel / slice_bytes));
  const double extra = std::max(0.0, 4.0 * nranks * tree_channels / cus - 1.0);
  return m.tree_base_us +
         2.0 * depth * (m.tree_hop_us[0] + m.tree_hop_us[1] * lines / 256.0) * (1.0 + m.tree_hop_crowd * extra) +
         (steps - 1.0) * m.tree_step_us * (1.0 + m.tree_step_crowd * extra);
}

}  // namespace ringsim
