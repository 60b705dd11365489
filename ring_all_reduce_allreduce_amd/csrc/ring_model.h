// ring_model.h -- protocol cost model of the ring collectives on one MI355X.
//
// Form of the model: "NCCL" book (aireadcode.com), ch. 5, ring.cc -- a ring
// collective's latency is nSteps hops of a per-hop latency, its bandwidth term
// is the bytes it moves over the achievable bandwidth (bus bandwidth times
// nRanks / nSteps), and the flag-packed protocols pay for their flags: LL
// half the bandwidth, LL128 a sixteenth. Here the two terms overlap (the
// ring pipelines steps while the first chunks are still in flight), so they
// are combined as a 2-norm rather than added:
//
//   t(proto) = base + sqrt((hops * hop_latency)^2 + (bytes / bandwidth)^2)
//
// with hops = 2(N-1) for the all-reduce and N-1 for reduce-scatter and
// all-gather, bytes = the HBM bytes of the method (FIFO bytes scaled by the
// line format: x2 for the flag protocol's 8-of-16-byte lines, x4/3 for the
// wide protocol's 12-of-16), and constants fitted to bench.py --sweep on
// MI355X (16 and 8 ranks and channels, 8 B .. 64 MiB per rank): a hop costs
// ~1.0 us (flag), ~1.1 us (wide) or ~2.45 us (bulk) when every chunk of
// the ring is busy; one line-protocol workgroup sustains ~11.5 (flag) or
// ~14 (wide) GB/s of method bytes, the bulk kernel ~6.9 TB/s in total.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>

namespace ringsim {

enum ModelProto : int { kModelBulk = 0, kModelFlag = 1, kModelWide = 2 };

struct RingModel {
  double base_us = 3.0;
  double hop_us[3] = {2.45, 1.0, 1.1};  // bulk, flag, wide
  double wg_gbs[3] = {0.0, 11.5, 14.0};   // line protocols: per (rank, channel) workgroup
  double line_max_gbs = 4000.0;           // line protocols' ceiling
  double bulk_gbs = 6900.0;
  // Double-binary tree (flag lines): per-hop latency, per-workgroup rate of
  // the ring-equivalent flag bytes, and the tree's ceiling.
  double tree_hop_us = 1.25;
  double tree_wg_gbs = 3.2;
  double tree_max_gbs = 1800.0;
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

// Predicted microseconds of one call.
inline double model_us(const RingModel& m, int coll, int nranks, int nchannels, double bytes_per_rank, int proto) {
  if (nranks <= 1) return m.base_us;
  const double hops = coll == kModelAllReduce ? 2.0 * (nranks - 1) : (double)(nranks - 1);
  const double bytes = model_bytes(coll, nranks, bytes_per_rank, proto);
  const double gbs = proto == kModelBulk ? m.bulk_gbs : std::min(m.line_max_gbs, m.wg_gbs[proto] * nranks * nchannels);
  return m.base_us + std::hypot(hops * m.hop_us[proto], bytes / (gbs * 1e3));
}

// Predicted microseconds of a double-binary-tree all-reduce: the reduce
// climbs `depth` hops to each root and the broadcast descends as many, all
// in flag-packed lines; the flag protocol's bytes move through the 4 x N x
// tree_channels workgroups (two trees, an up and a down role each), fitted to
// the tree's own sweeps (16 and 8 ranks: ~1.25 us per hop, ~1.8 TB/s at
// most).
inline double tree_model_us(const RingModel& m, int nranks, int depth, int tree_channels, double bytes_per_rank) {
  if (nranks <= 1) return m.base_us;
  const double bytes = model_bytes(kModelAllReduce, nranks, bytes_per_rank, kModelFlag);
  const double gbs = std::min(m.tree_max_gbs, m.tree_wg_gbs * 4.0 * nranks * tree_channels);
  return m.base_us + 2.0 * depth * m.tree_hop_us + bytes / (gbs * 1e3);
}

}  // namespace ringsim
