// ring_model.h -- protocol cost model of the ring collectives on one MI355X.
//
// Form of the model: "NCCL" book (aireadcode.com), ch. 5, ring.cc -- a ring
// collective's latency is nSteps hops of a per-hop latency, its bandwidth term
// is the bytes it moves over the achievable bandwidth (bus bandwidth times
// nRanks / nSteps), and the flag-packed (LL) protocol pays half the bandwidth
// because every 4 bytes of payload travel with a 4-byte flag. Here:
//
//   t(proto) = base + hops * hop_latency(proto) + bytes(proto) / bandwidth(proto)
//
// with hops = 2(N-1) for the all-reduce and N-1 for reduce-scatter and
// all-gather, bytes = the HBM bytes of the method (flag protocol: FIFO bytes
// doubled), and constants fitted to bench.py --sweep on MI355X (16 / 8 / 4
// ranks, 4..16 channels): a flag hop costs ~1.7 us and a bulk hop ~2.7 us
// when every chunk of the ring is busy; one flag-path workgroup sustains
// ~13 GB/s of method bytes, the bulk kernel ~6.9 TB/s in total.
#pragma once

#include <algorithm>
#include <cstddef>

namespace ringsim {

struct RingModel {
  double base_us = 3.0;
  double hop_us_flag = 1.7;
  double hop_us_bulk = 2.7;
  double flag_wg_gbs = 13.0;     // per (rank, channel) workgroup
  double flag_max_gbs = 4000.0;  // flag path ceiling
  double bulk_gbs = 6900.0;
};

enum ModelColl : int { kModelAllReduce = 0, kModelReduceScatter = 1, kModelAllGather = 2 };

// Method bytes of one call with S bytes per rank (all-reduce buffer,
// reduce-scatter input, all-gather output), summed over ranks.
inline double model_bytes(int coll, int nranks, double s, bool flag) {
  const double n = nranks;
  const double fifo = (coll == kModelAllReduce ? 4.0 * (n - 1.0) : 2.0 * (n - 1.0)) * s;
  const double user = coll == kModelAllReduce ? 2.0 * n * s : (n + 1.0) * s;
  return user + (flag ? 2.0 : 1.0) * fifo;
}

// Predicted microseconds of one call.
inline double model_us(const RingModel& m, int coll, int nranks, int nchannels, double bytes_per_rank, bool flag) {
  if (nranks <= 1) return m.base_us;
  const double hops = coll == kModelAllReduce ? 2.0 * (nranks - 1) : (double)(nranks - 1);
  const double bytes = model_bytes(coll, nranks, bytes_per_rank, flag);
  const double gbs = flag ? std::min(m.flag_max_gbs, m.flag_wg_gbs * nranks * nchannels) : m.bulk_gbs;
  return m.base_us + hops * (flag ? m.hop_us_flag : m.hop_us_bulk) + bytes / (gbs * 1e3);
}

// Predicted microseconds of a double-binary-tree all-reduce: the reduce
// climbs `depth` hops to each root and the broadcast descends as many, all
// in flag-packed lines; the flag protocol's bytes move through the 4 x N x
// tree_channels workgroups (two trees, an up and a down role each).
inline double tree_model_us(const RingModel& m, int nranks, int depth, int tree_channels, double bytes_per_rank) {
  if (nranks <= 1) return m.base_us;
  const double bytes = model_bytes(kModelAllReduce, nranks, bytes_per_rank, true);
  const double gbs = std::min(m.flag_max_gbs, m.flag_wg_gbs * 4.0 * nranks * tree_channels);
  return m.base_us + 2.0 * depth * m.hop_us_flag + bytes / (gbs * 1e3);
}

}  // namespace ringsim
