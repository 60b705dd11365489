// tree_lines.h -- double-binary-tree all-reduce over flag-packed lines
// ("NCCL" book, ch. 4: two binary trees, each reducing one half of the
// buffer up to its root and broadcasting it back down). Every FIFO step is
// one WIDE line per thread (line_format.h: 12 payload bytes and the flag in
// one 128-bit device-coherent access, 8 payload bytes for int64).
#pragma once

#include "line_format.h"
#include "tree_plan.h"

namespace ringsim {

// One slice of at most one line per thread: every line is the fold of the
// own operand (if any) and the input lines in child order (own first, then
// first child, then second child), stored to each output FIFO under that
// FIFO's flag and to the receive buffer. fin[j] / fout[j] (j < nin / nout)
// are this step's slots. Arrays are only ever indexed with unrolled
// constants.
template <int DT, int OP>
__device__ __forceinline__ void tree_lines(int nlines, int64_t nbytes, const char* lp, char* op, int nin,
                                           const Slot<kLineWide> (&fin)[2], const uint32_t (&flag_in)[2],
                                           int nout, const Slot<kLineWide> (&fout)[2],
                                           const uint32_t (&flag_out)[2], int vec_ok, bool& stop,
                                           const WaitCtx& wc) {
  using F = LineFmt<kLineWide, DT>;
  // One line per thread: the shortest path from a flag's arrival to the
  // next hop's store.
  const int li = threadIdx.x;
  if (li >= nlines) return;
  const int valid = (int)min64(F::PB, nbytes - (int64_t)li * F::PB);
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  if (lp) x = load_user<DT, F::PD>(lp + (int64_t)li * F::PB, valid, vec_ok);
  // Both children's lines are polled together: loads of both go out
  // before either is checked, and a round re-reads only what is missing.
  u32x4 v[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < nin) v[j] = fin[j].load(li);
  uint32_t pending = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < nin && !Slot<kLineWide>::ready(v[j], flag_in[j])) pending |= 1u << j;
  if (pending && !stop) {
    const uint64_t t0 = wall_clock64();
    uint32_t spins = 0, verdict = 0;
    while (pending) {
      if ((verdict = wait_verdict(wc, t0, ++spins)) != 0u) break;
      __builtin_amdgcn_s_sleep(1);
      compiler_fence();
      u32x4 w[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (pending & (1u << j)) w[j] = fin[j].load(li);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if ((pending & (1u << j)) && Slot<kLineWide>::ready(w[j], flag_in[j])) {
          v[j] = w[j];
          pending &= ~(1u << j);
        }
      }
    }
    if (verdict) {
      stop = true;
      if (verdict != kStopQuiet) raise_error(wc, verdict);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (j < nin) {
      const u32x4 y = Slot<kLineWide>::payload(v[j]);
      x = (lp || j > 0) ? reduce_payload<DT, OP, F::PD>(x, y) : y;
    }
  }
  drain_loads();
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < nout) fout[j].store(li, x, flag_out[j]);
  if (op) store_user<DT, F::PD>(op + (int64_t)li * F::PB, make_rsrc(op, nbytes), li * F::PB, x, valid, vec_ok);
}

// One workgroup per (rank, tree, channel, role). Role 0 folds the rank's own
// slice with its children's partials and passes the result to the parent;
// at the root the result is final: it is stored and sent down to the
// children. Role 1 receives the result from the parent, stores it and passes
// it on to the children. Every FIFO carries one step per slice of the
// channel; its producer owns `tail`, its consumer `head`, and a line's flag
// is the low 32 bits of (step + 1).
template <int DT, int OP>
__global__ void __launch_bounds__(kThreads) tree_line_kernel(TreeArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int64_t E = sizeof(T);
  constexpr int64_t A = 16 / E;
  const int b = blockIdx.x;
  const int role = b & 1;
  const int c = (b >> 1) % a.nchannels;
  const int t = ((b >> 1) / a.nchannels) & 1;
  const int v = ((b >> 1) / a.nchannels) >> 1;
  if (v == a.skip_rank) return;  // testing knob: a rank that never shows up
  const bool root = a.link[t][v][0] < 0;
  if (role == 1 && root) return;  // the root's up pass starts the broadcast
  const Range cr = tree_channel_range(a.count, t, c, a.nchannels, A);
  if (cr.hi <= cr.lo) return;
  using F = LineFmt<kLineWide, DT>;
  const int64_t slice = (int64_t)kThreads * F::PB / E;  // one line per thread
  const int64_t nsl = div_up(cr.hi - cr.lo, slice);

  // FIFOs on each side, in child-slot order; unused entries stay null.
  auto fifo_of = [&](int node, int dir) -> int64_t {
    return (((int64_t)t * a.ch_stride + c) * a.nranks + node) * 2 + dir;
  };
  const int k0 = a.link[t][v][1], k1 = a.link[t][v][2];
  const int kA = k0 >= 0 ? k0 : k1;  // first present child
  const int kB = k0 >= 0 ? k1 : -1;  // second present child
  const int nkids = (kA >= 0) + (kB >= 0);
  int64_t in_f[2] = {-1, -1}, out_f[2] = {-1, -1};
  int nin, nout;
  if (role == 0) {
    nin = nkids;
    in_f[0] = kA >= 0 ? fifo_of(kA, 0) : -1;
    in_f[1] = kB >= 0 ? fifo_of(kB, 0) : -1;
    if (root) {
      nout = nkids;
      out_f[0] = kA >= 0 ? fifo_of(kA, 1) : -1;
      out_f[1] = kB >= 0 ? fifo_of(kB, 1) : -1;
    } else {
      nout = 1;
      out_f[0] = fifo_of(v, 0);
    }
  } else {
    nin = 1;
    in_f[0] = fifo_of(v, 1);
    nout = nkids;
    out_f[0] = kA >= 0 ? fifo_of(kA, 1) : -1;
    out_f[1] = kB >= 0 ? fifo_of(kB, 1) : -1;
  }
  const int64_t fifo_bytes = (int64_t)a.nslots * a.slot_bytes;
  const char* in_fifo[2];
  const char* out_fifo[2];
  FifoCtr* in_ctr[2];
  FifoCtr* out_ctr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    in_fifo[j] = in_f[j] >= 0 ? a.fifo + in_f[j] * fifo_bytes : nullptr;
    out_fifo[j] = out_f[j] >= 0 ? a.fifo + out_f[j] * fifo_bytes : nullptr;
    in_ctr[j] = in_f[j] >= 0 ? a.ctr + in_f[j] : nullptr;
    out_ctr[j] = out_f[j] >= 0 ? a.ctr + out_f[j] : nullptr;
  }
  const char* own = role == 0 ? a.send[v] + cr.lo * E : nullptr;
  char* dst = (role == 1 || root) ? a.recv[v] + cr.lo * E : nullptr;

  __shared__ uint64_t s_base[4];
  __shared__ uint64_t s_head[2];
  if (threadIdx.x == 0) {
    // All four loads in flight before any value is used.
    uint64_t b[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      b[j] = j < nin ? ld_relaxed(&in_ctr[j]->head) : 0;
      b[2 + j] = j < nout ? ld_relaxed(&out_ctr[j]->tail) : 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s_base[j] = b[j];
  }
  __syncthreads();
  const uint64_t in_base[2] = {uniform64(s_base[0]), uniform64(s_base[1])};
  const uint64_t out_base[2] = {uniform64(s_base[2]), uniform64(s_base[3])};
  uint64_t head_known[2] = {out_base[0], out_base[1]};  // uniform
  uint64_t known_head[2] = {0, 0};                      // thread 0
  uint32_t in_slot[2], out_slot[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    in_slot[j] = (uint32_t)(in_base[j] % (uint64_t)a.nslots);
    out_slot[j] = (uint32_t)(out_base[j] % (uint64_t)a.nslots);
  }
  bool stop = false;
  const WaitCtx wc = wait_ctx(a);
  const uint64_t nslots = (uint64_t)a.nslots;

  for (int64_t s = 0; s < nsl; ++s) {
    // Space in every output FIFO: its consumer has drained step s - nslots.
    if ((uint64_t)s + 1 > nslots) {
      bool need_any = false;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j < nout) need_any |= head_known[j] < out_base[j] + s + 1 - nslots;
      if (need_any) {  // uniform branch
        if (threadIdx.x == 0) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (j < nout) {
              const uint64_t need = out_base[j] + s + 1 - nslots;
              if (!stop && known_head[j] < need) {
                known_head[j] = wait_geq(&out_ctr[j]->head, need, wc);
                stop = known_head[j] == 0;
              }
              s_head[j] = known_head[j] > need ? known_head[j] : need;
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (j < nout) head_known[j] = uniform64(s_head[j]);
        __syncthreads();
      }
    }
    const int64_t n = min64(slice, cr.hi - cr.lo - s * slice);
    const int64_t nbytes = n * E;
    const int nlines = (int)div_up(nbytes, (int64_t)F::PB);
    Slot<kLineWide> fin[2], fout[2];
    uint32_t flag_in[2], flag_out[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fin[j].init(j < nin ? in_fifo[j] + (int64_t)in_slot[j] * a.slot_bytes : nullptr, a.slot_bytes);
      fout[j].init(j < nout ? out_fifo[j] + (int64_t)out_slot[j] * a.slot_bytes : nullptr, a.slot_bytes);
      flag_in[j] = (uint32_t)(in_base[j] + s + 1);
      flag_out[j] = (uint32_t)(out_base[j] + s + 1);
    }
    tree_lines<DT, OP>(nlines, nbytes, own ? own + s * slice * E : nullptr, dst ? dst + s * slice * E : nullptr,
                       nin, fin, flag_in, nout, fout, flag_out, a.vec_ok, stop, wc);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      in_slot[j] = in_slot[j] + 1 == (uint32_t)a.nslots ? 0 : in_slot[j] + 1;
      out_slot[j] = out_slot[j] + 1 == (uint32_t)a.nslots ? 0 : out_slot[j] + 1;
    }
    if ((s + 1) % a.head_every == 0) {  // uniform: release drained slots
      __syncthreads();
      if (threadIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (j < nin) st_relaxed(&in_ctr[j]->head, in_base[j] + s + 1);
      }
    }
  }
  // Leave every counter at the steps this call moved, so the next call
  // starts from the same base on both sides of each FIFO.
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < nin) st_relaxed(&in_ctr[j]->head, in_base[j] + nsl);
      if (j < nout) st_relaxed(&out_ctr[j]->tail, out_base[j] + nsl);
    }
    // Past the flag span (graph replays only), checked off the step path.
    if ((nin > 0 && in_base[0] + nsl > kFlagSpanGuard) || (nout > 0 && out_base[0] + nsl > kFlagSpanGuard) ||
        (nin > 1 && in_base[1] + nsl > kFlagSpanGuard) || (nout > 1 && out_base[1] + nsl > kFlagSpanGuard))
      raise_error(wc, kErrFlagSpan);
  }
}

}  // namespace ringsim
