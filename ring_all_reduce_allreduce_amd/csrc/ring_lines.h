// ring_lines.h -- ring kernels over flag-packed FIFO lines ("NCCL" book,
// s. 2.4: LL and LL128 carry a flag inside the data, so the receiver polls
// the data itself; ch. 5: LL moves half a line of payload, LL128 120 of 128
// bytes). No tail counter and no fence sits on the data path: a line whose
// flag equals the step's flag carries that step's payload. The consumer's
// head counter is still published every few steps, for flow control only.
//
// The two line formats, FLAG and WIDE, are described in line_format.h.
//
// Lines carry a flag equal to the low 32 bits of (step + 1), taken from the
// monotonic step counters of the line protocols (the bulk protocol has
// counters of its own), so a line left over from an earlier step (of either
// format) never matches while a counter stays below 2^32 - 1: the host zeroes
// the line FIFOs and their counters before its calls could take a counter
// past that (kFlagSpanGuard). Both formats share one FIFO array per
// workgroup count.
//
// Workgroups per channel: a launch may split every unit over wpc = 1, 2, 4 or
// 8 workgroups per (rank, channel), each a pipeline of its own (own part of
// every unit, own counters, own 16 slots). Each wpc has its own FIFO array,
// so every FIFO byte is only ever written with flags of one pipeline's
// counters, which only grow: the no-match argument above holds whatever wpc
// earlier calls used.
//
// Steps are walked group by group (StepIter groups): a stage moves at most
// kLineGroupSteps slots before the next stage runs, which keeps one stage of
// a workgroup inside the FIFO part that is always free, so the chunk (and
// with it the partition and every result) is the same as the bulk
// protocol's.
#pragma once

#include "line_format.h"

namespace ringsim {

// Line modes: how the lines of a step map onto the 256 threads.
//   kLinesHalf  the host has checked that no step holds more than 128 lines:
//               consecutive steps alternate between the two halves of the
//               workgroup, one line per thread. A wave's loads and stores
//               share one counter (vmcnt), and a wave that reads a load's
//               result while its own stores are in flight waits for those
//               stores too; alternating halves lets one step's store
//               acknowledgements drain while the other half polls the next
//               step, which took ~20% off every hop on MI355X.
//   kLinesOne   at most 256 lines per step: every thread one line.
//   kLinesMulti any step (up to 4 lines per thread).
enum LineMode : int { kLinesMulti = 0, kLinesOne = 1, kLinesHalf = 2 };

template <int LP, int LM, int DT, int OP, int MODE>
__global__ void __launch_bounds__(kThreads) ring_line_kernel(RingArgs a) {
  using T = typename Elem<DT>::T;
  using F = LineFmt<LP, DT>;
  constexpr int64_t E = sizeof(T);
  constexpr int U = kFlagLinesPerThread;  // lines per thread in a full slot
  const Pipe p = locate(a);
  if (p.r == a.skip_rank) return;  // testing knob: a rank that never shows up
  __shared__ uint64_t s_base[2];
  __shared__ int s_credit;
  if (threadIdx.x == 0) {
    // Both loads in flight before either value is used.
    const uint64_t head = ld_relaxed(&p.in_ctr->head);
    const uint64_t tail = ld_relaxed(&p.out_ctr->tail);
    s_base[0] = head;
    s_base[1] = tail;
  }
  __syncthreads();
  const uint64_t in_base = uniform64(s_base[0]);
  const uint64_t out_base = uniform64(s_base[1]);
  const int nslots = a.nslots;
  // Per-call step counts and flags are 32-bit (a call moves far fewer than
  // 2^32 steps; flags are the low 32 bits of the 64-bit counters anyway), so
  // the per-step bookkeeping stays in scalar 32-bit arithmetic.
  uint32_t nrecv = 0, nsent = 0, nstep = 0;
  const uint32_t in_base32 = (uint32_t)in_base, out_base32 = (uint32_t)out_base;
  // Sends allowed before the consumer's head must be read again (uniform).
  // Both counters of a FIFO are equal when a call starts, so all slots are free.
  int credit = nslots;
  bool stop = false;  // per thread: stop waiting
  const WaitCtx wc = wait_ctx(a);
  uint32_t in_slot = (uint32_t)(in_base % (uint64_t)nslots);
  uint32_t out_slot = (uint32_t)(out_base % (uint64_t)nslots);

  const int64_t slice = (int64_t)(a.slot_bytes / 16) * F::PB / E;  // payload elements per slot
  StepIter<DT, MODE> it;
  it.init(a, p.r, p.c, p.w, slice, (int64_t)a.group * slice);
  for (; !it.done; it.next()) {
    const bool recv = it.recv, send = it.send;
    if (send && credit == 0) {  // uniform branch: wait until step nsent - nslots is drained
      if (threadIdx.x == 0) {
        const uint64_t need = out_base + nsent + 1 - (uint64_t)nslots;
        uint64_t h = need;
        if (!stop) {
          const uint64_t seen = wait_geq(&p.out_ctr->head, need, wc);
          stop = seen == 0;
          if (seen) h = seen;
        }
        s_credit = (int)(h + (uint64_t)nslots - (out_base + nsent));
      }
      __syncthreads();
      credit = uniform32(s_credit);
      __syncthreads();
    }
    const uint32_t flag_in = in_base32 + nrecv + 1;
    const uint32_t flag_out = out_base32 + nsent + 1;
    Slot<LP> fin, fout;
    fin.init(recv ? p.in_fifo + (int64_t)in_slot * a.slot_bytes : nullptr, a.slot_bytes);
    fout.init(send ? p.out_fifo + (int64_t)out_slot * a.slot_bytes : nullptr, a.slot_bytes);
    const int64_t nbytes = it.ns() * E;
    const int nlines = (int)div_up(nbytes, F::PB);  // <= kThreads * U
    const char* lp = it.use_local ? it.local() : nullptr;
    char* up = it.store ? it.out() : nullptr;
    const rsrc_t ur = make_rsrc(up, up ? nbytes : 0);
    if constexpr (LM != kLinesMulti) {
      // At most one line per thread (small messages): the shortest path from
      // a flag's arrival to the next hop's store.
      const int li = LM == kLinesHalf ? (int)threadIdx.x - (int)(nstep & 1u) * (kThreads / 2) : (int)threadIdx.x;
      if (li >= 0 && li < nlines && (LM != kLinesHalf || li < kThreads / 2)) {
        const int valid = (int)min64(F::PB, nbytes - (int64_t)li * F::PB);
        u32x4 loc = u32x4{0u, 0u, 0u, 0u};
        if (lp) loc = load_user<DT, F::PD>(lp + (int64_t)li * F::PB, valid, a.vec_ok);
        u32x4 x = loc;
        if (recv) {
          u32x4 v = fin.load(li);
          if (!stop && !Slot<LP>::ready(v, flag_in)) {
            const uint64_t t0 = wall_clock64();
            uint32_t spins = 0;
            while (!Slot<LP>::ready(v, flag_in)) {
              if (give_up(wc, t0, ++spins)) {
                stop = true;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
              compiler_fence();
              v = fin.load(li);
            }
          }
          x = Slot<LP>::payload(v);
          if (lp) x = reduce_payload<DT, OP, F::PD>(x, loc);
        }
        drain_loads();
        if (send) fout.store(li, x, flag_out);
        if (up) store_user<DT, F::PD>(up + (int64_t)li * F::PB, ur, li * F::PB, x, valid, a.vec_ok);
      }
    } else {
      // Several lines per thread: thread t owns lines t, t + 256, ...; all
      // of its own-operand loads and first polls are issued together, then
      // only lines whose flags have not arrived are polled again, every
      // round issuing all of its loads before it checks any of them (one
      // load latency per round, not per line).
      u32x4 x[U];
      u32x4 loc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int li = threadIdx.x + u * kThreads;
        loc[u] = u32x4{0u, 0u, 0u, 0u};
        if (lp && li < nlines)
          loc[u] = load_user<DT, F::PD>(lp + (int64_t)li * F::PB, (int)min64(F::PB, nbytes - (int64_t)li * F::PB),
                                        a.vec_ok);
      }
      if (recv) {
        u32x4 v[U];
        uint32_t pending = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          v[u] = u32x4{0u, 0u, 0u, 0u};
          if ((int)threadIdx.x + u * kThreads < nlines) v[u] = fin.load(threadIdx.x + u * kThreads);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if ((int)threadIdx.x + u * kThreads < nlines && !Slot<LP>::ready(v[u], flag_in)) pending |= 1u << u;
        if (pending && !stop) {
          const uint64_t t0 = wall_clock64();
          uint32_t spins = 0, verdict = 0;
          while (pending) {
            if ((verdict = wait_verdict(wc, t0, ++spins)) != 0u) break;
            __builtin_amdgcn_s_sleep(1);
            compiler_fence();
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
              if (pending & (1u << u)) w[u] = fin.load(threadIdx.x + u * kThreads);
#pragma unroll
            for (int u = 0; u < U; ++u) {
              if ((pending & (1u << u)) && Slot<LP>::ready(w[u], flag_in)) {
                v[u] = w[u];
                pending &= ~(1u << u);
              }
            }
          }
          if (verdict) {
            stop = true;
            if (verdict != kStopQuiet) raise_error(wc, verdict);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          x[u] = Slot<LP>::payload(v[u]);
          if (lp) x[u] = reduce_payload<DT, OP, F::PD>(x[u], loc[u]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = loc[u];
      }
      drain_loads();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int li = threadIdx.x + u * kThreads;
        if (li < nlines) {
          if (send) fout.store(li, x[u], flag_out);
          if (up)
            store_user<DT, F::PD>(up + (int64_t)li * F::PB, ur, li * F::PB, x[u],
                                  (int)min64(F::PB, nbytes - (int64_t)li * F::PB), a.vec_ok);
        }
      }
    }
    if (recv) {
      ++nrecv;
      in_slot = in_slot + 1 == (uint32_t)nslots ? 0 : in_slot + 1;
      if (nrecv % kFlagHeadEvery == 0) {  // uniform: release drained slots
        __syncthreads();
        if (threadIdx.x == 0) st_relaxed(&p.in_ctr->head, in_base + nrecv);
      }
    }
    ++nstep;
    if (send) {
      ++nsent;
      --credit;
      out_slot = out_slot + 1 == (uint32_t)nslots ? 0 : out_slot + 1;
    }
  }
  // Leave both counters at the number of steps this call moved, so the next
  // call (any protocol) starts from the same base on both sides.
  __syncthreads();
  if (threadIdx.x == 0) {
    st_relaxed(&p.in_ctr->head, in_base + nrecv);
    st_relaxed(&p.out_ctr->tail, out_base + nsent);
    // Past the flag span: only launches the host does not count (graph
    // replays) get here. Checked at the end, off every step's path (a check
    // at the start cost 0.5-9 us per call).
    if (in_base + nrecv > kFlagSpanGuard || out_base + nsent > kFlagSpanGuard) raise_error(wc, kErrFlagSpan);
  }
}

}  // namespace ringsim
