// ring_lines.h -- ring kernels over flag-packed FIFO lines ("NCCL" book,
// s. 2.4: LL and LL128 carry a flag inside the data, so the receiver polls
// the data itself; ch. 5: LL moves half a line of payload, LL128 120 of 128
// bytes). No tail counter and no fence sits on the data path: a line whose
// flag equals the step's flag carries that step's payload. The consumer's
// head counter is still published every few steps, for flow control only.
//
// Two line formats, both 16 bytes per lane:
//   FLAG  two 8-byte words {4-byte payload, 4-byte flag}, each written and
//         read as one 64-bit atomic access: 8 payload bytes per line.
//   WIDE  {12 bytes of payload, 4-byte flag}, written and read as one
//         128-bit device-coherent access: 12 payload bytes per line (8 for
//         int64, whose elements never straddle two lines). This is the
//         MI355X counterpart of LL128: NVLink delivers a warp's 128-byte
//         line whole, and here the unit that arrives whole is one lane's
//         naturally aligned 16-byte access, so the flag sits in every one.
//
// Lines carry a flag equal to the low 32 bits of (step + 1), taken from the
// same monotonic step counters as the bulk protocol, so a line left over from
// an earlier step (of either format) never matches: that would take 2^32
// steps on one FIFO. Both formats share one FIFO array per workgroup count.
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

#include "ringsim_device.h"

namespace ringsim {

namespace {

// FIFO line accesses of the WIDE format: device-coherent (SC1) 128-bit
// buffer accesses. Polling loops put a compiler fence before every re-read,
// so that a load is never hoisted out of its loop.
constexpr int kPolWideSt = 16;
constexpr int kPolWideLd = 16;

typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Waits until every load and store of the wave has completed (s_waitcnt
// vmcnt(0); expcnt and lgkmcnt left at their maxima). A step issues it once,
// where its operands are all in anyway, right before its stores: the
// compiler cannot tell on which paths the stored values are still in flight
// from their loads and otherwise waits for every earlier access before each
// store, so that each store also waits for the ones just issued, one memory
// round trip per line.
__device__ __forceinline__ void drain_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int LP, int DT>
struct LineFmt {
  // payload dwords per 16-byte line
  static constexpr int PD = LP == kLineFlag ? 2 : (DT == RINGSIM_INT64 ? 2 : 3);
  static constexpr int PB = 4 * PD;
};

// One FIFO slot seen as 16-byte lines.
template <int LP>
struct Slot {
  char* base;
  rsrc_t rs;

  __device__ __forceinline__ void init(const char* p, int bytes) {
    base = const_cast<char*>(p);
    if constexpr (LP == kLineWide) rs = make_rsrc(p, p ? bytes : 0);
  }

  // The raw 16 bytes of line li.
  __device__ __forceinline__ u32x4 load(int li) const {
    if constexpr (LP == kLineFlag) {
      const uint64_t* w = reinterpret_cast<const uint64_t*>(base) + 2 * li;
      const uint64_t v0 = ld_relaxed(w);
      const uint64_t v1 = ld_relaxed(w + 1);
      return u32x4{(uint32_t)v0, (uint32_t)(v0 >> 32), (uint32_t)v1, (uint32_t)(v1 >> 32)};
    } else {
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, li * 16, 0, kPolWideLd));
    }
  }

  static __device__ __forceinline__ bool ready(u32x4 v, uint32_t flag) {
    if constexpr (LP == kLineFlag) return v.y == flag && v.w == flag;
    else return v.w == flag;
  }

  static __device__ __forceinline__ u32x4 payload(u32x4 v) {
    if constexpr (LP == kLineFlag) return u32x4{v.x, v.z, 0u, 0u};
    else return u32x4{v.x, v.y, v.z, 0u};
  }

  __device__ __forceinline__ void store(int li, u32x4 x, uint32_t flag) const {
    if constexpr (LP == kLineFlag) {
      uint64_t* w = reinterpret_cast<uint64_t*>(base) + 2 * li;
      st_relaxed(w, ((uint64_t)flag << 32) | x.x);
      st_relaxed(w + 1, ((uint64_t)flag << 32) | x.y);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, flag}, rs, li * 16, 0, kPolWideSt);
    }
  }
};

// `valid` (<= PB) bytes of user data at p, as payload dwords; vector loads
// when the whole line is valid and buffers are 16-byte aligned (then p is
// 4-byte aligned), element loads otherwise.
template <int DT, int PD>
__device__ __forceinline__ u32x4 load_user(const char* p, int valid, int vec_ok) {
  using T = typename Elem<DT>::T;
  constexpr int PB = 4 * PD;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
  if (valid == PB && vec_ok) {
    if constexpr (PD == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      return u32x4{v.x, v.y, 0u, 0u};
    } else {
      return u32x4{w[0], w[1], w[2], 0u};
    }
  }
  union {
    u32x4 v;
    T e[16 / sizeof(T)];
  } u;
  u.v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < PB / (int)sizeof(T); ++q)
    if (q * (int)sizeof(T) < valid) u.e[q] = reinterpret_cast<const T*>(p)[q];
  return u.v;
}

// Stores `valid` bytes of a line's payload to user data at p = base + off;
// `ur` is a buffer resource over the step's output (whole 12-byte lines are
// stored with one 96-bit access through it).
template <int DT, int PD>
__device__ __forceinline__ void store_user(char* p, rsrc_t ur, int off, u32x4 x, int valid, int vec_ok) {
  using T = typename Elem<DT>::T;
  constexpr int PB = 4 * PD;
  if (valid == PB && vec_ok) {
    if constexpr (PD == 2) *reinterpret_cast<u32x2*>(p) = u32x2{x.x, x.y};
    else __builtin_amdgcn_raw_buffer_store_b96(u32x3{x.x, x.y, x.z}, ur, off, 0, 0);
    return;
  }
  union {
    u32x4 v;
    T e[16 / sizeof(T)];
  } u;
  u.v = x;
#pragma unroll
  for (int q = 0; q < PB / (int)sizeof(T); ++q)
    if (q * (int)sizeof(T) < valid) reinterpret_cast<T*>(p)[q] = u.e[q];
}

// op(a, b) on the payload dwords of one line.
template <int DT, int OP, int PD>
__device__ __forceinline__ u32x4 reduce_payload(u32x4 a, u32x4 b) {
  if constexpr (PD == 2) {
    const u32x2 z = VOp<DT, OP>::v2(u32x2{a.x, a.y}, u32x2{b.x, b.y});
    return u32x4{z.x, z.y, 0u, 0u};
  } else {
    static_assert(DT != RINGSIM_INT64, "int64 lines carry two payload dwords");
    return u32x4{VOp<DT, OP>::word(a.x, b.x), VOp<DT, OP>::word(a.y, b.y), VOp<DT, OP>::word(a.z, b.z), 0u};
  }
}

}  // namespace

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
    s_base[0] = ld_relaxed(&p.in_ctr->head);
    s_base[1] = ld_relaxed(&p.out_ctr->tail);
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
          if (threadIdx.x + u * kThreads < nlines) v[u] = fin.load(threadIdx.x + u * kThreads);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (threadIdx.x + u * kThreads < nlines && !Slot<LP>::ready(v[u], flag_in)) pending |= 1u << u;
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
  }
}

}  // namespace ringsim
