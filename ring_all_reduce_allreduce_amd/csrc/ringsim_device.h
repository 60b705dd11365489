// ringsim_device.h -- device-side building blocks shared by the ring, tree
// and copy kernels: element operators (one hop, rounded to the buffer type),
// bounded waits on step counters, the ring schedule iterator, pipeline
// addressing and flag-packed line helpers.
//
// Ring schedule ("NCCL" book, aireadcode.com, ch. 2, s. 2.2 channels, s. 2.3
// RingARAlgorithm, s. 2.4 protocols): workgroup (r, p) plays simulated rank r
// on pipeline p = (channel c, part w); at every stage it moves its part of the
// stage's chunk through the FIFO from rank r-1 into the FIFO to rank r+1,
// reducing with rank r's own data on the way. Every wait is bounded: a
// workgroup that waits longer than the timeout, or sees the abort word,
// records an error and stops waiting; the launch then runs to completion with
// undefined payload, and the host reports the error.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ring_plan.h"
#include "ringsim_internal.h"

namespace ringsim {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Element operators (one hop, rounded to the buffer type)
// ---------------------------------------------------------------------------

template <int OP>
__device__ __forceinline__ float op_f32(float a, float b) {
  if constexpr (OP == RINGSIM_SUM) {
    return a + b;
  } else if constexpr (OP == RINGSIM_PROD) {
    return a * b;
  } else if constexpr (OP == RINGSIM_MAX) {
    if (a > b) return a;
    if (b > a) return b;
    return __uint_as_float(__float_as_uint(a) & __float_as_uint(b));  // max(+0,-0) = +0
  } else {
    if (a < b) return a;
    if (b < a) return b;
    return __uint_as_float(__float_as_uint(a) | __float_as_uint(b));  // min(+0,-0) = -0
  }
}

template <int OP>
__device__ __forceinline__ uint32_t op_i32(uint32_t a, uint32_t b) {
  if constexpr (OP == RINGSIM_SUM) {
    return a + b;
  } else if constexpr (OP == RINGSIM_PROD) {
    return a * b;
  } else if constexpr (OP == RINGSIM_MAX) {
    return (int32_t)a > (int32_t)b ? a : b;
  } else {
    return (int32_t)a < (int32_t)b ? a : b;
  }
}

template <int OP>
__device__ __forceinline__ uint64_t op_i64(uint64_t a, uint64_t b) {
  if constexpr (OP == RINGSIM_SUM) {
    return a + b;
  } else if constexpr (OP == RINGSIM_PROD) {
    return a * b;
  } else if constexpr (OP == RINGSIM_MAX) {
    return (int64_t)a > (int64_t)b ? a : b;
  } else {
    return (int64_t)a < (int64_t)b ? a : b;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two float32 values -> packed bfloat16 pair, round to nearest even, with
// gfx950's conversion instruction (v_cvt_pk_bf16_f32: both halves at once).
__device__ __forceinline__ uint32_t to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ uint32_t to_bf16(float f) { return to_bf16x2(f, 0.0f) & 0xffffu; }

// Two bf16 values packed in a 32-bit word. Sum and product are computed in
// fp32 and rounded once; max and min pick one of the operands' halves (the
// result is exact), with -0 below +0.
template <int OP>
__device__ __forceinline__ uint32_t op_bf16x2(uint32_t a, uint32_t b) {
  if constexpr (OP == RINGSIM_SUM || OP == RINGSIM_PROD) {
    return to_bf16x2(op_f32<OP>(bf16_lo(a), bf16_lo(b)), op_f32<OP>(bf16_hi(a), bf16_hi(b)));
  } else {
    const uint32_t lo = __float_as_uint(op_f32<OP>(bf16_lo(a), bf16_lo(b))) >> 16;
    const uint32_t hi = __float_as_uint(op_f32<OP>(bf16_hi(a), bf16_hi(b))) & 0xffff0000u;
    return lo | hi;
  }
}

template <int DT>
struct Elem;
template <>
struct Elem<RINGSIM_INT32> { using T = uint32_t; };
template <>
struct Elem<RINGSIM_INT64> { using T = uint64_t; };
template <>
struct Elem<RINGSIM_FLOAT32> { using T = uint32_t; };
template <>
struct Elem<RINGSIM_BFLOAT16> { using T = uint16_t; };

// Reduction on 4-, 8- and 16-byte packets and on single elements.
template <int DT, int OP>
struct VOp {
  using T = typename Elem<DT>::T;

  static __device__ __forceinline__ uint32_t word(uint32_t a, uint32_t b) {
    if constexpr (DT == RINGSIM_FLOAT32) {
      return __float_as_uint(op_f32<OP>(__uint_as_float(a), __uint_as_float(b)));
    } else if constexpr (DT == RINGSIM_INT32) {
      return op_i32<OP>(a, b);
    } else {
      return op_bf16x2<OP>(a, b);
    }
  }

  static __device__ __forceinline__ u32x2 v2(u32x2 a, u32x2 b) {
    if constexpr (DT == RINGSIM_INT64) {
      const uint64_t x = ((uint64_t)a.y << 32) | a.x;
      const uint64_t y = ((uint64_t)b.y << 32) | b.x;
      const uint64_t z = op_i64<OP>(x, y);
      return u32x2{(uint32_t)z, (uint32_t)(z >> 32)};
    } else {
      return u32x2{word(a.x, b.x), word(a.y, b.y)};
    }
  }

  static __device__ __forceinline__ u32x4 v4(u32x4 a, u32x4 b) {
    const u32x2 lo = v2(u32x2{a.x, a.y}, u32x2{b.x, b.y});
    const u32x2 hi = v2(u32x2{a.z, a.w}, u32x2{b.z, b.w});
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  }

  static __device__ __forceinline__ T one(T a, T b) {
    if constexpr (DT == RINGSIM_INT64) {
      return op_i64<OP>(a, b);
    } else if constexpr (DT == RINGSIM_BFLOAT16) {
      return (T)(op_bf16x2<OP>(a, b) & 0xffffu);
    } else {
      return word(a, b);
    }
  }
};

// ---------------------------------------------------------------------------
// Synchronisation helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every global load and store this thread issued has completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A value that thread 0 broadcast through LDS is the same in every lane, but
// the compiler cannot know it: read through readfirstlane it lives in scalar
// registers, and so do the slot addresses and buffer resources derived from
// it. Otherwise every buffer access built on it runs in a loop over the
// distinct resource values of the wave (which happens to run once).
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int uniform32(int v) { return __builtin_amdgcn_readfirstlane(v); }

// What a waiting thread needs to give up cleanly; kept small so that it
// lives in registers rather than copying the kernel arguments.
struct WaitCtx {
  uint32_t* dev_abort;
  const uint32_t* host_abort;
  uint32_t* host_err;
  uint64_t timeout_ticks;
};

__device__ __forceinline__ WaitCtx wait_ctx(const RingArgs& a) {
  return WaitCtx{a.dev_abort, a.host_abort, a.host_err, a.timeout_ticks};
}

__device__ __forceinline__ bool host_abort_seen(const WaitCtx& w) {
  return __hip_atomic_load(w.host_abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u;
}

__device__ __forceinline__ bool dev_abort_seen(const WaitCtx& w) {
  return __hip_atomic_load(w.dev_abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Records the first error in the host-visible word and tells every other
// workgroup of the launch to stop waiting.
__device__ __forceinline__ void raise_error(WaitCtx w, uint32_t code) {
  atomicCAS_system(w.host_err, 0u, code);
  __hip_atomic_store(w.dev_abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called from spin loops with the spin count. Every 256 spins: the device
// abort word (another workgroup gave up; its error is already recorded) and
// the time bound. Every 16384 spins (about a millisecond of spinning): the
// host-mapped abort word -- reading host memory is a round trip over the
// host link, too slow and too contended to do on every miss.
__device__ __forceinline__ bool give_up(const WaitCtx& w, uint64_t t0, uint32_t it) {
  if (it & 255u) return false;
  if (dev_abort_seen(w)) return true;
  if ((it & 16383u) == 0u && host_abort_seen(w)) {
    raise_error(w, kErrAborted);
    return true;
  }
  if (wall_clock64() - t0 > w.timeout_ticks) {
    raise_error(w, kErrTimeout);
    return true;
  }
  return false;
}

// give_up() without memory side effects, for polling loops that must hold no
// store (so that their loads retire in issue order): 0 = keep waiting,
// kStopQuiet = stop (another workgroup already recorded an error), else the
// error code the caller records once it has left the loop.
constexpr uint32_t kStopQuiet = 0xffffffffu;
__device__ __forceinline__ uint32_t wait_verdict(const WaitCtx& w, uint64_t t0, uint32_t it) {
  if (it & 255u) return 0u;
  if (dev_abort_seen(w)) return kStopQuiet;
  if ((it & 16383u) == 0u && host_abort_seen(w)) return kErrAborted;
  if (wall_clock64() - t0 > w.timeout_ticks) return kErrTimeout;
  return 0u;
}

// Spins until *p >= target and returns the value seen, or returns 0 (never a
// valid answer: targets start at 1) after recording why it gave up.
__device__ __forceinline__ uint64_t wait_geq(const uint64_t* p, uint64_t target, WaitCtx w) {
  uint64_t v = ld_relaxed(p);
  if (v >= target) return v;
  const uint64_t t0 = wall_clock64();
  uint32_t it = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    v = ld_relaxed(p);
    if (v >= target) return v;
    if (give_up(w, t0, ++it)) return 0;
  }
}


struct Pipe {
  int r, c, w, pipe;
  int nxt;  // the next rank on the ring
  FifoCtr* in_ctr;
  FifoCtr* out_ctr;
  char* in_fifo;
  char* out_fifo;
};

__device__ __forceinline__ Pipe locate(const RingArgs& a) {
  Pipe p;
  const int P = a.nchannels * a.wpc;
  const int b = blockIdx.x;
  p.r = b / P;
  const int pl = b - p.r * P;
  p.c = pl / a.wpc;
  p.w = pl - p.c * a.wpc;
  p.pipe = p.c * a.pipe_mul + p.w;
  const int nxt = p.r + 1 == a.nranks ? 0 : p.r + 1;
  p.nxt = nxt;
  p.in_ctr = a.ctr + (int64_t)p.r * a.pipe_stride + p.pipe;
  p.out_ctr = a.ctr + (int64_t)nxt * a.pipe_stride + p.pipe;
  const int fpipe = p.c * a.fifo_mul + p.w;
  const int64_t fifo_bytes = (int64_t)a.nslots * a.slot_bytes;
  p.in_fifo = a.fifo + ((int64_t)p.r * a.fifo_stride + fpipe) * fifo_bytes;
  p.out_fifo = a.fifo + ((int64_t)nxt * a.fifo_stride + fpipe) * fifo_bytes;
  return p;
}


// ---------------------------------------------------------------------------
// Ring schedule
// ---------------------------------------------------------------------------

// Schedule iterator: walks the ring schedule of one workgroup one FIFO slot
// step at a time ("NCCL" book s. 2.3: a loop covers N chunks, stage j of rank
// r visits chunk (r + N - 1 - j) mod N; all-gather round j moves block r - j,
// "NCCL 专家课程 17", Bootstrap Ring 与 AllGather). Divisions happen once per
// loop (or for a ragged tail chunk), never per stage: the chunk / block index
// steps down by one each stage. Empty units produce no step.
//
// Groups: with group_elems > 0 a loop is walked group by group -- every
// stage moves only elements [g, g + group_elems) of its unit, then the
// stages are walked again for the next group, like a loop whose chunk is
// one group long. Sender and receiver of a FIFO still agree on the order of
// every step (stage j + 1 of rank r + 1 consumes exactly what stage j of
// rank r produced, group by group), and a step still reduces the same
// elements in the same rank order, so values do not change; but a stage puts
// at most one group into the FIFO, whatever the chunk size.
// Parts: with wpc workgroups per channel, workgroup w moves part w of every
// unit (alignUp(ceil(n / wpc), A) elements, clamped to the unit). The part
// bounds of a whole chunk and of the loop's ragged chunk are computed once per
// loop, so a stage costs no division.
template <int DT, int MODE>
struct StepIter {
  static constexpr int64_t E = sizeof(typename Elem<DT>::T);
  static constexpr int64_t A = 16 / E;
  // fixed per workgroup
  const char* send_r;
  char* recv_r;
  int64_t count, chunk, L, ch_lo;
  int slice;  // elements per step (a slot's payload)
  int N, r, w, wpc;
  // loop, group and stage
  int64_t off, rem, cur, part_lo, part_n;
  int glen, g_lo, umax;  // group length, start of the current group, longest unit of the loop
  // all-reduce: chunks [0, kfull) of the loop are whole, chunk kfull is the
  // ragged one (possibly empty), later ones are empty; this workgroup's part
  // of a whole chunk is [full_lo, full_lo + full_n), of the ragged one
  // [tail_lo, tail_lo + tail_n)
  int kfull, full_lo, full_n, tail_lo, tail_n;
  int j, idx;
  // current unit and step
  int64_t local_e, out_e;
  // unit length, current step inside it, end of its steps in this group;
  // 32-bit (a unit is at most one chunk, < 2^30 elements) to keep the
  // per-step bookkeeping in scalar 32-bit arithmetic
  int m, s, s_end;
  bool recv, use_local, send, store, done;

  __device__ __forceinline__ int nstages() const { return MODE == kAllReduce ? 2 * N - 1 : N; }

  __device__ __forceinline__ void begin_group() {
    j = 0;
    idx = MODE == kAllGather ? r : (r == 0 ? N - 1 : r - 1);
  }

  __device__ __forceinline__ void begin_loop() {
    rem = L - off;
    if constexpr (MODE == kAllReduce) {
      cur = ar_loop_chunk(rem, N, chunk, A);
      kfull = rem >= (int64_t)N * cur ? N : (int)(rem / cur);
      const int64_t tail = kfull < N ? rem - (int64_t)kfull * cur : 0;
      if (wpc == 1) {
        full_lo = tail_lo = 0;
        full_n = (int)cur;
        tail_n = (int)tail;
      } else {
        const Range pf = split_part(cur, wpc, w, A);
        const Range pt = split_part(tail, wpc, w, A);
        full_lo = (int)pf.lo;
        full_n = (int)(pf.hi - pf.lo);
        tail_lo = (int)pt.lo;
        tail_n = (int)(pt.hi - pt.lo);
      }
      umax = full_n;
    } else {
      cur = min64(chunk, rem);
      if (wpc == 1) {
        part_lo = 0;
        part_n = cur;
      } else {
        const Range pt = split_part(cur, wpc, w, A);
        part_lo = pt.lo;
        part_n = pt.hi - pt.lo;
      }
      umax = (int)part_n;
    }
    g_lo = 0;
    begin_group();
  }

  // The unit of the current stage, and its steps inside the current group.
  __device__ __forceinline__ void set_unit() {
    set_unit_range();
    s = g_lo;
    s_end = m - g_lo < glen ? m : g_lo + glen;
  }

  __device__ __forceinline__ void set_unit_range() {
    if constexpr (MODE == kAllReduce) {
      const bool whole = idx < kfull;
      m = whole ? full_n : (idx == kfull ? tail_n : 0);
      local_e = out_e = ch_lo + off + (int64_t)idx * cur + (whole ? full_lo : tail_lo);
      recv = j >= 1;
      use_local = j <= N - 1;
      send = j <= 2 * N - 3;
      store = j >= N - 1;
    } else if constexpr (MODE == kReduceScatter) {
      m = (int)part_n;
      out_e = ch_lo + off + part_lo;
      local_e = (int64_t)idx * count + out_e;
      recv = j >= 1;
      use_local = true;
      send = j <= N - 2;
      store = j == N - 1;
    } else {
      m = (int)part_n;
      local_e = ch_lo + off + part_lo;
      out_e = (int64_t)idx * count + local_e;
      recv = j >= 1;
      use_local = j == 0;
      send = j <= N - 2;
      store = true;
    }
  }

  // Moves to the next stage (then group, then loop) until a unit with a step
  // in the current group, or the end.
  __device__ __forceinline__ void next_unit() {
    do {
      ++j;
      idx = idx == 0 ? N - 1 : idx - 1;
      if (j == nstages()) {
        if (umax - g_lo > glen) {
          g_lo += glen;
          begin_group();
        } else {
          off += MODE == kAllReduce ? (int64_t)N * chunk : chunk;
          if (off >= L) {
            done = true;
            return;
          }
          begin_loop();
        }
      }
      set_unit();
    } while (s >= s_end);
  }

  // slice_elems: elements per FIFO slot step; group_elems: elements of a
  // unit that one stage moves before the next stage runs (0: the whole unit).
  __device__ __forceinline__ void init(const RingArgs& a, int rank, int c, int part, int64_t slice_elems,
                                       int64_t group_elems = 0) {
    N = a.nranks;
    r = rank;
    w = part;
    wpc = a.wpc;
    count = a.count;
    chunk = a.chunk;
    slice = (int)slice_elems;
    glen = group_elems > 0 ? (int)group_elems : 0x7fffffff;
    send_r = a.send[r];
    recv_r = a.recv[r];
    const Range ch = channel_range(a.count, a.nchannels, c, A);
    ch_lo = ch.lo;
    L = ch.hi - ch.lo;
    off = 0;
    done = L <= 0;
    if (done) return;
    begin_loop();
    set_unit();
    if (s >= s_end) next_unit();
  }

  __device__ __forceinline__ void next() {
    s += slice;
    if (s < s_end) return;
    next_unit();
  }

  __device__ __forceinline__ int64_t ns() const { return slice < s_end - s ? slice : s_end - s; }
  __device__ __forceinline__ const char* local() const { return send_r + (local_e + s) * E; }
  __device__ __forceinline__ char* out() const { return recv_r + (out_e + s) * E; }
};

// ---------------------------------------------------------------------------
// Flag-packed lines (8-byte words of {4-byte payload, 4-byte flag})
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ u32x2 load_payload(const char* p, int valid, int vec_ok) {
  using T = typename Elem<DT>::T;
  if (valid == 8 && vec_ok) return *reinterpret_cast<const u32x2*>(p);
  union {
    u32x2 v;
    T e[8 / sizeof(T)];
  } u;
  u.v = u32x2{0u, 0u};
#pragma unroll
  for (int q = 0; q < (int)(8 / sizeof(T)); ++q)
    if (q * (int)sizeof(T) < valid) u.e[q] = reinterpret_cast<const T*>(p)[q];
  return u.v;
}

template <int DT>
__device__ __forceinline__ void store_payload(char* p, u32x2 x, int valid, int vec_ok) {
  using T = typename Elem<DT>::T;
  if (valid == 8 && vec_ok) {
    *reinterpret_cast<u32x2*>(p) = x;
    return;
  }
  union {
    u32x2 v;
    T e[8 / sizeof(T)];
  } u;
  u.v = x;
#pragma unroll
  for (int q = 0; q < (int)(8 / sizeof(T)); ++q)
    if (q * (int)sizeof(T) < valid) reinterpret_cast<T*>(p)[q] = u.e[q];
}

__device__ __forceinline__ WaitCtx wait_ctx(const TreeArgs& a) {
  return WaitCtx{a.dev_abort, a.host_abort, a.host_err, a.timeout_ticks};
}


// ---------------------------------------------------------------------------
// Buffer resources and launch helpers
// ---------------------------------------------------------------------------

// A raw buffer resource over [p, p + bytes): accesses outside it are dropped
// (stores) or read as zero (loads) by the hardware.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit raw data, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// The same for a p and bytes that are equal in every lane of the wave but
// that the compiler cannot prove so: they are read from the first lane, so
// that the resource lives in scalar registers (a resource in vector registers
// makes the compiler wrap every access in a loop over its distinct values).
__device__ __forceinline__ rsrc_t make_uniform_rsrc(const void* p, int64_t bytes) {
  void* u = reinterpret_cast<void*>(uniform64(reinterpret_cast<uint64_t>(p)));
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, uniform32((int)bytes), kRsrcWord3);
}

// Instantiates L::run<DT, OP, MODE> for the runtime mode, dtype and op (the
// all-gather moves bytes only, so it has one instantiation per dtype).
template <typename L>
hipError_t dispatch_ring(const RingArgs& a, int mode, int dtype, int op, hipStream_t s) {
  auto by_op = [&](auto dt, auto md) -> hipError_t {
    constexpr int DT = decltype(dt)::value;
    constexpr int MODE = decltype(md)::value;
    if constexpr (MODE == kAllGather) {
      return L::template run<DT, RINGSIM_SUM, MODE>(a, s);
    } else {
      switch (op) {
        case RINGSIM_SUM: return L::template run<DT, RINGSIM_SUM, MODE>(a, s);
        case RINGSIM_PROD: return L::template run<DT, RINGSIM_PROD, MODE>(a, s);
        case RINGSIM_MAX: return L::template run<DT, RINGSIM_MAX, MODE>(a, s);
        case RINGSIM_MIN: return L::template run<DT, RINGSIM_MIN, MODE>(a, s);
        default: return hipErrorInvalidValue;
      }
    }
  };
  auto by_dtype = [&](auto md) -> hipError_t {
    switch (dtype) {
      case RINGSIM_INT32: return by_op(std::integral_constant<int, RINGSIM_INT32>{}, md);
      case RINGSIM_INT64: return by_op(std::integral_constant<int, RINGSIM_INT64>{}, md);
      case RINGSIM_FLOAT32: return by_op(std::integral_constant<int, RINGSIM_FLOAT32>{}, md);
      case RINGSIM_BFLOAT16: return by_op(std::integral_constant<int, RINGSIM_BFLOAT16>{}, md);
      default: return hipErrorInvalidValue;
    }
  };
  switch (mode) {
    case kAllReduce: return by_dtype(std::integral_constant<int, kAllReduce>{});
    case kReduceScatter: return by_dtype(std::integral_constant<int, kReduceScatter>{});
    case kAllGather: return by_dtype(std::integral_constant<int, kAllGather>{});
    default: return hipErrorInvalidValue;
  }
}

// Resident workgroups of `kernel` per CU with `lds` bytes of dynamic LDS.
template <typename K>
int occupancy(K kernel, size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, lds) != hipSuccess) return 0;
  return n;
}

}  // namespace ringsim
