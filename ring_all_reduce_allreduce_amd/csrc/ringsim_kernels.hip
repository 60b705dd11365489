// ringsim_kernels.hip -- ring collective kernels for CDNA4 (gfx950).
//
// One launch runs a whole collective. Workgroup (r, p) plays simulated rank r
// on pipeline p = (channel c, part w): it walks the ring schedule of its
// channel and, at every stage, moves its part of the stage's chunk through the
// FIFO from rank r-1 into the FIFO to rank r+1, reducing with rank r's own
// data on the way ("NCCL" book, aireadcode.com, ch. 2, s. 2.2 channels,
// s. 2.3 RingARAlgorithm, s. 2.4 protocols). The workgroups of one pipeline
// form a ring of producer/consumer pairs; workgroup ids are rank-major so
// that, when the pipeline count is a multiple of 8, every workgroup of a
// pipeline is dispatched to the same XCD and its FIFO traffic stays behind
// one L2.
//
// Two protocols:
//   bulk  FIFO slots hold raw payload; readiness travels in separate 64-bit
//         step counters (tail: slots filled, head: slots drained). Slot data
//         is written and read with device-scope coherent (SC1) accesses, so a
//         counter published once those accesses have completed is enough to
//         order them; no L2 writeback or invalidate is needed (Simple).
//   flag  FIFO lines of 16 bytes carry two {4-byte payload, 4-byte flag}
//         words; each 8-byte word is written and read as one 64-bit access,
//         so a receiver that sees the expected flag also sees its payload.
//         No fences on the data path; head is published every few steps for
//         flow control only (LL).
// Every wait is bounded: a workgroup that waits longer than the timeout, or
// sees the abort word, records an error and stops waiting; the launch then
// runs to completion with undefined payload, and the host reports the error.
#include <hip/hip_runtime.h>

#include "ring_plan.h"
#include "tree_plan.h"
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

// ---------------------------------------------------------------------------
// Bulk data movement: one FIFO slot worth of a unit
// ---------------------------------------------------------------------------

// FIFO slots are accessed through buffer resources (bounds-checked against the
// slot size) with device-scope coherence (SC1): a store is visible to every
// XCD once it completes and a load never returns a stale line, so a step
// counter published after the stores complete is all the consumer needs - no
// L2 writeback or invalidate on the data path. User buffers use plain global
// accesses marked non-temporal (each byte is touched once per launch).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit raw data, no swizzle
constexpr int kPolFifo = 16;            // SC1: device scope
constexpr int kPolFifoStream = 16 | 2;  // SC1 + NT: device scope, no reuse expected

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

template <typename T>
__device__ __forceinline__ T fifo_ld(rsrc_t r, int off) {
  if constexpr (sizeof(T) == 2) return (T)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kPolFifoStream);
  else if constexpr (sizeof(T) == 4) return (T)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kPolFifoStream);
  else return (T)__builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolFifoStream));
}

template <typename T>
__device__ __forceinline__ void fifo_st(T v, rsrc_t r, int off) {
  if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, kPolFifo);
  else if constexpr (sizeof(T) == 4) __builtin_amdgcn_raw_buffer_store_b32((unsigned int)v, r, off, 0, kPolFifo);
  else __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, (uint64_t)v), r, off, 0, kPolFifo);
}

__device__ __forceinline__ u32x4 fifo_ld4(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolFifoStream));
}
__device__ __forceinline__ void fifo_st4(u32x4 v, rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolFifo);
}

// Whole 16-byte vectors: x = src (FIFO when SRC_FIFO, else user data loc),
// x = op(x, loc) when RED, then x -> FIFO fout and/or user uout. Full tiles run
// unguarded so that every load of a tile is in flight before the first use.
template <int DT, int OP, bool SRC_FIFO, bool RED, bool FOUT, bool UOUT, bool LOC_LDS = false>
__device__ __forceinline__ void move_vec(int64_t nv, rsrc_t fin, const u32x4* __restrict__ loc, rsrc_t fout,
                                         u32x4* __restrict__ uout) {
  const int tid = threadIdx.x;
  constexpr int kTile = kThreads * kUnroll;
  // The rank's own operand: staged in LDS by the previous step, or streamed
  // from HBM (read once: non-temporal).
  auto load_loc = [&](int i) -> u32x4 {
    if constexpr (LOC_LDS) return loc[i];
    else return __builtin_nontemporal_load(loc + i);
  };
  auto load_src = [&](int i) -> u32x4 {
    if constexpr (SRC_FIFO) return fifo_ld4(fin, i * 16);
    else return load_loc(i);
  };
  auto store = [&](int i, u32x4 v) {
    if constexpr (FOUT) fifo_st4(v, fout, i * 16);
    if constexpr (UOUT) __builtin_nontemporal_store(v, uout + i);
  };
  int base = 0;
  const int n = (int)nv;
  for (; base + kTile <= n; base += kTile) {
    u32x4 v[kUnroll];
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_src(base + u * kThreads + tid);
    if constexpr (RED) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) x[u] = load_loc(base + u * kThreads + tid);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = VOp<DT, OP>::v4(v[u], x[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) store(base + u * kThreads + tid, v[u]);
  }
  for (int i = base + tid; i < n; i += kThreads) {
    u32x4 v = load_src(i);
    if constexpr (RED) v = VOp<DT, OP>::v4(v, load_loc(i));
    store(i, v);
  }
}

// One FIFO slot worth of a unit (n elements): x = fin ? (loc ? op(fin, loc)
// : fin) : loc, then x -> fout and/or uout. fin/fout are FIFO slots of
// slot_bytes; loc/uout are user data, vector-moved only when vec_ok.
// `staged` (LDS, may be null) holds the whole-vector part of `loc`, loaded by
// the previous step; the rest of `loc` is read from memory.
template <int DT, int OP>
__device__ __forceinline__ void move_slice(int64_t n, const char* fin, const char* loc, char* fout, char* uout,
                                           int slot_bytes, int vec_ok, const u32x4* staged = nullptr) {
  using T = typename Elem<DT>::T;
  constexpr int A = 16 / (int)sizeof(T);
  const int64_t nv = vec_ok ? n / A : 0;
  const rsrc_t rin = make_rsrc(fin, fin ? slot_bytes : 0);
  const rsrc_t rout = make_rsrc(fout, fout ? slot_bytes : 0);
  const u32x4* l4 = reinterpret_cast<const u32x4*>(loc);
  u32x4* u4 = reinterpret_cast<u32x4*>(uout);
  if (nv > 0 && staged && loc) {
    if (fin) {
      if (fout && uout) move_vec<DT, OP, true, true, true, true, true>(nv, rin, staged, rout, u4);
      else if (fout) move_vec<DT, OP, true, true, true, false, true>(nv, rin, staged, rout, u4);
      else move_vec<DT, OP, true, true, false, true, true>(nv, rin, staged, rout, u4);
    } else {
      if (fout && uout) move_vec<DT, OP, false, false, true, true, true>(nv, rin, staged, rout, u4);
      else move_vec<DT, OP, false, false, true, false, true>(nv, rin, staged, rout, u4);
    }
  } else if (nv > 0) {
    if (fin && loc) {
      if (fout && uout) move_vec<DT, OP, true, true, true, true>(nv, rin, l4, rout, u4);
      else if (fout) move_vec<DT, OP, true, true, true, false>(nv, rin, l4, rout, u4);
      else move_vec<DT, OP, true, true, false, true>(nv, rin, l4, rout, u4);
    } else if (fin) {
      if (fout && uout) move_vec<DT, OP, true, false, true, true>(nv, rin, l4, rout, u4);
      else if (fout) move_vec<DT, OP, true, false, true, false>(nv, rin, l4, rout, u4);
      else move_vec<DT, OP, true, false, false, true>(nv, rin, l4, rout, u4);
    } else {
      if (fout && uout) move_vec<DT, OP, false, false, true, true>(nv, rin, l4, rout, u4);
      else move_vec<DT, OP, false, false, true, false>(nv, rin, l4, rout, u4);
    }
  }
  // Elements past the last whole vector (or all of them when user buffers
  // are not 16-byte aligned).
  const T* l1 = reinterpret_cast<const T*>(loc);
  T* o1 = reinterpret_cast<T*>(uout);
  for (int64_t i = nv * A + threadIdx.x; i < n; i += kThreads) {
    const int off = (int)(i * (int64_t)sizeof(T));
    T x = fin ? fifo_ld<T>(rin, off) : l1[i];
    if (fin && loc) x = VOp<DT, OP>::one(x, l1[i]);
    if (fout) fifo_st<T>(x, rout, off);
    if (uout) o1[i] = x;
  }
}

struct Pipe {
  int r, c, w, pipe;
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
  p.in_ctr = a.ctr + (int64_t)p.r * a.pipe_stride + p.pipe;
  p.out_ctr = a.ctr + (int64_t)nxt * a.pipe_stride + p.pipe;
  const int fpipe = p.c * a.fifo_mul + p.w;
  const int64_t fifo_bytes = (int64_t)a.nslots * a.slot_bytes;
  p.in_fifo = a.fifo + ((int64_t)p.r * a.fifo_stride + fpipe) * fifo_bytes;
  p.out_fifo = a.fifo + ((int64_t)nxt * a.fifo_stride + fpipe) * fifo_bytes;
  return p;
}

// ---------------------------------------------------------------------------
// Bulk kernel
// ---------------------------------------------------------------------------

// Schedule iterator: walks the ring schedule of one workgroup one FIFO slot
// step at a time ("NCCL" book s. 2.3: a loop covers N chunks, stage j of rank
// r visits chunk (r + N - 1 - j) mod N; all-gather round j moves block r - j,
// "NCCL 专家课程 17", Bootstrap Ring 与 AllGather). Divisions happen once per
// loop (or for a ragged tail chunk), never per stage: the chunk / block index
// steps down by one each stage. Empty units produce no step.
template <int DT, int MODE>
struct StepIter {
  static constexpr int64_t E = sizeof(typename Elem<DT>::T);
  static constexpr int64_t A = 16 / E;
  // fixed per workgroup
  const char* send_r;
  char* recv_r;
  int64_t count, chunk, L, ch_lo, slice;
  int N, r, w, wpc;
  // loop and stage
  int64_t off, rem, cur, sub_full, part_lo, part_n;
  int j, idx;
  // current unit and step
  int64_t m, s, local_e, out_e;
  bool recv, use_local, send, store, done;

  __device__ __forceinline__ int nstages() const { return MODE == kAllReduce ? 2 * N - 1 : N; }

  __device__ __forceinline__ void begin_loop() {
    rem = L - off;
    if constexpr (MODE == kAllReduce) {
      cur = ar_loop_chunk(rem, N, chunk, A);
      sub_full = align_up(div_up(cur, wpc), A);
    } else {
      cur = min64(chunk, rem);
      const Range pt = split_part(cur, wpc, w, A);
      part_lo = pt.lo;
      part_n = pt.hi - pt.lo;
    }
    j = 0;
    idx = MODE == kAllGather ? r : (r == 0 ? N - 1 : r - 1);
  }

  __device__ __forceinline__ void set_unit() {
    s = 0;
    if constexpr (MODE == kAllReduce) {
      const int64_t clo = min64((int64_t)idx * cur, rem);
      const int64_t n = min64(clo + cur, rem) - clo;
      const int64_t sub = n == cur ? sub_full : align_up(div_up(n, wpc), A);
      const int64_t plo = min64((int64_t)w * sub, n);
      m = min64(plo + sub, n) - plo;
      local_e = out_e = ch_lo + off + clo + plo;
      recv = j >= 1;
      use_local = j <= N - 1;
      send = j <= 2 * N - 3;
      store = j >= N - 1;
    } else if constexpr (MODE == kReduceScatter) {
      m = part_n;
      out_e = ch_lo + off + part_lo;
      local_e = (int64_t)idx * count + out_e;
      recv = j >= 1;
      use_local = true;
      send = j <= N - 2;
      store = j == N - 1;
    } else {
      m = part_n;
      local_e = ch_lo + off + part_lo;
      out_e = (int64_t)idx * count + local_e;
      recv = j >= 1;
      use_local = j == 0;
      send = j <= N - 2;
      store = true;
    }
  }

  // Moves to the next stage (and loop) until a non-empty unit or the end.
  __device__ __forceinline__ void next_unit() {
    do {
      ++j;
      idx = idx == 0 ? N - 1 : idx - 1;
      if (j == nstages()) {
        off += MODE == kAllReduce ? (int64_t)N * chunk : chunk;
        if (off >= L) {
          done = true;
          return;
        }
        begin_loop();
      }
      set_unit();
    } while (m == 0);
  }

  __device__ __forceinline__ void init(const RingArgs& a, int rank, int c, int part, int64_t slice_elems) {
    N = a.nranks;
    r = rank;
    w = part;
    wpc = a.wpc;
    count = a.count;
    chunk = a.chunk;
    slice = slice_elems;
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
    if (m == 0) next_unit();
  }

  __device__ __forceinline__ void next() {
    s += slice;
    if (s < m) return;
    next_unit();
  }

  __device__ __forceinline__ int64_t ns() const { return min64(slice, m - s); }
  __device__ __forceinline__ const char* local() const { return send_r + (local_e + s) * E; }
  __device__ __forceinline__ char* out() const { return recv_r + (out_e + s) * E; }
};

// Stages the whole-vector part of a step's own operand into LDS with
// direct-to-LDS 128-bit loads (gfx950): lane i of a wave writes 16 bytes at
// the wave's base + 16 i, so LDS holds the same layout as memory.
__device__ __forceinline__ void stage_to_lds(const char* src, int64_t nv, u32x4* lds) {
  const int lane = threadIdx.x & 63;
  for (int64_t i = threadIdx.x; i < nv; i += kThreads) {
    auto g = (__attribute__((address_space(1))) void*)(const_cast<char*>(src) + i * 16);
    auto l = (__attribute__((address_space(3))) void*)(lds + (i - lane));
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
  }
}

template <int DT, int OP, int MODE>
__global__ void __launch_bounds__(kThreads) ring_bulk_kernel(RingArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int64_t A = 16 / (int64_t)sizeof(T);
  extern __shared__ u32x4 lds_stage[];  // [2][slot_bytes / 16] when a.lds_stage
  const Pipe p = locate(a);
  if (p.r == a.skip_rank) return;  // testing knob: a rank that never shows up
  __shared__ uint64_t s_base[2];
  if (threadIdx.x == 0) {
    // Each side's own counter tells where the previous call left this FIFO.
    s_base[0] = ld_relaxed(&p.in_ctr->head);
    s_base[1] = ld_relaxed(&p.out_ctr->tail);
  }
  __syncthreads();
  const uint64_t in_base = s_base[0];
  const uint64_t out_base = s_base[1];
  const uint64_t nslots = (uint64_t)a.nslots;
  const int64_t stage_vecs = a.slot_bytes / 16;
  uint64_t nrecv = 0, nsent = 0;
  uint64_t known_tail = 0, known_head = 0;  // meaningful in thread 0 only
  bool stop = false;                         // thread 0: stop waiting
  const WaitCtx wc = wait_ctx(a);
  // Slot of the next receive / send: (base + count) mod nslots, advanced
  // without a division.
  uint32_t in_slot = (uint32_t)(in_base % nslots);
  uint32_t out_slot = (uint32_t)(out_base % nslots);

  StepIter<DT, MODE> it;
  it.init(a, p.r, p.c, p.w, a.slot_bytes / (int64_t)sizeof(T));
  StepIter<DT, MODE> nx = it;
  if (!nx.done) nx.next();
  const bool lds = a.lds_stage && a.vec_ok;
  int buf = 0;
  if (lds && !it.done && it.use_local) {
    stage_to_lds(it.local(), it.ns() / A, lds_stage);
    wait_vmem();
    __syncthreads();
  }

  while (!it.done) {
    const bool recv = it.recv, send = it.send;
    if (threadIdx.x == 0 && !stop) {
      // A counter value seen earlier may already cover this step. The
      // barrier below keeps every thread's slot accesses after the wait.
      const uint64_t need_tail = in_base + nrecv + 1;
      if (recv && known_tail < need_tail) {
        known_tail = wait_geq(&p.in_ctr->tail, need_tail, wc);
        stop = known_tail == 0;
      }
      const uint64_t need_head = out_base + nsent + 1 - nslots;
      if (!stop && send && nsent + 1 > nslots && known_head < need_head) {
        known_head = wait_geq(&p.out_ctr->head, need_head, wc);
        stop = known_head == 0;
      }
    }
    __syncthreads();
    const int64_t ns = it.ns();
    const char* fin = recv ? p.in_fifo + (int64_t)in_slot * a.slot_bytes : nullptr;
    char* fout = send ? p.out_fifo + (int64_t)out_slot * a.slot_bytes : nullptr;
    move_slice<DT, OP>(ns, fin, it.use_local ? it.local() : nullptr, fout, it.store ? it.out() : nullptr,
                       a.slot_bytes, a.vec_ok, lds && it.use_local ? lds_stage + buf * stage_vecs : nullptr);
    // The next step's own operand streams into the other LDS buffer while
    // this step's stores drain.
    if (lds && !nx.done && nx.use_local) stage_to_lds(nx.local(), nx.ns() / A, lds_stage + (buf ^ 1) * stage_vecs);
    // Every thread's FIFO stores (device-coherent), FIFO loads and staging
    // loads have completed before thread 0 publishes the new tail and head.
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0) {
      if (send) st_relaxed(&p.out_ctr->tail, out_base + nsent + 1);
      if (recv) st_relaxed(&p.in_ctr->head, in_base + nrecv + 1);
    }
    if (recv) {
      ++nrecv;
      in_slot = in_slot + 1 == (uint32_t)nslots ? 0 : in_slot + 1;
    }
    if (send) {
      ++nsent;
      out_slot = out_slot + 1 == (uint32_t)nslots ? 0 : out_slot + 1;
    }
    buf ^= 1;
    it = nx;
    if (!nx.done) nx.next();
  }
}

// ---------------------------------------------------------------------------
// Flag-packed kernel
// ---------------------------------------------------------------------------

// Flag-packed FIFO line: 16 bytes {payload word 0, flag, payload word 1,
// flag}; each 8-byte half is written and read as one 64-bit access, so a
// matching flag vouches for the word stored with it. Polls until both flags
// equal `flag` (or the wait is abandoned) and returns the two payload words.
__device__ __forceinline__ u32x2 poll_line(const uint64_t* line, uint32_t flag, bool& stop, const WaitCtx& w) {
  uint64_t v0 = ld_relaxed(line);
  uint64_t v1 = ld_relaxed(line + 1);
  if (!stop && ((uint32_t)(v0 >> 32) != flag || (uint32_t)(v1 >> 32) != flag)) {
    const uint64_t t0 = wall_clock64();
    uint32_t it = 0;
    while ((uint32_t)(v0 >> 32) != flag || (uint32_t)(v1 >> 32) != flag) {
      if (give_up(w, t0, ++it)) {
        stop = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      v0 = ld_relaxed(line);
      v1 = ld_relaxed(line + 1);
    }
  }
  return u32x2{(uint32_t)v0, (uint32_t)v1};
}

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

template <int DT, int OP, int MODE>
__global__ void __launch_bounds__(kThreads) ring_flag_kernel(RingArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int64_t E = sizeof(T);
  const Pipe p = locate(a);
  if (p.r == a.skip_rank) return;  // testing knob: a rank that never shows up
  __shared__ uint64_t s_base[2];
  __shared__ uint64_t s_head;
  if (threadIdx.x == 0) {
    s_base[0] = ld_relaxed(&p.in_ctr->head);
    s_base[1] = ld_relaxed(&p.out_ctr->tail);
  }
  __syncthreads();
  const uint64_t in_base = s_base[0];
  const uint64_t out_base = s_base[1];
  const uint64_t nslots = (uint64_t)a.nslots;
  uint64_t nrecv = 0, nsent = 0;
  uint64_t head_known = out_base;  // uniform across the workgroup
  uint64_t known_head = 0;         // thread 0
  bool stop = false;               // per thread: stop waiting
  const WaitCtx wc = wait_ctx(a);
  uint32_t in_slot = (uint32_t)(in_base % nslots);
  uint32_t out_slot = (uint32_t)(out_base % nslots);

  StepIter<DT, MODE> it;
  it.init(a, p.r, p.c, p.w, (a.slot_bytes / 2) / E);  // payload is half of a slot
  for (; !it.done; it.next()) {
    const bool recv = it.recv, send = it.send;
    if (send && nsent + 1 > nslots) {
      const uint64_t need = out_base + nsent + 1 - nslots;
      if (head_known < need) {  // uniform branch
        if (threadIdx.x == 0) {
          if (!stop && known_head < need) {
            known_head = wait_geq(&p.out_ctr->head, need, wc);
            stop = known_head == 0;
          }
          s_head = known_head > need ? known_head : need;
        }
        __syncthreads();
        head_known = s_head;
        __syncthreads();
      }
    }
    const uint32_t flag_in = (uint32_t)(in_base + nrecv + 1);
    const uint32_t flag_out = (uint32_t)(out_base + nsent + 1);
    const uint64_t* fin = recv ? reinterpret_cast<const uint64_t*>(p.in_fifo + (int64_t)in_slot * a.slot_bytes) : nullptr;
    uint64_t* fout = send ? reinterpret_cast<uint64_t*>(p.out_fifo + (int64_t)out_slot * a.slot_bytes) : nullptr;
    const int64_t nbytes = it.ns() * E;
    const int nlines = (int)div_up(nbytes, 8);  // <= kThreads * kFlagLinesPerThread
    const char* lp = it.use_local ? it.local() : nullptr;
    char* op = it.store ? it.out() : nullptr;
    if (nlines <= kThreads) {
      // At most one line per thread (small messages): the shortest path from
      // a flag's arrival to the next hop's store.
      const int li = threadIdx.x;
      if (li < nlines) {
        const int valid = (int)min64(8, nbytes - (int64_t)li * 8);
        u32x2 loc = u32x2{0u, 0u};
        if (lp) loc = load_payload<DT>(lp + (int64_t)li * 8, valid, a.vec_ok);
        u32x2 x;
        if (fin) {
          x = poll_line(fin + 2 * li, flag_in, stop, wc);
          if (lp) x = VOp<DT, OP>::v2(x, loc);
        } else {
          x = loc;
        }
        if (fout) {
          st_relaxed(fout + 2 * li, ((uint64_t)flag_out << 32) | x.x);
          st_relaxed(fout + 2 * li + 1, ((uint64_t)flag_out << 32) | x.y);
        }
        if (op) store_payload<DT>(op + (int64_t)li * 8, x, valid, a.vec_ok);
      }
    } else {
      // Several lines per thread: each thread owns lines tid, tid + 256, ...;
      // all of its own-operand loads and first flag polls are issued together,
      // then only lines whose flags have not arrived are polled again.
      u32x2 x[kFlagLinesPerThread];
      u32x2 loc[kFlagLinesPerThread];
#pragma unroll
      for (int u = 0; u < kFlagLinesPerThread; ++u) {
        const int li = threadIdx.x + u * kThreads;
        loc[u] = u32x2{0u, 0u};
        if (lp && li < nlines) loc[u] = load_payload<DT>(lp + li * 8, (int)min64(8, nbytes - li * 8), a.vec_ok);
      }
      if (fin) {
        uint64_t v0[kFlagLinesPerThread], v1[kFlagLinesPerThread];
#pragma unroll
        for (int u = 0; u < kFlagLinesPerThread; ++u) {
          const int li = threadIdx.x + u * kThreads;
          v0[u] = v1[u] = 0;
          if (li < nlines) {
            v0[u] = ld_relaxed(fin + 2 * li);
            v1[u] = ld_relaxed(fin + 2 * li + 1);
          }
        }
        uint32_t pending = 0;
#pragma unroll
        for (int u = 0; u < kFlagLinesPerThread; ++u) {
          const int li = threadIdx.x + u * kThreads;
          if (li < nlines && ((uint32_t)(v0[u] >> 32) != flag_in || (uint32_t)(v1[u] >> 32) != flag_in))
            pending |= 1u << u;
        }
        if (pending && !stop) {
          const uint64_t t0 = wall_clock64();
          uint32_t spins = 0;
          while (pending) {
            if (give_up(wc, t0, ++spins)) {
              stop = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int u = 0; u < kFlagLinesPerThread; ++u) {
              if (pending & (1u << u)) {
                const int li = threadIdx.x + u * kThreads;
                v0[u] = ld_relaxed(fin + 2 * li);
                v1[u] = ld_relaxed(fin + 2 * li + 1);
                if ((uint32_t)(v0[u] >> 32) == flag_in && (uint32_t)(v1[u] >> 32) == flag_in) pending &= ~(1u << u);
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kFlagLinesPerThread; ++u) {
          x[u] = u32x2{(uint32_t)v0[u], (uint32_t)v1[u]};
          if (lp) x[u] = VOp<DT, OP>::v2(x[u], loc[u]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kFlagLinesPerThread; ++u) x[u] = loc[u];
      }
#pragma unroll
      for (int u = 0; u < kFlagLinesPerThread; ++u) {
        const int li = threadIdx.x + u * kThreads;
        if (li < nlines) {
          if (fout) {
            st_relaxed(fout + 2 * li, ((uint64_t)flag_out << 32) | x[u].x);
            st_relaxed(fout + 2 * li + 1, ((uint64_t)flag_out << 32) | x[u].y);
          }
          if (op) store_payload<DT>(op + li * 8, x[u], (int)min64(8, nbytes - li * 8), a.vec_ok);
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
    if (send) {
      ++nsent;
      out_slot = out_slot + 1 == (uint32_t)nslots ? 0 : out_slot + 1;
    }
  }
  // Leave both counters at the number of steps this call moved, so the next
  // call (either protocol) starts from the same base on both sides.
  __syncthreads();
  if (threadIdx.x == 0) {
    st_relaxed(&p.in_ctr->head, in_base + nrecv);
    st_relaxed(&p.out_ctr->tail, out_base + nsent);
  }
}

// ---------------------------------------------------------------------------
// Double-binary-tree all-reduce (flag-packed lines)
// ---------------------------------------------------------------------------

__device__ __forceinline__ WaitCtx wait_ctx(const TreeArgs& a) {
  return WaitCtx{a.dev_abort, a.host_abort, a.host_err, a.timeout_ticks};
}

// One slice: every line is the fold of the own operand (if any) and the
// input lines in child order (own first, then first child, then second
// child), stored to each output FIFO under that FIFO's flag and to the
// receive buffer. fin[j] / fout[j] (j < nin / nout) point at this step's
// slots. Arrays are only ever indexed with unrolled constants.
template <int DT, int OP>
__device__ __forceinline__ void tree_lines(int nlines, int64_t nbytes, const char* lp, char* op, int nin,
                                           const uint64_t* const (&fin)[2], const uint32_t (&flag_in)[2],
                                           int nout, uint64_t* const (&fout)[2], const uint32_t (&flag_out)[2],
                                           int vec_ok, bool& stop, const WaitCtx& wc) {
  if (nlines <= kThreads) {
    // At most one line per thread: the shortest path from a flag's arrival
    // to the next hop's store.
    const int li = threadIdx.x;
    if (li >= nlines) return;
    const int valid = (int)min64(8, nbytes - (int64_t)li * 8);
    u32x2 x = u32x2{0u, 0u};
    if (lp) x = load_payload<DT>(lp + (int64_t)li * 8, valid, vec_ok);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < nin) {
        const u32x2 y = poll_line(fin[j] + 2 * li, flag_in[j], stop, wc);
        x = (lp || j > 0) ? VOp<DT, OP>::v2(x, y) : y;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < nout) {
        st_relaxed(fout[j] + 2 * li, ((uint64_t)flag_out[j] << 32) | x.x);
        st_relaxed(fout[j] + 2 * li + 1, ((uint64_t)flag_out[j] << 32) | x.y);
      }
    }
    if (op) store_payload<DT>(op + (int64_t)li * 8, x, valid, vec_ok);
    return;
  }
  // Several lines per thread (lines tid, tid + 256, ...): issue every load
  // first, then poll again only the lines whose flags are still missing.
  constexpr int U = kFlagLinesPerThread;
  u32x2 x[U];
  uint64_t v0[2][U], v1[2][U];
  uint32_t pending = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int li = threadIdx.x + u * kThreads;
    x[u] = u32x2{0u, 0u};
    if (lp && li < nlines) x[u] = load_payload<DT>(lp + (int64_t)li * 8, (int)min64(8, nbytes - (int64_t)li * 8), vec_ok);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v0[j][u] = v1[j][u] = 0;
      if (j < nin && li < nlines) {
        v0[j][u] = ld_relaxed(fin[j] + 2 * li);
        v1[j][u] = ld_relaxed(fin[j] + 2 * li + 1);
        if ((uint32_t)(v0[j][u] >> 32) != flag_in[j] || (uint32_t)(v1[j][u] >> 32) != flag_in[j])
          pending |= 1u << (j * U + u);
      }
    }
  }
  if (pending && !stop) {
    const uint64_t t0 = wall_clock64();
    uint32_t spins = 0;
    while (pending) {
      if (give_up(wc, t0, ++spins)) {
        stop = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (pending & (1u << (j * U + u))) {
            const int li = threadIdx.x + u * kThreads;
            v0[j][u] = ld_relaxed(fin[j] + 2 * li);
            v1[j][u] = ld_relaxed(fin[j] + 2 * li + 1);
            if ((uint32_t)(v0[j][u] >> 32) == flag_in[j] && (uint32_t)(v1[j][u] >> 32) == flag_in[j])
              pending &= ~(1u << (j * U + u));
          }
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int li = threadIdx.x + u * kThreads;
    if (li < nlines) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j < nin) {
          const u32x2 y = u32x2{(uint32_t)v0[j][u], (uint32_t)v1[j][u]};
          x[u] = (lp || j > 0) ? VOp<DT, OP>::v2(x[u], y) : y;
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j < nout) {
          st_relaxed(fout[j] + 2 * li, ((uint64_t)flag_out[j] << 32) | x[u].x);
          st_relaxed(fout[j] + 2 * li + 1, ((uint64_t)flag_out[j] << 32) | x[u].y);
        }
      }
      if (op) store_payload<DT>(op + (int64_t)li * 8, x[u], (int)min64(8, nbytes - (int64_t)li * 8), vec_ok);
    }
  }
}

// One workgroup per (rank, tree, channel, role). Role 0 folds the rank's own
// slice with its children's partials and passes the result to the parent;
// at the root the result is final: it is stored and sent down to the
// children. Role 1 receives the result from the parent, stores it and passes
// it on to the children. Every FIFO carries one step per slice of the
// channel; its producer owns `tail`, its consumer `head`, and a line's flag
// is the low 32 bits of (step + 1).
template <int DT, int OP>
__global__ void __launch_bounds__(kThreads) tree_flag_kernel(TreeArgs a) {
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
  const int64_t slice = (a.slot_bytes / 2) / E;
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
  const int64_t fifo_words = (int64_t)a.nslots * a.slot_bytes / 8;
  const uint64_t* in_fifo[2];
  uint64_t* out_fifo[2];
  FifoCtr* in_ctr[2];
  FifoCtr* out_ctr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    in_fifo[j] = in_f[j] >= 0 ? reinterpret_cast<const uint64_t*>(a.fifo) + in_f[j] * fifo_words : nullptr;
    out_fifo[j] = out_f[j] >= 0 ? reinterpret_cast<uint64_t*>(a.fifo) + out_f[j] * fifo_words : nullptr;
    in_ctr[j] = in_f[j] >= 0 ? a.ctr + in_f[j] : nullptr;
    out_ctr[j] = out_f[j] >= 0 ? a.ctr + out_f[j] : nullptr;
  }
  const char* own = role == 0 ? a.send[v] + cr.lo * E : nullptr;
  char* dst = (role == 1 || root) ? a.recv[v] + cr.lo * E : nullptr;

  __shared__ uint64_t s_base[4];
  __shared__ uint64_t s_head[2];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s_base[j] = j < nin ? ld_relaxed(&in_ctr[j]->head) : 0;
      s_base[2 + j] = j < nout ? ld_relaxed(&out_ctr[j]->tail) : 0;
    }
  }
  __syncthreads();
  const uint64_t in_base[2] = {s_base[0], s_base[1]};
  const uint64_t out_base[2] = {s_base[2], s_base[3]};
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
          if (j < nout) head_known[j] = s_head[j];
        __syncthreads();
      }
    }
    const int64_t n = min64(slice, cr.hi - cr.lo - s * slice);
    const int64_t nbytes = n * E;
    const int nlines = (int)div_up(nbytes, 8);
    const uint64_t* fin[2];
    uint64_t* fout[2];
    uint32_t flag_in[2], flag_out[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fin[j] = j < nin ? in_fifo[j] + (int64_t)in_slot[j] * (a.slot_bytes / 8) : nullptr;
      fout[j] = j < nout ? out_fifo[j] + (int64_t)out_slot[j] * (a.slot_bytes / 8) : nullptr;
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
  }
}

// ---------------------------------------------------------------------------
// Copy kernel: all-to-all blocks, or one-rank local copies
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(kThreads) copy_kernel(CopyArgs a) {
  const int blk = blockIdx.y;
  int src_rank, dst_rank;
  int64_t src_off = 0, dst_off = 0;
  if (a.transpose) {
    dst_rank = blk / a.nranks;
    src_rank = blk - dst_rank * a.nranks;
    src_off = (int64_t)dst_rank * a.block_bytes;
    dst_off = (int64_t)src_rank * a.block_bytes;
  } else {
    src_rank = dst_rank = blk;
  }
  const char* src = a.src[src_rank] + src_off;
  char* dst = a.dst[dst_rank] + dst_off;
  const int tid = threadIdx.x;
  if (a.vec_ok) {
    const int64_t nv = a.block_bytes / 16;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* d4 = reinterpret_cast<u32x4*>(dst);
    const int64_t tile = (int64_t)kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * tile; base < nv; base += (int64_t)gridDim.x * tile) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        if (i < nv) v[u] = __builtin_nontemporal_load(s4 + i);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        if (i < nv) __builtin_nontemporal_store(v[u], d4 + i);
      }
    }
    for (int64_t i = nv * 16 + (int64_t)blockIdx.x * kThreads + tid; i < a.block_bytes;
         i += (int64_t)gridDim.x * kThreads)
      dst[i] = src[i];
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.block_bytes; i += (int64_t)gridDim.x * kThreads)
      dst[i] = src[i];
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------

template <int DT, int OP, int MODE>
static hipError_t launch_bulk_t(const RingArgs& a, hipStream_t s) {
  const int grid = a.nranks * a.nchannels * a.wpc;
  const size_t lds = a.lds_stage ? 2 * (size_t)a.slot_bytes : 0;
  hipLaunchKernelGGL((ring_bulk_kernel<DT, OP, MODE>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT, int OP, int MODE>
static hipError_t launch_flag_t(const RingArgs& a, hipStream_t s) {
  const int grid = a.nranks * a.nchannels * a.wpc;
  hipLaunchKernelGGL((ring_flag_kernel<DT, OP, MODE>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <bool FLAG, int DT, int OP, int MODE>
static hipError_t launch_t(const RingArgs& a, hipStream_t s) {
  if constexpr (FLAG) return launch_flag_t<DT, OP, MODE>(a, s);
  else return launch_bulk_t<DT, OP, MODE>(a, s);
}

template <bool FLAG, int DT, int MODE>
static hipError_t dispatch_op(const RingArgs& a, int op, hipStream_t s) {
  if constexpr (MODE == kAllGather) {
    (void)op;
    return launch_t<FLAG, DT, RINGSIM_SUM, MODE>(a, s);
  } else {
    switch (op) {
      case RINGSIM_SUM: return launch_t<FLAG, DT, RINGSIM_SUM, MODE>(a, s);
      case RINGSIM_PROD: return launch_t<FLAG, DT, RINGSIM_PROD, MODE>(a, s);
      case RINGSIM_MAX: return launch_t<FLAG, DT, RINGSIM_MAX, MODE>(a, s);
      case RINGSIM_MIN: return launch_t<FLAG, DT, RINGSIM_MIN, MODE>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
}

template <bool FLAG, int MODE>
static hipError_t dispatch_dtype(const RingArgs& a, int dtype, int op, hipStream_t s) {
  switch (dtype) {
    case RINGSIM_INT32: return dispatch_op<FLAG, RINGSIM_INT32, MODE>(a, op, s);
    case RINGSIM_INT64: return dispatch_op<FLAG, RINGSIM_INT64, MODE>(a, op, s);
    case RINGSIM_FLOAT32: return dispatch_op<FLAG, RINGSIM_FLOAT32, MODE>(a, op, s);
    case RINGSIM_BFLOAT16: return dispatch_op<FLAG, RINGSIM_BFLOAT16, MODE>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool FLAG>
static hipError_t dispatch_mode(const RingArgs& a, int mode, int dtype, int op, hipStream_t s) {
  switch (mode) {
    case kAllReduce: return dispatch_dtype<FLAG, kAllReduce>(a, dtype, op, s);
    case kReduceScatter: return dispatch_dtype<FLAG, kReduceScatter>(a, dtype, op, s);
    case kAllGather: return dispatch_dtype<FLAG, kAllGather>(a, dtype, op, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ring_bulk(const RingArgs& a, int mode, int dtype, int op, hipStream_t s) {
  return dispatch_mode<false>(a, mode, dtype, op, s);
}

hipError_t launch_ring_flag(const RingArgs& a, int mode, int dtype, int op, hipStream_t s) {
  return dispatch_mode<true>(a, mode, dtype, op, s);
}

template <int DT>
static hipError_t tree_dispatch_op(const TreeArgs& a, int op, hipStream_t s) {
  const int grid = a.nranks * 2 * a.nchannels * 2;
  switch (op) {
    case RINGSIM_SUM: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_SUM>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_PROD: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_PROD>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MAX: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_MAX>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MIN: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_MIN>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tree_flag(const TreeArgs& a, int dtype, int op, hipStream_t s) {
  switch (dtype) {
    case RINGSIM_INT32: return tree_dispatch_op<RINGSIM_INT32>(a, op, s);
    case RINGSIM_INT64: return tree_dispatch_op<RINGSIM_INT64>(a, op, s);
    case RINGSIM_FLOAT32: return tree_dispatch_op<RINGSIM_FLOAT32>(a, op, s);
    case RINGSIM_BFLOAT16: return tree_dispatch_op<RINGSIM_BFLOAT16>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  const int nblocks = a.transpose ? a.nranks * a.nranks : a.nranks;
  const int64_t tile = a.vec_ok ? (int64_t)kThreads * kUnroll * 16 : (int64_t)kThreads;
  int64_t tiles = div_up(a.block_bytes, tile);
  const int64_t cap = max64(1, 4096 / nblocks);
  if (tiles > cap) tiles = cap;
  if (tiles < 1) tiles = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)tiles, (unsigned)nblocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename K>
static int occ(K k, size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, lds) != hipSuccess) return 0;
  return n;
}

int ring_blocks_per_cu(size_t bulk_lds_bytes) {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_OCC_DT(DT)                                                                 \
  acc(occ(ring_bulk_kernel<DT, RINGSIM_SUM, kAllReduce>, bulk_lds_bytes));            \
  acc(occ(ring_bulk_kernel<DT, RINGSIM_MAX, kAllReduce>, bulk_lds_bytes));            \
  acc(occ(ring_bulk_kernel<DT, RINGSIM_PROD, kReduceScatter>, bulk_lds_bytes));       \
  acc(occ(ring_bulk_kernel<DT, RINGSIM_SUM, kAllGather>, bulk_lds_bytes));            \
  acc(occ(ring_flag_kernel<DT, RINGSIM_SUM, kAllReduce>, 0));                         \
  acc(occ(ring_flag_kernel<DT, RINGSIM_MIN, kReduceScatter>, 0));                     \
  acc(occ(ring_flag_kernel<DT, RINGSIM_SUM, kAllGather>, 0));
  RS_OCC_DT(RINGSIM_INT32)
  RS_OCC_DT(RINGSIM_INT64)
  RS_OCC_DT(RINGSIM_FLOAT32)
  RS_OCC_DT(RINGSIM_BFLOAT16)
#undef RS_OCC_DT
  return m == (1 << 30) ? 0 : m;
}

int tree_blocks_per_cu() {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_TREE_OCC_DT(DT)                              \
  acc(occ(tree_flag_kernel<DT, RINGSIM_SUM>, 0));       \
  acc(occ(tree_flag_kernel<DT, RINGSIM_PROD>, 0));      \
  acc(occ(tree_flag_kernel<DT, RINGSIM_MAX>, 0));       \
  acc(occ(tree_flag_kernel<DT, RINGSIM_MIN>, 0));
  RS_TREE_OCC_DT(RINGSIM_INT32)
  RS_TREE_OCC_DT(RINGSIM_INT64)
  RS_TREE_OCC_DT(RINGSIM_FLOAT32)
  RS_TREE_OCC_DT(RINGSIM_BFLOAT16)
#undef RS_TREE_OCC_DT
  return m == (1 << 30) ? 0 : m;
}

}  // namespace ringsim
