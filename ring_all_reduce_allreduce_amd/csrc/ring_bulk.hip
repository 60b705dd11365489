// ring_bulk.hip -- the bulk ring kernel (Simple protocol, "NCCL" book,
// s. 2.4): FIFO slots hold raw payload and readiness travels in separate
// 64-bit step counters (tail: slots filled, head: slots drained). Slot data
// is written and read with device-scope coherent (SC1) accesses, so a
// counter published once those accesses have completed is enough to order
// them; no L2 writeback or invalidate is needed. Workgroup ids are
// rank-major, so that when the pipeline count is a multiple of 8 every
// workgroup of a pipeline is dispatched to the same XCD.
#include "ringsim_device.h"

namespace ringsim {

// ---------------------------------------------------------------------------
// Bulk data movement: one FIFO slot worth of a unit
// ---------------------------------------------------------------------------

// FIFO slots are accessed through buffer resources (bounds-checked against the
// slot size) with device-scope coherence (SC1): a store is visible to every
// XCD once it completes and a load never returns a stale line, so a step
// counter published after the stores complete is all the consumer needs - no
// L2 writeback or invalidate on the data path. User buffers use plain global
// accesses marked non-temporal (each byte is touched once per launch).
constexpr int kPolFifo = 16;            // SC1: device scope
constexpr int kPolFifoStream = 16 | 2;  // SC1 + NT: device scope, no reuse expected

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
  if (base < n) {
    // The last, partial tile: the same shape with every access guarded, so
    // that all its loads are in flight before the first use and its stores
    // leave together (a loop over it would wait for each store before the
    // next load).
    u32x4 v[kUnroll];
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * kThreads + tid < n) v[u] = load_src(base + u * kThreads + tid);
    if constexpr (RED) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kThreads + tid < n) x[u] = load_loc(base + u * kThreads + tid);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kThreads + tid < n) v[u] = VOp<DT, OP>::v4(v[u], x[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (base + u * kThreads + tid < n) store(base + u * kThreads + tid, v[u]);
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
  const rsrc_t rin = make_uniform_rsrc(fin, fin ? slot_bytes : 0);
  const rsrc_t rout = make_uniform_rsrc(fout, fout ? slot_bytes : 0);
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


// ---------------------------------------------------------------------------
// Bulk kernel
// ---------------------------------------------------------------------------

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

template <int DT, int OP, int MODE, int VAR>
__global__ void __launch_bounds__(kThreads) ring_bulk_kernel(RingArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int64_t A = 16 / (int64_t)sizeof(T);
  extern __shared__ u32x4 lds_stage[];  // [2][slot_bytes / 16] when a.lds_stage
  const Pipe p = locate(a);
  if (p.r == a.skip_rank) return;  // testing knob: a rank that never shows up
  __shared__ uint64_t s_base[2];
  if (threadIdx.x == 0) {
    // Each side's own counter tells where the previous call left this FIFO
    // (both loads in flight before either value is used).
    const uint64_t head = ld_relaxed(&p.in_ctr->head);
    const uint64_t tail = ld_relaxed(&p.out_ctr->tail);
    s_base[0] = head;
    s_base[1] = tail;
  }
  __syncthreads();
  const uint64_t in_base = uniform64(s_base[0]);
  const uint64_t out_base = uniform64(s_base[1]);
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

  // Step groups (a.group > 0): a stage moves at most a.group slot steps
  // before the next stage runs, so a FIFO of 2 x a.group slots suffices
  // whatever the chunk size.
  const int64_t slice = a.slot_bytes / (int64_t)sizeof(T);
  StepIter<DT, MODE> it;
  it.init(a, p.r, p.c, p.w, slice, VAR == kBulkGrouped ? (int64_t)a.group * slice : 0);
  StepIter<DT, MODE> nx = it;
  if (!nx.done) nx.next();
  const bool lds = a.lds_stage && a.vec_ok;
  // Debug FIFO integrity records of the slots this workgroup reads and
  // writes (null unless the communicator was created with RINGSIM_DEBUG_FIFO).
  FifoEcho* echo_in = nullptr;
  FifoEcho* echo_out = nullptr;
  if constexpr (VAR == kBulkEcho) {
    const int fpipe = p.c * a.fifo_mul + p.w;
    echo_in = a.echo + ((int64_t)p.r * a.fifo_stride + fpipe) * a.nslots;
    echo_out = a.echo + ((int64_t)p.nxt * a.fifo_stride + fpipe) * a.nslots;
  }
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
      if (VAR == kBulkEcho && !stop && recv) {
        // Debug: the slot must hold the step and size this step expects.
        const FifoEcho* e = echo_in + in_slot;
        const uint64_t step = __hip_atomic_load(&e->step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t bytes = __hip_atomic_load(&e->bytes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (step != in_base + nrecv || bytes != (uint32_t)(it.ns() * (int64_t)sizeof(T))) raise_error(wc, kErrFifoEcho);
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
    if (VAR == kBulkEcho && send && threadIdx.x == 0) {
      // Debug: completes with the slot's data, before the tail is published.
      FifoEcho* e = echo_out + out_slot;
      __hip_atomic_store(&e->step, out_base + nsent, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&e->bytes, (uint32_t)(ns * (int64_t)sizeof(T)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
// Host-side dispatch
// ---------------------------------------------------------------------------

namespace {

struct BulkLaunch {
  template <int DT, int OP, int MODE>
  static hipError_t run(const RingArgs& a, hipStream_t s) {
    const int grid = a.nranks * a.nchannels * a.wpc;
    const size_t lds = a.lds_stage ? 2 * (size_t)a.slot_bytes : 0;
    if (a.group > 0) {
      if constexpr (MODE != kAllReduce) {
        return hipErrorInvalidValue;  // step groups serve the all-reduce only
      } else {
        if (a.echo) return hipErrorInvalidValue;
        hipLaunchKernelGGL((ring_bulk_kernel<DT, OP, MODE, kBulkGrouped>), dim3(grid), dim3(kThreads), lds, s, a);
      }
    } else if (a.echo) {
      hipLaunchKernelGGL((ring_bulk_kernel<DT, OP, MODE, kBulkEcho>), dim3(grid), dim3(kThreads), lds, s, a);
    } else {
      hipLaunchKernelGGL((ring_bulk_kernel<DT, OP, MODE, kBulkPlain>), dim3(grid), dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_ring_bulk(const RingArgs& a, int mode, int dtype, int op, hipStream_t s) {
  return dispatch_ring<BulkLaunch>(a, mode, dtype, op, s);
}

int bulk_blocks_per_cu(size_t lds_bytes) {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_OCC_BULK(DT)                                                                    \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_SUM, kAllReduce, kBulkPlain>, lds_bytes));      \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_MAX, kAllReduce, kBulkPlain>, lds_bytes));      \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_PROD, kReduceScatter, kBulkPlain>, lds_bytes)); \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_SUM, kAllGather, kBulkPlain>, lds_bytes));      \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_SUM, kAllReduce, kBulkGrouped>, lds_bytes));    \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_MAX, kAllReduce, kBulkGrouped>, lds_bytes));    \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_SUM, kAllReduce, kBulkEcho>, lds_bytes));       \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_PROD, kReduceScatter, kBulkEcho>, lds_bytes));  \
  acc(occupancy(ring_bulk_kernel<DT, RINGSIM_SUM, kAllGather, kBulkEcho>, lds_bytes));
  RS_OCC_BULK(RINGSIM_INT32)
  RS_OCC_BULK(RINGSIM_INT64)
  RS_OCC_BULK(RINGSIM_FLOAT32)
  RS_OCC_BULK(RINGSIM_BFLOAT16)
#undef RS_OCC_BULK
  return m == (1 << 30) ? 0 : m;
}

}  // namespace ringsim
