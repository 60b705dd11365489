// line_format.h -- the two flag-packed FIFO line formats shared by the ring
// line kernels and the double-binary-tree kernel ("NCCL" book, s. 2.4: LL
// and LL128 carry a flag inside the data, so the receiver polls the data
// itself; ch. 5: LL moves half a line of payload, LL128 120 of 128 bytes).
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

}  // namespace ringsim
