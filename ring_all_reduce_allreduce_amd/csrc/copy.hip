// copy.hip -- all-to-all as a block transpose, one-rank local copies, and
// the zero fill that resets FIFOs and counters.
#include <algorithm>

#include "ringsim_device.h"

namespace ringsim {

constexpr int64_t kCopyWorkgroups = 1024;

// ---------------------------------------------------------------------------
// Copy kernel: all-to-all blocks, or one-rank local copies
// ---------------------------------------------------------------------------

// Block b of the launch: all-to-all block (source rank, destination rank) =
// (b mod N, b / N), read at the destination's offset in the source buffer
// and written at the source's offset in the destination buffer; or, for local
// copies, rank b's whole buffer.
struct CopyBlock {
  const char* src;
  char* dst;
};

__device__ __forceinline__ CopyBlock copy_block(const CopyArgs& a, int b) {
  if (a.transpose) {
    const int d = b / a.nranks, s = b - d * a.nranks;
    return CopyBlock{a.src[s] + (int64_t)d * a.block_bytes, a.dst[d] + (int64_t)s * a.block_bytes};
  }
  return CopyBlock{a.src[b], a.dst[b]};
}

// The workgroups walk the tiles of all blocks with one stride (a flat grid of
// a few per compute unit beats one grid row per block: every workgroup keeps
// streaming instead of finishing its block early). A tile is 256 threads x 8
// vectors of 16 bytes, non-temporal both ways (each byte is touched once).
__global__ void __launch_bounds__(kThreads) copy_kernel(CopyArgs a) {
  const int nblk = a.transpose ? a.nranks * a.nranks : a.nranks;
  const int tid = threadIdx.x;
  int64_t nv = 0;  // whole vectors per block
  if (a.vec_ok) {
    nv = a.block_bytes / 16;
    constexpr int64_t kTile = (int64_t)kThreads * kUnroll;
    const int64_t per_block = div_up(nv, kTile);
    const int64_t total = per_block * nblk;
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
      const int b = (int)(t / per_block);
      const int64_t base = (t - (int64_t)b * per_block) * kTile;
      const CopyBlock cb = copy_block(a, b);
      const u32x4* s4 = reinterpret_cast<const u32x4*>(cb.src) + base;
      u32x4* d4 = reinterpret_cast<u32x4*>(cb.dst) + base;
      u32x4 v[kUnroll];
      if (base + kTile <= nv) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(s4 + u * kThreads + tid);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], d4 + u * kThreads + tid);
      } else {
        const int64_t left = nv - base;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          if (u * kThreads + tid < left) v[u] = __builtin_nontemporal_load(s4 + u * kThreads + tid);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          if (u * kThreads + tid < left) __builtin_nontemporal_store(v[u], d4 + u * kThreads + tid);
      }
    }
  }
  // Bytes past the last whole vector of every block (all of them when the
  // buffers are not 16-byte aligned).
  const int64_t rest = a.block_bytes - nv * 16;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < rest * nblk; i += (int64_t)gridDim.x * kThreads) {
    const int b = (int)(i / rest);
    const CopyBlock cb = copy_block(a, b);
    const int64_t off = nv * 16 + (i - (int64_t)b * rest);
    cb.dst[off] = cb.src[off];
  }
}


__global__ void __launch_bounds__(kThreads) zero_kernel(u32x4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, p + i);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(kCopyWorkgroups, div_up(n, kThreads)));
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, static_cast<u32x4*>(p), n);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  const int nblk = a.transpose ? a.nranks * a.nranks : a.nranks;
  const int64_t per_block = a.vec_ok ? div_up(a.block_bytes / 16, (int64_t)kThreads * kUnroll)
                                     : div_up(a.block_bytes, (int64_t)kThreads);
  // About four workgroups per compute unit, never more than there are tiles.
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(kCopyWorkgroups, per_block * nblk));
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ringsim
