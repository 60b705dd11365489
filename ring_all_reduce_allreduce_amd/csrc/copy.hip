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
// units of V, non-temporal both ways (each byte is touched once). V is the
// widest of 16, 8, 4, 2 and 1 bytes that divides the block size and every
// buffer address, so blocks that are not whole 16-byte vectors still move in
// elements, not bytes.
template <typename V>
__global__ void __launch_bounds__(kThreads) copy_kernel(CopyArgs a) {
  const int nblk = a.transpose ? a.nranks * a.nranks : a.nranks;
  const int tid = threadIdx.x;
  const int64_t nu = a.block_bytes / (int64_t)sizeof(V);  // units per block
  constexpr int64_t kTile = (int64_t)kThreads * kUnroll;
  const int64_t per_block = div_up(nu, kTile);
  const int64_t total = per_block * nblk;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    const int b = (int)(t / per_block);
    const int64_t base = (t - (int64_t)b * per_block) * kTile;
    const CopyBlock cb = copy_block(a, b);
    const V* s = reinterpret_cast<const V*>(cb.src) + base;
    V* d = reinterpret_cast<V*>(cb.dst) + base;
    V v[kUnroll];
    if (base + kTile <= nu) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(s + u * kThreads + tid);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], d + u * kThreads + tid);
    } else {
      const int64_t left = nu - base;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (u * kThreads + tid < left) v[u] = __builtin_nontemporal_load(s + u * kThreads + tid);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (u * kThreads + tid < left) __builtin_nontemporal_store(v[u], d + u * kThreads + tid);
    }
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
  // Widest unit that divides the block size and every buffer address.
  uint64_t g = (uint64_t)a.block_bytes | 16u;
  for (int r = 0; r < a.nranks; ++r) g |= (uint64_t)(uintptr_t)a.src[r] | (uint64_t)(uintptr_t)a.dst[r];
  const int unit = (int)(g & (~g + 1));  // lowest set bit: 1, 2, 4, 8 or 16
  const int64_t per_block = div_up(a.block_bytes / unit, (int64_t)kThreads * kUnroll);
  // About four workgroups per compute unit, never more than there are tiles.
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(kCopyWorkgroups, per_block * nblk));
  const dim3 gd((unsigned)grid), bd(kThreads);
  switch (unit) {
    case 16: hipLaunchKernelGGL(copy_kernel<u32x4>, gd, bd, 0, s, a); break;
    case 8: hipLaunchKernelGGL(copy_kernel<u32x2>, gd, bd, 0, s, a); break;
    case 4: hipLaunchKernelGGL(copy_kernel<uint32_t>, gd, bd, 0, s, a); break;
    case 2: hipLaunchKernelGGL(copy_kernel<uint16_t>, gd, bd, 0, s, a); break;
    default: hipLaunchKernelGGL(copy_kernel<uint8_t>, gd, bd, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace ringsim
