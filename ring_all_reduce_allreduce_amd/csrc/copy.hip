// copy.hip -- all-to-all as a block transpose, and one-rank local copies.
#include "ringsim_device.h"

namespace ringsim {

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

}  // namespace ringsim
