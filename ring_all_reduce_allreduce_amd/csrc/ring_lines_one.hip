// ring_lines_one.hip -- instantiations of the line-protocol ring kernel for
// steps of at most one line per thread (256 lines).
#include "ring_lines.h"

namespace ringsim {

namespace {

// Local to this file: the other instantiation file has its own launcher.
template <int LP>
struct LineLaunch {
  template <int DT, int OP, int MODE>
  static hipError_t run(const RingArgs& a, hipStream_t s) {
    const int grid = a.nranks * a.nchannels * a.wpc;
    hipLaunchKernelGGL((ring_line_kernel<LP, kLinesOne, DT, OP, MODE>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_ring_lines_one(const RingArgs& a, int line_proto, int mode, int dtype, int op, hipStream_t s) {
  if (line_proto == kLineWide) return dispatch_ring<LineLaunch<kLineWide>>(a, mode, dtype, op, s);
  return dispatch_ring<LineLaunch<kLineFlag>>(a, mode, dtype, op, s);
}

int line_one_blocks_per_cu() {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_OCC_LINE(LP, DT)                                                           \
  acc(occupancy(ring_line_kernel<LP, kLinesOne, DT, RINGSIM_SUM, kAllReduce>, 0));      \
  acc(occupancy(ring_line_kernel<LP, kLinesOne, DT, RINGSIM_MIN, kReduceScatter>, 0));  \
  acc(occupancy(ring_line_kernel<LP, kLinesOne, DT, RINGSIM_SUM, kAllGather>, 0));
  RS_OCC_LINE(kLineFlag, RINGSIM_INT32)
  RS_OCC_LINE(kLineFlag, RINGSIM_INT64)
  RS_OCC_LINE(kLineFlag, RINGSIM_FLOAT32)
  RS_OCC_LINE(kLineFlag, RINGSIM_BFLOAT16)
  RS_OCC_LINE(kLineWide, RINGSIM_INT32)
  RS_OCC_LINE(kLineWide, RINGSIM_INT64)
  RS_OCC_LINE(kLineWide, RINGSIM_FLOAT32)
  RS_OCC_LINE(kLineWide, RINGSIM_BFLOAT16)
#undef RS_OCC_LINE
  return m == (1 << 30) ? 0 : m;
}

}  // namespace ringsim
