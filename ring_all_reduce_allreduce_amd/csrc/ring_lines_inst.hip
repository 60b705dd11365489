// ring_lines_inst.hip -- instantiations of the line-protocol ring kernel for
// one line mode, with its launcher and occupancy query. The build compiles
// this file once per mode, defining RINGSIM_LINE_MODE (kLinesHalf: steps of
// at most 128 lines, alternating the two workgroup halves; kLinesOne: at most
// 256 lines, one per thread; kLinesMulti: any step, several lines per thread)
// and RINGSIM_LINE_NAME (half, one, multi: the suffix of the two functions
// below, as declared in ringsim_internal.h). Each mode is a translation unit
// of its own, so that the modes compile in parallel and each kernel keeps its
// own register allocation.
#include "ring_lines.h"

#if !defined(RINGSIM_LINE_MODE) || !defined(RINGSIM_LINE_NAME)
#error "compile with -DRINGSIM_LINE_MODE=kLines{Half,One,Multi} -DRINGSIM_LINE_NAME={half,one,multi}"
#endif

#define RS_CAT2(a, b) a##b
#define RS_CAT(a, b) RS_CAT2(a, b)
#define RS_LAUNCH RS_CAT(launch_ring_lines_, RINGSIM_LINE_NAME)
#define RS_BLOCKS RS_CAT(RS_CAT(line_, RINGSIM_LINE_NAME), _blocks_per_cu)

namespace ringsim {

namespace {

constexpr int kMode = RINGSIM_LINE_MODE;

template <int LP>
struct LineLaunch {
  template <int DT, int OP, int MODE>
  static hipError_t run(const RingArgs& a, hipStream_t s) {
    const int grid = a.nranks * a.nchannels * a.wpc;
    hipLaunchKernelGGL((ring_line_kernel<LP, kMode, DT, OP, MODE>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
};

}  // namespace

hipError_t RS_LAUNCH(const RingArgs& a, int line_proto, int mode, int dtype, int op, hipStream_t s) {
  if (line_proto == kLineWide) return dispatch_ring<LineLaunch<kLineWide>>(a, mode, dtype, op, s);
  return dispatch_ring<LineLaunch<kLineFlag>>(a, mode, dtype, op, s);
}

int RS_BLOCKS() {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_OCC_LINE(LP, DT)                                                      \
  acc(occupancy(ring_line_kernel<LP, kMode, DT, RINGSIM_SUM, kAllReduce>, 0));     \
  acc(occupancy(ring_line_kernel<LP, kMode, DT, RINGSIM_MIN, kReduceScatter>, 0)); \
  acc(occupancy(ring_line_kernel<LP, kMode, DT, RINGSIM_SUM, kAllGather>, 0));
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
