// tree.hip -- instantiations and launch of the double-binary-tree kernel.
#include "tree_lines.h"

namespace ringsim {

namespace {

template <int DT>
hipError_t tree_dispatch_op(const TreeArgs& a, int op, hipStream_t s) {
  const int grid = a.nranks * 2 * a.nchannels * 2;
  switch (op) {
    case RINGSIM_SUM: hipLaunchKernelGGL((tree_line_kernel<DT, RINGSIM_SUM>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_PROD: hipLaunchKernelGGL((tree_line_kernel<DT, RINGSIM_PROD>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MAX: hipLaunchKernelGGL((tree_line_kernel<DT, RINGSIM_MAX>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MIN: hipLaunchKernelGGL((tree_line_kernel<DT, RINGSIM_MIN>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_kernel(const TreeArgs& a, int dtype, int op, hipStream_t s) {
  switch (dtype) {
    case RINGSIM_INT32: return tree_dispatch_op<RINGSIM_INT32>(a, op, s);
    case RINGSIM_INT64: return tree_dispatch_op<RINGSIM_INT64>(a, op, s);
    case RINGSIM_FLOAT32: return tree_dispatch_op<RINGSIM_FLOAT32>(a, op, s);
    case RINGSIM_BFLOAT16: return tree_dispatch_op<RINGSIM_BFLOAT16>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

int tree_blocks_per_cu() {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_TREE_OCC_DT(DT)                                         \
  acc(occupancy(tree_line_kernel<DT, RINGSIM_SUM>, 0));      \
  acc(occupancy(tree_line_kernel<DT, RINGSIM_PROD>, 0));     \
  acc(occupancy(tree_line_kernel<DT, RINGSIM_MAX>, 0));      \
  acc(occupancy(tree_line_kernel<DT, RINGSIM_MIN>, 0));
  RS_TREE_OCC_DT(RINGSIM_INT32)
  RS_TREE_OCC_DT(RINGSIM_INT64)
  RS_TREE_OCC_DT(RINGSIM_FLOAT32)
  RS_TREE_OCC_DT(RINGSIM_BFLOAT16)
#undef RS_TREE_OCC_DT
  return m == (1 << 30) ? 0 : m;
}

}  // namespace ringsim
