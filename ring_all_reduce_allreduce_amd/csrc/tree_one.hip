// tree_one.hip -- instantiations of the double-binary-tree kernel for
// slices of at most one line per thread (small messages).
#include "tree_flag.h"

namespace ringsim {

namespace {

template <int DT>
hipError_t tree_dispatch_op(const TreeArgs& a, int op, hipStream_t s) {
  const int grid = a.nranks * 2 * a.nchannels * 2;
  switch (op) {
    case RINGSIM_SUM: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_SUM, true>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_PROD: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_PROD, true>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MAX: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_MAX, true>), dim3(grid), dim3(kThreads), 0, s, a); break;
    case RINGSIM_MIN: hipLaunchKernelGGL((tree_flag_kernel<DT, RINGSIM_MIN, true>), dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_one(const TreeArgs& a, int dtype, int op, hipStream_t s) {
  switch (dtype) {
    case RINGSIM_INT32: return tree_dispatch_op<RINGSIM_INT32>(a, op, s);
    case RINGSIM_INT64: return tree_dispatch_op<RINGSIM_INT64>(a, op, s);
    case RINGSIM_FLOAT32: return tree_dispatch_op<RINGSIM_FLOAT32>(a, op, s);
    case RINGSIM_BFLOAT16: return tree_dispatch_op<RINGSIM_BFLOAT16>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

int tree_one_blocks_per_cu() {
  int m = 1 << 30;
  auto acc = [&](int v) { m = v < m ? v : m; };
#define RS_TREE_OCC_DT(DT)                                         \
  acc(occupancy(tree_flag_kernel<DT, RINGSIM_SUM, true>, 0));      \
  acc(occupancy(tree_flag_kernel<DT, RINGSIM_PROD, true>, 0));     \
  acc(occupancy(tree_flag_kernel<DT, RINGSIM_MAX, true>, 0));      \
  acc(occupancy(tree_flag_kernel<DT, RINGSIM_MIN, true>, 0));
  RS_TREE_OCC_DT(RINGSIM_INT32)
  RS_TREE_OCC_DT(RINGSIM_INT64)
  RS_TREE_OCC_DT(RINGSIM_FLOAT32)
  RS_TREE_OCC_DT(RINGSIM_BFLOAT16)
#undef RS_TREE_OCC_DT
  return m == (1 << 30) ? 0 : m;
}

}  // namespace ringsim
