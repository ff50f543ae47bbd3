// Instantiations of the top-K kernels for f16 inputs.
#include "topk_launch.hpp"

namespace sfa {

hipError_t launch_topk_f16(int DK, int DV, bool alias, int WH, const TopkParams& p, int grid, int64_t nrows,
                           hipStream_t s, bool* found) {
  *found = true;
#define SFA_CASE(a, b)                                                          \
  if (DK == a && DV == b) {                                                     \
    if (alias) {                                                                \
      if (WH == 1) return launch_topk_one<half_t, a, b, true, 1>(p, grid, nrows, s);  \
      if (WH == 2) return launch_topk_one<half_t, a, b, true, 2>(p, grid, nrows, s);  \
      if (WH == 4) return launch_topk_one<half_t, a, b, true, 4>(p, grid, nrows, s);  \
    } else {                                                                    \
      if (WH == 1) return launch_topk_one<half_t, a, b, false, 1>(p, grid, nrows, s); \
      if (WH == 2) return launch_topk_one<half_t, a, b, false, 2>(p, grid, nrows, s); \
      if (WH == 4) return launch_topk_one<half_t, a, b, false, 4>(p, grid, nrows, s); \
    }                                                                           \
  }
  SFA_TOPK_DIMS(SFA_CASE)
#undef SFA_CASE
  *found = false;
  return hipErrorInvalidValue;
}

}  // namespace sfa
