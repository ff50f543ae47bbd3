// Instantiations of the top-K kernels: f16 inputs, value in its own rows.
#include "topk_launch.hpp"

namespace sfa {

hipError_t launch_topk_f16_sep(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid, int64_t nrows,
                              hipStream_t s, bool* found) {
  *found = true;
#define SFA_CASE(a, b)                                                                   \
  if (DK == a && DV == b) {                                                              \
    if (MT == 8 && WH == 1 && wide) return launch_topk_one<half_t, a, b, false, 8, 1, true>(p, grid, nrows, s); \
    if (MT == 8 && WH == 1) return launch_topk_one<half_t, a, b, false, 8, 1, false>(p, grid, nrows, s); \
    if (MT == 16 && WH == 1 && wide) return launch_topk_one<half_t, a, b, false, 16, 1, true>(p, grid, nrows, s); \
    if (MT == 16 && WH == 1) return launch_topk_one<half_t, a, b, false, 16, 1, false>(p, grid, nrows, s); \
    if (MT == 16 && WH == 2) return launch_topk_one<half_t, a, b, false, 16, 2, false>(p, grid, nrows, s); \
    if (MT == 16 && WH == 4) return launch_topk_one<half_t, a, b, false, 16, 4, false>(p, grid, nrows, s); \
    if (MT == 32 && WH == 1) return launch_topk_one<half_t, a, b, false, 32, 1, false>(p, grid, nrows, s); \
    if (MT == 32 && WH == 2) return launch_topk_one<half_t, a, b, false, 32, 2, false>(p, grid, nrows, s); \
    if (MT == 32 && WH == 4) return launch_topk_one<half_t, a, b, false, 32, 4, false>(p, grid, nrows, s); \
    if (MT == 32 && WH == 8) return launch_topk_one<half_t, a, b, false, 32, 8, false>(p, grid, nrows, s); \
    if (MT == 64 && WH == 1) return launch_topk_one<half_t, a, b, false, 64, 1, false>(p, grid, nrows, s); \
  }
  SFA_TOPK_DIMS(SFA_CASE)
#undef SFA_CASE
  *found = false;
  return hipErrorInvalidValue;
}

int occupancy_topk_f16_sep(int DK, int DV, int MT, int WH, bool wide) {
#define SFA_CASE(a, b)                                                                       \
  if (DK == a && DV == b) {                                                                  \
    if (MT == 8 && WH == 1 && wide) return occupancy_topk_one<half_t, a, b, false, 8, 1, true>();   \
    if (MT == 8 && WH == 1) return occupancy_topk_one<half_t, a, b, false, 8, 1, false>();          \
    if (MT == 16 && WH == 1 && wide) return occupancy_topk_one<half_t, a, b, false, 16, 1, true>(); \
    if (MT == 16 && WH == 1) return occupancy_topk_one<half_t, a, b, false, 16, 1, false>();        \
    if (MT == 16 && WH == 2) return occupancy_topk_one<half_t, a, b, false, 16, 2, false>();        \
    if (MT == 16 && WH == 4) return occupancy_topk_one<half_t, a, b, false, 16, 4, false>();        \
    if (MT == 32 && WH == 1) return occupancy_topk_one<half_t, a, b, false, 32, 1, false>();        \
    if (MT == 32 && WH == 2) return occupancy_topk_one<half_t, a, b, false, 32, 2, false>();        \
    if (MT == 32 && WH == 4) return occupancy_topk_one<half_t, a, b, false, 32, 4, false>();        \
    if (MT == 32 && WH == 8) return occupancy_topk_one<half_t, a, b, false, 32, 8, false>();        \
    if (MT == 64 && WH == 1) return occupancy_topk_one<half_t, a, b, false, 64, 1, false>();        \
  }
  SFA_TOPK_DIMS(SFA_CASE)
#undef SFA_CASE
  return 0;
}

}  // namespace sfa
