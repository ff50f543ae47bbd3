// Host-side launch configuration of the top-K kernels (shared by the
// instantiation units and the C-ABI entry points).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_kernel.hpp"

namespace sfa {

enum class Dt { f16 = 0, bf16 = 1 };

// Largest slot-parallel wave count (<= 4/WH) whose staged buffers fit in LDS.
constexpr int topk_ws_for(int DK, int DV, bool alias, int WH) {
  for (int ws = 4 / WH; ws >= 1; ws /= 2) {
    const int ch = 32 * ws;
    const int kbuf = ch * DK * 2;
    const int vbuf = alias ? 0 : ch * DV * 2;
    const int lds = 2 * (kbuf + vbuf) + kMaxSplitLen * 4;
    const bool merge_ok = ws == 1 || ws * WH * 16 * (DV + 2) * 4 <= 2 * (kbuf + vbuf);
    if (lds <= 160 * 1024 && merge_ok) return ws;
  }
  return 0;
}

struct TopkLaunch {
  int WH, WS;
  int grid;
  int threads;
  int lds_bytes;
};

// Launches topk_fwd (and topk_merge when nsplit > 1) for one (dtype, Dk, Dv, alias, WH).
// Returns hipErrorInvalidValue when no kernel is compiled for that combination.
hipError_t launch_topk_f16(int DK, int DV, bool alias, int WH, const TopkParams& p, int grid,
                           int64_t nrows, hipStream_t s, bool* found);
hipError_t launch_topk_bf16(int DK, int DV, bool alias, int WH, const TopkParams& p, int grid,
                            int64_t nrows, hipStream_t s, bool* found);

template <typename T, int DK, int DV, bool ALIAS, int WH>
hipError_t launch_topk_one(const TopkParams& p, int grid, int64_t nrows, hipStream_t s) {
  constexpr int WS = topk_ws_for(DK, DV, ALIAS, WH);
  static_assert(WS >= 1, "no configuration fits");
  using C = TopkCfg<T, DK, DV, ALIAS, WH, WS>;
  auto kern = topk_fwd<T, DK, DV, ALIAS, WH, WS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), C::LDS_BYTES, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nsplit > 1) {
    constexpr int PER_ROW = DV / 4;
    const int64_t threads = nrows * PER_ROW;
    const int mgrid = (int)((threads + 255) / 256);
    hipLaunchKernelGGL((topk_merge<T, DV>), dim3(mgrid), dim3(256), 0, s, p, nrows);
    e = hipGetLastError();
  }
  return e;
}

// Head-dim pairs with a compiled kernel.
#define SFA_TOPK_DIMS(X) \
  X(64, 64)              \
  X(128, 128)            \
  X(192, 128)            \
  X(192, 192)            \
  X(256, 256)            \
  X(512, 512)            \
  X(576, 512)

inline bool topk_dims_supported(int DK, int DV) {
#define SFA_CHECK_DIMS(a, b) \
  if (DK == a && DV == b) return true;
  SFA_TOPK_DIMS(SFA_CHECK_DIMS)
#undef SFA_CHECK_DIMS
  return false;
}

inline int topk_ws_runtime(int DK, int DV, bool alias, int WH) { return topk_ws_for(DK, DV, alias, WH); }

}  // namespace sfa
