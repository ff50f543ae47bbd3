// Host-side launch configuration of the top-K kernels (shared by the
// instantiation units and the C-ABI entry points).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_kernel.hpp"

namespace sfa {

inline int topk_ws_for(int DK, int DV, bool alias, int MT, int WH) { return topk_pick(DK, DV, alias, MT, WH) / 16; }

// Head tile (MFMA N dim) and head tiles per workgroup for G query heads per KV head:
// 32-wide tiles (32x32x16 MFMA, half the LDS operand traffic per flop) whenever the
// staged buffers fit in LDS, else 16-wide tiles.
struct HeadTiling {
  int MT, WH;
};
inline HeadTiling head_tiling(int G, int DK, int DV, bool alias) {
  if (G <= 16) return {16, 1};
  const int wh32 = G <= 32 ? 1 : (G <= 64 ? 2 : 4);
  if (topk_pick(DK, DV, alias, 32, wh32) > 0) return {32, wh32};
  return {16, G <= 32 ? 2 : 4};
}

// Workgroups of this configuration that fit on one CU by LDS.
inline int topk_wgs_per_cu(int DK, int DV, bool alias, int MT, int WH) {
  const int pick = topk_pick(DK, DV, alias, MT, WH);
  if (pick == 0) return 1;
  const int ws = pick / 16, nbuf = pick % 16;
  const int lds = nbuf * topk_chunk_bytes(DK, DV, alias, ws) + topk_qlds_bytes(DK, DV, MT, WH) + kIdxReserve;
  const int n = (160 * 1024) / lds;
  return n > 0 ? n : 1;
}

// Largest index-slot count per work item that fits next to the ring in LDS.
inline int topk_max_split_len(int DK, int DV, bool alias, int MT, int WH) {
  const int pick = topk_pick(DK, DV, alias, MT, WH);
  if (pick == 0) return 0;
  const int ws = pick / 16, nbuf = pick % 16;
  const int fixed = nbuf * topk_chunk_bytes(DK, DV, alias, ws) + topk_qlds_bytes(DK, DV, MT, WH);
  int len = (160 * 1024 - fixed) / 4;
  len = len / (32 * ws) * (32 * ws);
  return len < kMaxSplitLen ? len : kMaxSplitLen;
}

// Launches topk_fwd (and topk_merge when nsplit > 1) for one (dtype, Dk, Dv, alias, MT, WH).
// *found is false when no kernel is compiled for that combination.
hipError_t launch_topk_f16_alias(int DK, int DV, int MT, int WH, const TopkParams& p, int grid, int64_t nrows,
                                 hipStream_t s, bool* found);
hipError_t launch_topk_f16_sep(int DK, int DV, int MT, int WH, const TopkParams& p, int grid, int64_t nrows,
                               hipStream_t s, bool* found);
hipError_t launch_topk_bf16_alias(int DK, int DV, int MT, int WH, const TopkParams& p, int grid, int64_t nrows,
                                  hipStream_t s, bool* found);
hipError_t launch_topk_bf16_sep(int DK, int DV, int MT, int WH, const TopkParams& p, int grid, int64_t nrows,
                                hipStream_t s, bool* found);

template <typename T, int DK, int DV, bool ALIAS, int MT, int WH>
hipError_t launch_topk_one(const TopkParams& p, int grid, int64_t nrows, hipStream_t s) {
  constexpr int PICK = topk_pick(DK, DV, ALIAS, MT, WH);
  constexpr int WS = PICK / 16, NBUF = PICK % 16;
  if constexpr (PICK == 0) {
    return hipErrorInvalidValue;  // never selected by head_tiling
  } else {
  using C = TopkCfg<T, DK, DV, ALIAS, MT, WH, WS, NBUF>;
  auto kern = topk_fwd<T, DK, DV, ALIAS, MT, WH, WS, NBUF>;
  constexpr int kMaxLds = 160 * 1024;
  // the dynamic-LDS limit is a property of the function: set it once per process
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
  hipError_t e = attr;
  if (e != hipSuccess) return e;
  const int lds = C::LDS_FIXED + ((p.split_len * 4 + 15) & ~15);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, s, p);
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

}  // namespace sfa
