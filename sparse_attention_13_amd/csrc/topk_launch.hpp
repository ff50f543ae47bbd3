// Host-side launch configuration of the top-K kernels (shared by the
// instantiation units and the C-ABI entry points).
#pragma once

#include <mutex>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_dvs.hpp"

namespace sfa {

// Raises a kernel's dynamic-LDS limit to `bytes`, once per (kernel, device): the limit is a
// per-device property of the function.  Thread-safe; later calls take a lock and a short scan.
inline hipError_t ensure_lds_limit(const void* kern, int bytes) {
  struct Done { const void* kern; int dev; };
  static std::mutex mu;
  static Done done[256];
  static int n = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (done[i].kern == kern && done[i].dev == dev) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && n < 256) done[n++] = Done{kern, dev};
  return e;
}


// MT == kDvsHeads selects topk_fwd_dvs (64 query vectors per 8-wave workgroup, one chunk of
// 32 slots at a time); other MT values select topk_fwd with MT-wide head tiles.
inline int topk_ws_for(int DK, int DV, bool alias, int MT, int WH, bool wide) {
  if (MT == kDvsHeads) return dvs_supported(DK, DV, alias) ? 1 : 0;
  return topk_pick(DK, DV, alias, MT, WH, wide) / 16;
}

// Head tile (MFMA N dim) and head tiles per workgroup for G query heads per KV head:
// 32-wide tiles (32x32x16 MFMA, half the LDS operand traffic per flop) whenever the
// staged buffers fit in LDS, else 16-wide tiles.
struct HeadTiling {
  int MT, WH;
};
inline HeadTiling head_tiling(int G, int DK, int DV, bool alias) {
  // up to 8 query vectors: the packed 16-wide tile (both slot groups of a 32-slot part side by
  // side), which keeps its two copies of Q^T in registers up to Dk = 256
  if (G <= 8 && DK <= 256) return {8, 1};
  if (G <= 16) return {16, 1};
  // 32-wide head tiles hold 32 x DV fp32 accumulators per wave: past DV = 256 they leave too
  // few registers for the rest (spills).  Wide value heads with many query vectors split the
  // PV product over dv instead (topk_fwd_dvs); with few, 16-wide head tiles.
  if (DV > 256) {
    if (G > 32 && dvs_supported(DK, DV, alias)) return {kDvsHeads, 1};
    return {16, G <= 32 ? 2 : 4};
  }
  // up to 8 waves of 32 heads: past 128 heads (block-sparse rows) two waves share each SIMD,
  // which leaves room for the accumulators of Dv <= 128 only
  const int wh32 = G <= 32 ? 1 : (G <= 64 ? 2 : (G <= 128 || DV > 128 ? 4 : 8));
  if (topk_pick(DK, DV, alias, 32, wh32, false) > 0) return {32, wh32};
  return {16, G <= 32 ? 2 : 4};
}

// Resident workgroups per CU of the f16 topk_fwd kernel for (Dk, Dv, alias, MT, WH, wide), from
// the runtime's occupancy calculator (registers, LDS and waves of the compiled kernel); 0 when
// it cannot tell (no such kernel, no device).
int occupancy_topk_f16_alias(int DK, int DV, int MT, int WH, bool wide);
int occupancy_topk_f16_sep(int DK, int DV, int MT, int WH, bool wide);

// Resident workgroups per CU of the compiled kernel (occupancy_topk_f16_*), cached per device
// and configuration; 0 when unknown.  The f16 kernel stands for both 16-bit types (the bf16
// instantiations differ by a few registers at most), so that a plan does not depend on the dtype.
inline int topk_kernel_occupancy(int DK, int DV, bool alias, int MT, int WH, bool wide) {
  struct Entry { int dev, DK, DV, MT, WH, alias, wide, n; };
  static std::mutex mu;
  static Entry cache[128];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i) {
    const Entry& e = cache[i];
    if (e.dev == dev && e.DK == DK && e.DV == DV && e.MT == MT && e.WH == WH && e.alias == (int)alias &&
        e.wide == (int)wide)
      return e.n;
  }
  const int n = alias ? occupancy_topk_f16_alias(DK, DV, MT, WH, wide) : occupancy_topk_f16_sep(DK, DV, MT, WH, wide);
  if (used < 128) cache[used++] = Entry{dev, DK, DV, MT, WH, (int)alias, (int)wide, n};
  return n;
}

// Workgroups of this configuration that fit on one CU: by LDS, and by the compiled kernel's
// registers where the runtime can tell (an 8-wave workgroup at two waves per SIMD is alone on its
// CU whatever LDS it leaves free).
inline int topk_wgs_per_cu(int DK, int DV, bool alias, int MT, int WH, bool wide) {
  if (MT == kDvsHeads) return 1;
  const int pick = topk_pick(DK, DV, alias, MT, WH, wide);
  if (pick == 0) return 1;
  const int ws = pick / 16, nbuf = pick % 16;
  const int lds = nbuf * topk_chunk_bytes(DK, DV, alias, ws, MT) + topk_qlds_bytes(DK, DV, MT, WH) + kIdxReserve;
  int n = (160 * 1024) / lds;
  const int occ = topk_kernel_occupancy(DK, DV, alias, MT, WH, wide);
  if (occ > 0 && occ < n) n = occ;
  return n > 0 ? n : 1;
}

// Largest index-slot count per work item that fits next to the ring in LDS.
inline int topk_max_split_len(int DK, int DV, bool alias, int MT, int WH, bool wide) {
  if (MT == kDvsHeads) return dvs_max_split_len(DK, DV, alias);
  const int pick = topk_pick(DK, DV, alias, MT, WH, wide);
  if (pick == 0) return 0;
  const int ws = pick / 16, nbuf = pick % 16;
  const int fixed = nbuf * topk_chunk_bytes(DK, DV, alias, ws, MT) + topk_qlds_bytes(DK, DV, MT, WH) + kTopkFlagBytes;
  int len = (160 * 1024 - fixed) / 4;
  len = len / (32 * ws) * (32 * ws);
  return len < kTopkMaxSplitLen ? len : kTopkMaxSplitLen;
}

// Launches topk_fwd (and topk_merge when nsplit > 1) for one (dtype, Dk, Dv, alias, MT, WH).
// *found is false when no kernel is compiled for that combination.
hipError_t launch_topk_f16_alias(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid, int64_t nrows,
                                 hipStream_t s, bool* found);
hipError_t launch_topk_f16_sep(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid, int64_t nrows,
                               hipStream_t s, bool* found);
hipError_t launch_topk_bf16_alias(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid, int64_t nrows,
                                  hipStream_t s, bool* found);
hipError_t launch_topk_bf16_sep(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid, int64_t nrows,
                                hipStream_t s, bool* found);
// fp16 kernels that apply per-head logit factors (launches with p.fq or p.fk set)
hipError_t launch_topk_f16_alias_hf(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid,
                                    int64_t nrows, hipStream_t s, bool* found);
hipError_t launch_topk_f16_sep_hf(int DK, int DV, int MT, int WH, bool wide, const TopkParams& p, int grid,
                                  int64_t nrows, hipStream_t s, bool* found);

template <typename T, int DV>
hipError_t launch_topk_merge(const TopkParams& p, int64_t nrows, hipStream_t s) {
  constexpr int PER_ROW = DV / 8;
  const int64_t threads = nrows * PER_ROW;
  const int mgrid = (int)((threads + 255) / 256);
  hipLaunchKernelGGL((topk_merge<T, DV>), dim3(mgrid), dim3(256), 0, s, p, nrows);
  return hipGetLastError();
}

template <typename T, int DK, int DV, bool ALIAS>
hipError_t launch_dvs_one(const TopkParams& p, int grid, int64_t nrows, hipStream_t s) {
  if constexpr (!dvs_supported(DK, DV, ALIAS) || DV <= 256) {
    return hipErrorInvalidValue;  // never selected by head_tiling
  } else {
    constexpr int NBUF = dvs_nbuf(DK, DV, ALIAS);
    using C = DvsCfg<T, DK, DV, ALIAS, NBUF>;
    auto kern = topk_fwd_dvs<T, DK, DV, ALIAS, NBUF>;
    constexpr int kMaxLds = 160 * 1024;
    hipError_t e = ensure_lds_limit((const void*)kern, kMaxLds);
    if (e != hipSuccess) return e;
    const int lds = C::LDS_FIXED + ((p.split_len * 4 + 15) & ~15);
    if (lds > kMaxLds || p.HB * kDvsHeads < p.G) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return p.nsplit > 1 ? launch_topk_merge<T, DV>(p, nrows, s) : hipSuccess;
  }
}

// Workgroups per CU of one topk_fwd instantiation at the LDS the planner assumes (ring, Q^T,
// flags and kIdxReserve bytes of index slots); 0 when unknown.
template <typename T, int DK, int DV, bool ALIAS, int MT, int WH, bool WIDE>
int occupancy_topk_one() {
  if constexpr (MT == kDvsHeads) {
    return 1;
  } else {
    constexpr int PICK = topk_pick(DK, DV, ALIAS, MT, WH, WIDE);
    constexpr int WS = PICK / 16, NBUF = PICK % 16;
    if constexpr (PICK == 0 || (MT == 32 && DV > 256) || (WH == 8 && (MT != 32 || DV > 128)) ||
                  (MT == 8 && (WH != 1 || DK > 256))) {
      return 0;
    } else {
      using C = TopkCfg<T, DK, DV, ALIAS, MT, WH, WS, NBUF>;
      const void* kern = (const void*)topk_fwd<T, DK, DV, ALIAS, MT, WH, WS, NBUF, false>;
      if (ensure_lds_limit(kern, 160 * 1024) != hipSuccess) return 0;
      int n = 0;
      const size_t lds = (size_t)(C::LDS_FIXED - kTopkFlagBytes + kIdxReserve);
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, C::NT, lds) != hipSuccess) return 0;
      return n;
    }
  }
}

template <typename T, int DK, int DV, bool ALIAS, int MT, int WH, bool WIDE, bool HF = false>
hipError_t launch_topk_one(const TopkParams& p, int grid, int64_t nrows, hipStream_t s) {
  if constexpr (MT == kDvsHeads) {
    static_assert(WH == 1, "one 64-vector block per workgroup");
    return launch_dvs_one<T, DK, DV, ALIAS>(p, grid, nrows, s);
  } else {
  constexpr int PICK = topk_pick(DK, DV, ALIAS, MT, WH, WIDE);
  constexpr int WS = PICK / 16, NBUF = PICK % 16;
  if constexpr (PICK == 0 || (MT == 32 && DV > 256) || (WH == 8 && (MT != 32 || DV > 128)) ||
                (MT == 8 && (WH != 1 || DK > 256))) {
    return hipErrorInvalidValue;  // never selected by head_tiling
  } else {
  using C = TopkCfg<T, DK, DV, ALIAS, MT, WH, WS, NBUF>;
  auto kern = topk_fwd<T, DK, DV, ALIAS, MT, WH, WS, NBUF, HF>;
  constexpr int kMaxLds = 160 * 1024;
  hipError_t e = ensure_lds_limit((const void*)kern, kMaxLds);
  if (e != hipSuccess) return e;
  const int lds = C::LDS_FIXED + ((p.split_len * 4 + 15) & ~15) + (p.bm_words ? C::MASK_BYTES : 0);
  if (lds > kMaxLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return p.nsplit > 1 ? launch_topk_merge<T, DV>(p, nrows, s) : hipSuccess;
  }
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
  X(576, 512)            \
  X(576, 576)

// Launch plan of one call: head tiling, workgroup shape, topK split.
struct TopkPlan {
  int MT, WH, WS, HB, nsplit, split_len, grid;
  bool wide;        // single-wave workgroups with a two-chunk ring (topk_pick)
  int64_t rows;     // query vectors (rows of the split workspace)
  size_t ws_bytes;  // float workspace for split partials (0 when nsplit == 1)
};

// Plans `items` index lists of at most max_slots slots, each shared by G query vectors
// (virtual heads), on a device with `cus` compute units.  WS == 0: nothing fits.  ragged: the
// lists have different lengths (block-sparse rows); every item takes only the splits its own
// list needs, so when the longest lists alone force a split the splits are made as long as
// allowed and the other lists stay whole.
inline TopkPlan plan_topk(int64_t items, int G, int max_slots, int DK, int DV, bool alias, int cus,
                          bool ragged = false) {
  TopkPlan pl{};
  const HeadTiling ht = head_tiling(G, DK, DV, alias);
  pl.MT = ht.MT;
  pl.WH = ht.WH;
  // many more work items than CUs: single-wave workgroups, as many per CU as LDS allows
  pl.wide = false;
  if ((pl.MT == 16 || pl.MT == 8) && pl.WH == 1) {
    const int wgs = topk_wgs_per_cu(DK, DV, alias, pl.MT, 1, true);
    pl.wide = topk_pick(DK, DV, alias, pl.MT, 1, true) > 0 && items >= 2 * (int64_t)cus * wgs;
  }
  pl.WS = topk_ws_for(DK, DV, alias, pl.MT, pl.WH, pl.wide);
  pl.HB = (G + pl.MT * pl.WH - 1) / (pl.MT * pl.WH);
  const int ch = 32 * (pl.WS > 0 ? pl.WS : 1);
  const int64_t base = items * pl.HB;
  // one full wave of resident workgroups; splitting further only adds partial traffic
  const int64_t target = (int64_t)cus * topk_wgs_per_cu(DK, DV, alias, pl.MT, pl.WH, pl.wide);
  int nsplit = 1;
  if (base > 0 && base < target) nsplit = (int)((target + base - 1) / base);
  const int slots = max_slots > 0 ? max_slots : 1;
  const int max_split = (slots + ch - 1) / ch;
  if (nsplit > max_split) nsplit = max_split;
  const int max_len = topk_max_split_len(DK, DV, alias, pl.MT, pl.WH, pl.wide);
  if (max_len <= 0) {
    pl.WS = 0;
    return pl;
  }
  const int min_split = (slots + max_len - 1) / max_len;
  if (nsplit < min_split) nsplit = min_split;
  int len = (slots + nsplit - 1) / nsplit;
  len = (len + ch - 1) / ch * ch;
  if (ragged && nsplit == min_split && nsplit > 1) len = max_len / ch * ch;
  pl.split_len = len;
  pl.nsplit = (slots + len - 1) / len;
  pl.grid = (int)(base * pl.nsplit);
  pl.rows = items * G;
  pl.ws_bytes = pl.nsplit > 1 ? (size_t)pl.rows * pl.nsplit * ((size_t)DV + 2) * sizeof(float) + 256 : 0;
  return pl;
}

// Launches the kernels of a plan for (dtype, head dims, alias); *found is false when no
// kernel is compiled for that combination.
inline hipError_t launch_topk(bool f16, bool alias, int DK, int DV, const TopkPlan& pl, const TopkParams& p,
                              hipStream_t s, bool* found) {
  const bool hf = p.fq || p.fk || p.fv;
  if (hf && !f16) {
    *found = false;  // per-head factors come with FP8 inputs, which run in fp16
    return hipErrorInvalidValue;
  }
  auto fn = f16 ? (hf ? (alias ? launch_topk_f16_alias_hf : launch_topk_f16_sep_hf)
                      : (alias ? launch_topk_f16_alias : launch_topk_f16_sep))
                : (alias ? launch_topk_bf16_alias : launch_topk_bf16_sep);
  return fn(DK, DV, pl.MT, pl.WH, pl.wide, p, pl.grid, pl.rows, s, found);
}

// Compute units of the current device (cached per device; 256 if the query fails).
inline int device_cu_count() {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev] = {0};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDev && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDev) cached[dev] = cus;
  return cus;
}

// The gather addresses a row as base + row * pitch in 32 bits (24-bit multiply): rows and
// pitches below 2^24 and every row of a (b, kv head) slice within 4 GiB of the slice base.
inline bool topk_rows_addressable(int64_t rows, int64_t pitch_elems, int64_t row_elems) {
  if (rows < 1 || rows >= (1 << 24) || pitch_elems < 0 || pitch_elems * 2 >= (1 << 24)) return false;
  return ((rows - 1) * pitch_elems + row_elems) * 2 <= 0xffffffffLL;
}

// Compiled head-dim pair that serves a call with head dims (Dk, Dv) (multiples of 64, Dv <= Dk):
// the pair with the smallest DK >= Dk, then the smallest DV >= Dv.  The kernels take the call's
// dims at run time (q columns past Dk enter the products as zeros, output columns past Dv are
// not stored), so a pair serves every smaller one.  False when none is large enough.
inline bool topk_kernel_dims(int Dk, int Dv, int* DK, int* DV) {
  int bk = 0, bv = 0;
#define SFA_PICK_DIMS(a, b)                                                             \
  if (a >= Dk && b >= Dv && (bk == 0 || a < bk || (a == bk && b < bv))) {              \
    bk = a;                                                                             \
    bv = b;                                                                             \
  }
  SFA_TOPK_DIMS(SFA_PICK_DIMS)
#undef SFA_PICK_DIMS
  if (bk == 0) return false;
  *DK = bk;
  *DV = bv;
  return true;
}

}  // namespace sfa
