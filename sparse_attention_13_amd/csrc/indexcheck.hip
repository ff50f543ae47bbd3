// sfa_validate_indices: a debug check of the top-K operator's sparseIndices (the operator
// page, section 3, requires every index to lie in [0, S2)).  It counts the slots whose index
// is outside that range and the index rows (b, s1, n2) that list some position twice (the
// kernels treat such a row's slots one by one, as the page's reference gather does).
//
// One workgroup per index row at a time: the row's indices are entered into an LDS bitmap of
// S2 bits with atomic ORs (a bit that was already set is a repeat), then cleared again by
// the same slots, so the bitmap is cleared once per workgroup, not once per row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sfa.h"
#include "topk_launch.hpp"

namespace {

constexpr int kCheckThreads = 256;
constexpr int kMaxBitmapBytes = 128 * 1024;  // S2 <= 1,048,576

struct CheckArgs {
  const int32_t* idx;
  int64_t st[3];  // element strides of (batch, query row, KV head) rows
  int B, S1, N2, topK, S2;
  int32_t* counts;  // [0] slots out of range, [1] rows with a repeated index
};

__global__ __launch_bounds__(kCheckThreads) void check_indices(CheckArgs a) {
  extern __shared__ uint32_t bits[];
  __shared__ int row_oob, row_dup;
  const int words = (a.S2 + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kCheckThreads) bits[w] = 0u;
  const int64_t rows = (int64_t)a.B * a.S1 * a.N2;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int n2 = (int)(r % a.N2);
    const int s1 = (int)((r / a.N2) % a.S1);
    const int b = (int)(r / ((int64_t)a.N2 * a.S1));
    const int32_t* row = a.idx + (int64_t)b * a.st[0] + (int64_t)s1 * a.st[1] + (int64_t)n2 * a.st[2];
    if (threadIdx.x == 0) {
      row_oob = 0;
      row_dup = 0;
    }
    __syncthreads();  // bitmap clear and row counters visible
    int oob = 0, dup = 0;
    for (int i = threadIdx.x; i < a.topK; i += kCheckThreads) {
      const int j = row[i];
      if (j < 0 || j >= a.S2) {
        ++oob;
        continue;
      }
      const uint32_t bit = 1u << (j & 31);
      if (atomicOr(&bits[j >> 5], bit) & bit) dup = 1;
    }
    if (oob) atomicAdd(&row_oob, oob);
    if (dup) atomicOr(&row_dup, 1);
    __syncthreads();  // every slot entered
    for (int i = threadIdx.x; i < a.topK; i += kCheckThreads) {
      const int j = row[i];
      if (j >= 0 && j < a.S2) bits[j >> 5] = 0u;
    }
    if (threadIdx.x == 0) {
      if (row_oob) atomicAdd(&a.counts[0], row_oob);
      if (row_dup) atomicAdd(&a.counts[1], 1);
    }
    __syncthreads();  // bitmap clear before the next row
  }
}

}  // namespace

extern "C" sfa_status sfa_validate_indices(const sfa_shape* shape, const sfa_strides* strides, sfa_layout layout,
                                           const int32_t* sparse_indices, int32_t* counts, hipStream_t stream) {
  if (!shape) return SFA_ERR_NULL;
  if (layout != SFA_BSND && layout != SFA_BNSD) return SFA_ERR_LAYOUT;
  if (shape->B < 0 || shape->S1 < 0 || shape->S2 < 1 || shape->N2 < 1) return SFA_ERR_SHAPE;
  if (shape->topK < 1 || shape->topK > shape->S2) return SFA_ERR_TOPK;
  if (!counts) return SFA_ERR_NULL;
  if ((int64_t)(shape->S2 + 31) / 32 * 4 > kMaxBitmapBytes) return SFA_ERR_UNSUPPORTED;
  CheckArgs a;
  a.idx = sparse_indices;
  a.B = shape->B;
  a.S1 = shape->S1;
  a.N2 = shape->N2;
  a.topK = shape->topK;
  a.S2 = shape->S2;
  a.counts = counts;
  // layout-order strides of the index tensor, or contiguous ones; canonical (b, s1, n2) order
  int64_t lo[3];
  if (strides) {
    for (int i = 0; i < 3; ++i) lo[i] = strides->idx[i];
  } else if (layout == SFA_BSND) {
    lo[2] = shape->topK; lo[1] = (int64_t)shape->N2 * shape->topK; lo[0] = (int64_t)shape->S1 * lo[1];
  } else {
    lo[2] = shape->topK; lo[1] = (int64_t)shape->S1 * shape->topK; lo[0] = (int64_t)shape->N2 * lo[1];
  }
  for (int i = 0; i < 3; ++i)
    if (lo[i] < 0) return SFA_ERR_LAYOUT;
  a.st[0] = lo[0];
  a.st[1] = layout == SFA_BSND ? lo[1] : lo[2];
  a.st[2] = layout == SFA_BSND ? lo[2] : lo[1];
  if (hipMemsetAsync(counts, 0, 2 * sizeof(int32_t), stream) != hipSuccess) return SFA_ERR_HIP;
  const int64_t rows = (int64_t)shape->B * shape->S1 * shape->N2;
  if (rows == 0) return SFA_OK;
  if (!sparse_indices) return SFA_ERR_NULL;
  const int lds = (shape->S2 + 31) / 32 * 4;
  if (sfa::ensure_lds_limit((const void*)check_indices, kMaxBitmapBytes) != hipSuccess) return SFA_ERR_HIP;
  const int64_t cap = (int64_t)sfa::device_cu_count() * 4;
  const int grid = (int)(rows < cap ? rows : cap);
  hipLaunchKernelGGL(check_indices, dim3(grid), dim3(kCheckThreads), lds, stream, a);
  return hipGetLastError() == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}
