// BSR plan / run entry points (flashinfer.sparse, BlockSparseAttentionWrapper:
// plan() validates and stages the block pattern once, run() may then be called
// repeatedly) and the instantiations of the block-sparse kernel.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "../../include/sfa.h"
#include "bsr_kernel.hpp"

struct bsr_plan_t {
  int M, N, R, C, Hq, Hkv, D, causal, MB, NB, nnz;
  sfa_dtype dtype;
  float scale;
  int32_t* d_indptr;
  int32_t* d_indices;
  int32_t* d_order;
  int32_t* pinned;  // host staging of the async copy; freed after the copy completes
  hipEvent_t copied;
};

namespace {

constexpr int kNQ128 = 2;  // query tiles per wave for D <= 128
constexpr int kNQ256 = 1;

size_t int_bytes(int MB, int nnz) { return ((size_t)(MB + 1) + (size_t)nnz + (size_t)MB) * 4 + 256; }

template <typename T, int D, int NQ>
hipError_t launch_bsr(const sfa::BsrParams& p, hipStream_t s) {
  using C = sfa::BsrCfg<T, D, NQ>;
  auto kern = sfa::bsr_fwd<T, D, NQ>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(p.n_items), dim3(C::NT), C::LDS_BYTES, s, p);
  return hipGetLastError();
}

int nq_for(int D) { return D <= 128 ? kNQ128 : kNQ256; }

}  // namespace

extern "C" {

size_t bsr_plan_int_bytes(int M, int N, int R, int C, int num_qo_heads, int num_kv_heads, int nnz) {
  (void)N; (void)C; (void)num_qo_heads; (void)num_kv_heads;
  if (M < 0 || R < 1 || nnz < 0) return 0;
  const int MB = (M + R - 1) / R;
  return int_bytes(MB, nnz);
}

sfa_status bsr_plan(bsr_plan_t** plan, const int32_t* indptr, const int32_t* indices, int M, int N, int R, int C,
                    int num_qo_heads, int num_kv_heads, int head_dim, int causal, float sm_scale, sfa_dtype dtype,
                    void* int_workspace, size_t int_workspace_bytes, hipStream_t stream) {
  if (!plan || !indptr) return SFA_ERR_NULL;
  *plan = nullptr;
  if (dtype != SFA_FP16 && dtype != SFA_BF16) return SFA_ERR_DTYPE;
  if (M < 0 || N < 1 || R < 1 || C < 1 || num_qo_heads < 1 || num_kv_heads < 1) return SFA_ERR_SHAPE;
  if (N % C != 0) return SFA_ERR_SHAPE;
  if (num_qo_heads % num_kv_heads != 0) return SFA_ERR_GQA;
  if (head_dim < 64 || head_dim % 64) return SFA_ERR_HEAD_DIM;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return SFA_ERR_UNSUPPORTED;
  if (causal && M > N) return SFA_ERR_CAUSAL;
  if (!isfinite(sm_scale)) return SFA_ERR_SCALE;
  const int MB = (M + R - 1) / R, NB = N / C;
  if (indptr[0] != 0) return SFA_ERR_PLAN;
  for (int i = 0; i < MB; ++i)
    if (indptr[i + 1] < indptr[i]) return SFA_ERR_PLAN;
  const int nnz = indptr[MB];
  if (nnz > 0 && !indices) return SFA_ERR_NULL;
  std::vector<int> seen(NB, -1);
  for (int i = 0; i < MB; ++i) {
    if (indptr[i + 1] - indptr[i] > sfa::kBsrMaxBlocks) return SFA_ERR_UNSUPPORTED;
    for (int t = indptr[i]; t < indptr[i + 1]; ++t) {
      const int c = indices[t];
      if (c < 0 || c >= NB || seen[c] == i) return SFA_ERR_INDEX;
      seen[c] = i;
    }
  }
  const int G = num_qo_heads / num_kv_heads;
  const int64_t qv = (int64_t)R * G;
  const int64_t qt = (qv + 64 * nq_for(head_dim) - 1) / (64 * nq_for(head_dim));
  const int64_t items = (int64_t)num_kv_heads * MB * qt;
  if (items > 0x7fffffffLL || (int64_t)R * G > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;
  const size_t need = int_bytes(MB, nnz);
  if (!int_workspace || int_workspace_bytes < need) return SFA_ERR_WORKSPACE;

  // block rows, longest key list first (simple load balancing of the grid)
  std::vector<int32_t> order(MB);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return indptr[a + 1] - indptr[a] > indptr[b + 1] - indptr[b];
  });

  bsr_plan_t* pl = (bsr_plan_t*)calloc(1, sizeof(bsr_plan_t));
  if (!pl) return SFA_ERR_HIP;
  const size_t n_ints = (size_t)(MB + 1) + nnz + MB;
  if (hipHostMalloc((void**)&pl->pinned, n_ints * 4, hipHostMallocDefault) != hipSuccess) {
    free(pl);
    return SFA_ERR_HIP;
  }
  memcpy(pl->pinned, indptr, (size_t)(MB + 1) * 4);
  if (nnz) memcpy(pl->pinned + MB + 1, indices, (size_t)nnz * 4);
  memcpy(pl->pinned + MB + 1 + nnz, order.data(), (size_t)MB * 4);
  int32_t* base = (int32_t*)(((uintptr_t)int_workspace + 255) & ~(uintptr_t)255);
  pl->d_indptr = base;
  pl->d_indices = base + MB + 1;
  pl->d_order = base + MB + 1 + nnz;
  if (hipEventCreateWithFlags(&pl->copied, hipEventDisableTiming) != hipSuccess ||
      hipMemcpyAsync(base, pl->pinned, n_ints * 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(pl->copied, stream) != hipSuccess) {
    (void)hipHostFree(pl->pinned);
    free(pl);
    return SFA_ERR_HIP;
  }
  pl->M = M; pl->N = N; pl->R = R; pl->C = C;
  pl->Hq = num_qo_heads; pl->Hkv = num_kv_heads; pl->D = head_dim;
  pl->causal = causal ? 1 : 0;
  pl->MB = MB; pl->NB = NB; pl->nnz = nnz;
  pl->dtype = dtype;
  pl->scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)head_dim));
  *plan = pl;
  return SFA_OK;
}

sfa_status bsr_run(const bsr_plan_t* pl, const void* q, const void* k, const void* v, void* out, float* lse,
                   hipStream_t stream) {
  if (!pl) return SFA_ERR_PLAN;
  if (pl->M == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if (mis & 15u) return SFA_ERR_LAYOUT;
  sfa::BsrParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.indptr = pl->d_indptr;
  p.indices = pl->d_indices;
  p.order = pl->d_order;
  p.M = pl->M; p.N = pl->N; p.R = pl->R; p.C = pl->C;
  p.Hq = pl->Hq; p.Hkv = pl->Hkv; p.G = pl->Hq / pl->Hkv;
  p.causal = pl->causal;
  p.scale_log2 = (float)((double)pl->scale * 1.4426950408889634);
  p.MB = pl->MB;
  p.QV = pl->R * p.G;
  const int nq = nq_for(pl->D);
  p.QT = (p.QV + 64 * nq - 1) / (64 * nq);
  p.n_items = pl->Hkv * pl->MB * p.QT;
  if (p.n_items == 0) return SFA_OK;
  hipError_t e;
  const bool f16 = pl->dtype == SFA_FP16;
  switch (pl->D) {
    case 64:
      e = f16 ? launch_bsr<sfa::half_t, 64, kNQ128>(p, stream) : launch_bsr<sfa::bfloat_t, 64, kNQ128>(p, stream);
      break;
    case 128:
      e = f16 ? launch_bsr<sfa::half_t, 128, kNQ128>(p, stream) : launch_bsr<sfa::bfloat_t, 128, kNQ128>(p, stream);
      break;
    case 256:
      e = f16 ? launch_bsr<sfa::half_t, 256, kNQ256>(p, stream) : launch_bsr<sfa::bfloat_t, 256, kNQ256>(p, stream);
      break;
    default:
      return SFA_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

sfa_status bsr_destroy(bsr_plan_t* pl) {
  if (!pl) return SFA_OK;
  if (pl->copied) {
    (void)hipEventSynchronize(pl->copied);  // the staging buffer feeds an async copy
    (void)hipEventDestroy(pl->copied);
  }
  if (pl->pinned) (void)hipHostFree(pl->pinned);
  free(pl);
  return SFA_OK;
}

}  // extern "C"
