// BSR plan / run entry points (flashinfer.sparse, BlockSparseAttentionWrapper:
// plan() validates and stages the block pattern once, run() may then be called
// repeatedly).
//
// A block row of the BSR mask is a top-K problem in disguise: its R x (Hq / Hkv)
// query vectors of one KV head share one key list, the concatenated key rows of the
// row's stored blocks.  plan() expands the block list into that key list (CSR over
// block rows) and run() launches the top-K kernels with one work item per (block
// row, KV head): the "heads" of an item are its query vectors (query row
// br * R + h / G, query head hk * G + h % G), each with its own bottom-right causal
// limit.  Keys of a stored block are consecutive rows, so the gather stays coalesced.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/sfa.h"
#include "fp8.hpp"
#include "topk_launch.hpp"

struct bsr_plan_t {
  int M, N, R, C, Hq, Hkv, D, causal, MB, max_keys;
  int64_t nkeys;
  int64_t nwords;    // 32-slot mask words (0: no per-block mask)
  int32_t* d_wptr;   // [MB + 1] first mask word of each block row
  int32_t* d_wflag;  // [nwords] some bit of the word is clear
  uint32_t* d_words; // [nwords][R] mask bits per query row of the block row
  sfa_dtype dtype;
  float scale;
  int32_t* d_kptr;   // [MB + 1] key-list offsets of the block rows
  int32_t* d_keys;   // [nkeys] key rows
  float* d_split;    // split partials (may be unused)
  size_t split_bytes;
  int32_t* pinned;   // host staging of the async copy; freed with the plan
  hipEvent_t copied;
};

namespace {

// Head dim of the compiled kernels that serve head dim D (0: none); the kernels take D itself
// at run time.
int kernel_dim(int D) {
  int DK = 0, DV = 0;
  return sfa::topk_kernel_dims(D, D, &DK, &DV) && DK == DV ? DK : 0;
}

// Device bytes of a plan: key list + offsets, the mask words when there is a per-block mask,
// then the split workspace (the larger of the plans with and without V aliasing K, decided
// at run time).
struct Sizes {
  int64_t nkeys, nwords;
  int max_keys;
  size_t key_bytes, mask_bytes, split_bytes;
};

Sizes plan_sizes(const int32_t* indptr, int MB, int R, int C, int Hq, int Hkv, int D, bool masked) {
  Sizes z{};
  z.nkeys = (int64_t)indptr[MB] * C;
  for (int i = 0; i < MB; ++i) {
    const int keys = (indptr[i + 1] - indptr[i]) * C;
    z.max_keys = std::max(z.max_keys, keys);
    z.nwords += (keys + 31) / 32;
  }
  z.key_bytes = (((size_t)(MB + 1) + (size_t)z.nkeys) * 4 + 255) & ~(size_t)255;
  if (!masked) z.nwords = 0;
  z.mask_bytes = masked ? (((size_t)(MB + 1) + (size_t)z.nwords * (1 + (size_t)R)) * 4 + 255) & ~(size_t)255 : 0;
  const int G = R * (Hq / Hkv);
  const int cus = sfa::device_cu_count();
  size_t split = 0;
  for (int alias = 0; alias < 2; ++alias) {
    const sfa::TopkPlan pl =
        sfa::plan_topk((int64_t)MB * Hkv, G, z.max_keys, kernel_dim(D), kernel_dim(D), alias != 0, cus, true);
    split = std::max(split, pl.ws_bytes);
  }
  z.split_bytes = split;
  return z;
}

sfa_status validate(const int32_t* indptr, const int32_t* indices, int M, int N, int R, int C, int Hq, int Hkv,
                    int D, int causal) {
  if (!indptr) return SFA_ERR_NULL;
  if (M < 0 || N < 1 || R < 1 || C < 1 || Hq < 1 || Hkv < 1) return SFA_ERR_SHAPE;
  if (N % C != 0) return SFA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SFA_ERR_GQA;
  if (D < 64 || D % 64) return SFA_ERR_HEAD_DIM;
  if (kernel_dim(D) == 0) return SFA_ERR_UNSUPPORTED;
  if (causal && M > N) return SFA_ERR_CAUSAL;
  const int MB = (M + R - 1) / R, NB = N / C;
  if (indptr[0] != 0) return SFA_ERR_PLAN;
  for (int i = 0; i < MB; ++i)
    if (indptr[i + 1] < indptr[i]) return SFA_ERR_PLAN;
  const int nnz = indptr[MB];
  if (nnz > 0 && !indices) return SFA_ERR_NULL;
  if ((int64_t)nnz * C > 0x7fffffffLL || (int64_t)R * (Hq / Hkv) > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;
  std::vector<int> seen(NB, -1);
  for (int i = 0; i < MB; ++i)
    for (int t = indptr[i]; t < indptr[i + 1]; ++t) {
      const int c = indices[t];
      if (c < 0 || c >= NB || seen[c] == i) return SFA_ERR_INDEX;
      seen[c] = i;
    }
  return SFA_OK;
}

}  // namespace

extern "C" {

size_t bsr_plan_workspace_bytes(const int32_t* indptr, const int32_t* indices, const uint8_t* mask, int M, int N,
                                int R, int C, int num_qo_heads, int num_kv_heads, int head_dim) {
  if (validate(indptr, indices, M, N, R, C, num_qo_heads, num_kv_heads, head_dim, 0) != SFA_OK) return 0;
  const int MB = (M + R - 1) / R;
  const Sizes z = plan_sizes(indptr, MB, R, C, num_qo_heads, num_kv_heads, head_dim, mask != nullptr);
  return z.key_bytes + z.mask_bytes + 256;
}

size_t bsr_plan_float_workspace_bytes(const int32_t* indptr, const int32_t* indices, int M, int N, int R, int C,
                                      int num_qo_heads, int num_kv_heads, int head_dim) {
  if (validate(indptr, indices, M, N, R, C, num_qo_heads, num_kv_heads, head_dim, 0) != SFA_OK) return 0;
  const int MB = (M + R - 1) / R;
  const Sizes z = plan_sizes(indptr, MB, R, C, num_qo_heads, num_kv_heads, head_dim, false);
  return z.split_bytes > 0 ? z.split_bytes + 256 : 0;
}

sfa_status bsr_plan(bsr_plan_t** plan, const int32_t* indptr, const int32_t* indices, const uint8_t* mask, int M,
                    int N, int R, int C, int num_qo_heads, int num_kv_heads, int head_dim, int causal,
                    float sm_scale, sfa_dtype dtype, void* workspace, size_t workspace_bytes, void* float_workspace,
                    size_t float_workspace_bytes, hipStream_t stream) {
  if (!plan) return SFA_ERR_NULL;
  *plan = nullptr;
  if (dtype != SFA_FP16 && dtype != SFA_BF16) return SFA_ERR_DTYPE;
  const sfa_status st = validate(indptr, indices, M, N, R, C, num_qo_heads, num_kv_heads, head_dim, causal);
  if (st != SFA_OK) return st;
  if (!isfinite(sm_scale)) return SFA_ERR_SCALE;
  const int MB = (M + R - 1) / R;
  const Sizes z = plan_sizes(indptr, MB, R, C, num_qo_heads, num_kv_heads, head_dim, mask != nullptr);
  const int64_t items = (int64_t)MB * num_kv_heads;
  for (int alias = 0; alias < 2; ++alias) {
    const sfa::TopkPlan pl = sfa::plan_topk(items, R * (num_qo_heads / num_kv_heads), z.max_keys,
                                            kernel_dim(head_dim), kernel_dim(head_dim), alias != 0,
                                            sfa::device_cu_count(), true);
    if (pl.WS < 1) return SFA_ERR_UNSUPPORTED;
    if ((int64_t)pl.grid > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;
  }
  if (!workspace || workspace_bytes < z.key_bytes + z.mask_bytes + 256) return SFA_ERR_WORKSPACE;
  if (z.split_bytes > 0 && (!float_workspace || float_workspace_bytes < z.split_bytes + 256)) return SFA_ERR_WORKSPACE;

  bsr_plan_t* pl = (bsr_plan_t*)calloc(1, sizeof(bsr_plan_t));
  if (!pl) return SFA_ERR_HIP;
  // staged as one image of the device layout: key offsets + keys, padding, mask words
  const size_t stage_bytes = z.key_bytes + z.mask_bytes;
  if (hipHostMalloc((void**)&pl->pinned, stage_bytes + 4, hipHostMallocDefault) != hipSuccess) {
    free(pl);
    return SFA_ERR_HIP;
  }
  memset(pl->pinned, 0, stage_bytes);
  // key list: block row br holds, block after block, the C key rows of each stored block
  int32_t* kptr = pl->pinned;
  int32_t* keys = pl->pinned + MB + 1;
  for (int i = 0; i <= MB; ++i) kptr[i] = indptr[i] * C;
  for (int t = 0; t < indptr[MB]; ++t)
    for (int c = 0; c < C; ++c) keys[(int64_t)t * C + c] = indices[t] * C + c;
  if (mask) {
    // per block row, 32-slot words of its key list; word w of row br, query row i holds bit b
    // = mask[t][i][j] for slot s = 32 (w - wptr[br]) + b = (t - indptr[br]) C + j; slots past
    // the list and rows past M stay set (they are masked by other means)
    int32_t* wptr = (int32_t*)((char*)pl->pinned + z.key_bytes);
    int32_t* wflag = wptr + MB + 1;
    uint32_t* words = (uint32_t*)(wflag + z.nwords);
    wptr[0] = 0;
    for (int br = 0; br < MB; ++br) {
      const int nk = (indptr[br + 1] - indptr[br]) * C;
      wptr[br + 1] = wptr[br] + (nk + 31) / 32;
      const int rows = std::min(R, M - br * R);
      for (int w = wptr[br]; w < wptr[br + 1]; ++w)
        for (int i = 0; i < R; ++i) {
          uint32_t bits = 0xffffffffu;
          if (i < rows)
            for (int b = 0; b < 32; ++b) {
              const int s = 32 * (w - wptr[br]) + b;
              if (s >= nk) break;
              const int64_t t = indptr[br] + s / C;
              if (!mask[(t * R + i) * C + s % C]) bits &= ~(1u << b);
            }
          words[(int64_t)w * R + i] = bits;
          if (bits != 0xffffffffu) wflag[w] = 1;
        }
    }
  }

  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  pl->d_kptr = (int32_t*)base;
  pl->d_keys = pl->d_kptr + MB + 1;
  pl->nwords = z.nwords;
  if (mask) {
    pl->d_wptr = (int32_t*)(base + z.key_bytes);
    pl->d_wflag = pl->d_wptr + MB + 1;
    pl->d_words = (uint32_t*)(pl->d_wflag + z.nwords);
  }
  pl->d_split = z.split_bytes > 0 ? (float*)(((uintptr_t)float_workspace + 255) & ~(uintptr_t)255) : nullptr;
  pl->split_bytes = z.split_bytes;
  if (hipEventCreateWithFlags(&pl->copied, hipEventDisableTiming) != hipSuccess ||
      hipMemcpyAsync(base, pl->pinned, stage_bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(pl->copied, stream) != hipSuccess) {
    (void)hipHostFree(pl->pinned);
    free(pl);
    return SFA_ERR_HIP;
  }
  pl->M = M; pl->N = N; pl->R = R; pl->C = C;
  pl->Hq = num_qo_heads; pl->Hkv = num_kv_heads; pl->D = head_dim;
  pl->causal = (causal && !mask) ? 1 : 0;  // the page ignores causal when a mask is given
  pl->MB = MB;
  pl->max_keys = z.max_keys;
  pl->nkeys = z.nkeys;
  pl->dtype = dtype;
  pl->scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)head_dim));
  *plan = pl;
  return SFA_OK;
}

static sfa_status bsr_launch(const bsr_plan_t* pl, const void* q, const void* k, const void* v, void* out,
                             float* lse, const float* fq, const float* fk, const float* fv, hipStream_t stream,
                             bool dry = false) {
  if (!pl) return SFA_ERR_PLAN;
  if (pl->M == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if (mis & 15u) return SFA_ERR_LAYOUT;
  const bool alias = v == k;
  if (!sfa::topk_rows_addressable(pl->N, (int64_t)pl->Hkv * pl->D, pl->D)) return SFA_ERR_UNSUPPORTED;
  const int Gh = pl->Hq / pl->Hkv;
  const int KD = kernel_dim(pl->D);  // compiled head dim serving pl->D
  const sfa::TopkPlan tp = sfa::plan_topk((int64_t)pl->MB * pl->Hkv, pl->R * Gh, pl->max_keys, KD, KD, alias,
                                          sfa::device_cu_count(), true);
  if (tp.WS < 1) return SFA_ERR_UNSUPPORTED;
  if (pl->d_words && tp.MT == sfa::kDvsHeads) return SFA_ERR_UNSUPPORTED;  // no element mask there
  if (tp.ws_bytes > pl->split_bytes) return SFA_ERR_WORKSPACE;  // device changed since the plan
  const int64_t D = pl->D, Hq = pl->Hq, Hkv = pl->Hkv, R = pl->R;

  sfa::TopkParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.idx = pl->d_keys;
  p.slot_ptr = pl->d_kptr;
  p.out = (uint16_t*)out;
  p.lse = lse;
  // (batch, block row, query head, query row inside the block row)
  p.qs[0] = 0; p.qs[1] = R * Hq * D; p.qs[2] = D; p.qs[3] = Hq * D;
  p.os[0] = 0; p.os[1] = R * Hq * D; p.os[2] = D; p.os[3] = Hq * D;
  p.ls[0] = 0; p.ls[1] = R * Hq; p.ls[2] = 1; p.ls[3] = Hq;
  // (batch, key row, KV head)
  p.ks[0] = 0; p.ks[1] = Hkv * D; p.ks[2] = D;
  p.vs[0] = 0; p.vs[1] = Hkv * D; p.vs[2] = D;
  if (tp.nsplit > 1) {
    p.ws_o = pl->d_split;
    p.ws_ml = pl->d_split + (size_t)tp.rows * tp.nsplit * KD;
  }
  p.B = 1;
  p.S1 = pl->MB;
  p.S2 = pl->N;
  p.N2 = pl->Hkv;
  p.G = pl->R * Gh;
  p.HR = Gh;
  p.RS = pl->R;
  p.QROWS = pl->M;
  p.topK = pl->max_keys;
  p.causal = pl->causal;
  p.dk = p.dv = pl->D;
  p.scale_log2 = (float)((double)pl->scale * 1.4426950408889634);
  p.fq = fq;
  p.fk = fk;
  p.fv = fv;
  p.bm_words = pl->d_words;
  p.bm_wptr = pl->d_wptr;
  p.bm_wflag = pl->d_wflag;
  p.nsplit = tp.nsplit;
  p.split_len = tp.split_len;
  p.HB = tp.HB;
  p.n_items = tp.grid;
  if (p.n_items == 0) return SFA_OK;
  if (dry) return SFA_OK;  // every check passed; nothing enqueued
  bool found = false;
  const hipError_t e = sfa::launch_topk(pl->dtype == SFA_FP16, alias, KD, KD, tp, p, stream, &found);
  if (!found) return SFA_ERR_UNSUPPORTED;
  return e == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

sfa_status bsr_run(const bsr_plan_t* pl, const void* q, const void* k, const void* v, void* out, float* lse,
                   hipStream_t stream) {
  return bsr_launch(pl, q, k, v, out, lse, nullptr, nullptr, nullptr, stream);
}

size_t bsr_fp8_workspace_bytes(const bsr_plan_t* pl) {
  if (!pl) return 0;
  return sfa::fp8_copies_bytes((int64_t)pl->M * pl->Hq * pl->D, (int64_t)pl->N * pl->Hkv * pl->D);
}

sfa_status bsr_run_fp8(const bsr_plan_t* pl, const void* q, const void* k, const void* v, sfa_fp8 q_fmt,
                       sfa_fp8 kv_fmt, const float* scale_q, const float* scale_k, const float* scale_v, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!pl) return SFA_ERR_PLAN;
  if (pl->dtype != SFA_FP16) return SFA_ERR_DTYPE;
  if ((q_fmt != SFA_FP8_E4M3 && q_fmt != SFA_FP8_E5M2) || (kv_fmt != SFA_FP8_E4M3 && kv_fmt != SFA_FP8_E5M2))
    return SFA_ERR_DTYPE;
  if (pl->M == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)workspace) & 15u) return SFA_ERR_LAYOUT;
  if (!workspace || workspace_bytes < bsr_fp8_workspace_bytes(pl)) return SFA_ERR_WORKSPACE;
  // the fp16 launch's own checks run before anything is enqueued (q, k, v stand in for the copies)
  const sfa_status st = bsr_launch(pl, q, k, v == k ? k : (const void*)out, out, lse, scale_q, scale_k, scale_v,
                                   stream, true);
  if (st != SFA_OK) return st;
  void *q16, *k16, *v16;
  const hipError_t e = sfa::fp8_expand_qkv(q, k, v, (int)q_fmt, (int)kv_fmt, (int64_t)pl->M * pl->Hq * pl->D,
                                           (int64_t)pl->N * pl->Hkv * pl->D, pl->D, pl->Hkv, workspace, &q16, &k16,
                                           &v16, stream);
  if (e != hipSuccess) return SFA_ERR_HIP;
  return bsr_launch(pl, q16, k16, v16, out, lse, scale_q, scale_k, scale_v, stream);
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
