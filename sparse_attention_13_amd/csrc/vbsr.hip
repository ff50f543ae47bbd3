// Variable block-sparse plan / run entry points (flashinfer.sparse,
// VariableBlockSparseAttentionWrapper: per-KV-head block grids with variable block
// row and column sizes, q / k / v in HND layout).
//
// Like the BSR form, a block row is a top-K problem in disguise: its query rows (times
// the Hq / Hkv query heads of its KV head) share one key list, the concatenated key
// ranges of the row's attended column blocks.  plan() builds one key list per (KV head,
// block row) and an item table that cuts every block row into pieces of at most RS query
// rows; run() launches the top-K kernels with one work item per piece, whose "heads" are
// its query vectors (query row row0 + h / G, query head kvh * G + h % G).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "../../include/sfa.h"
#include "fp8.hpp"
#include "topk_launch.hpp"

struct vbsr_plan_t {
  int M, N, Hq, Hkv, D, causal, RS, max_keys;
  int64_t items;
  sfa_dtype dtype;
  float scale;
  int32_t* d_kptr;          // [Hkv * MB + 1] key-list offsets
  int32_t* d_keys;          // key rows (local to the KV head)
  sfa::TopkItem* d_itab;    // [items]
  float* d_split;           // split partials (may be unused)
  size_t split_bytes;
  void* pinned;             // host staging of the async copy; freed with the plan
  hipEvent_t copied;
};

namespace {

// Head dim of the compiled kernels that serve head dim D (0: none); the kernels take D itself
// at run time.
int kernel_dim(int D) {
  int DK = 0, DV = 0;
  return sfa::topk_kernel_dims(D, D, &DK, &DV) && DK == DV ? DK : 0;
}

// Most query vectors one work item carries (as in the BSR form's 64-row blocks of 4 heads).
constexpr int kMaxItemVectors = 256;

struct VSizes {
  int M, N, RS, max_keys;
  int64_t items, nkeys;
  size_t key_bytes, itab_bytes, split_bytes;
};

sfa_status validate(const uint8_t* bmap, const int32_t* rsz, const int32_t* csz, int Hkv, int MB, int NB, int Hq,
                    int D, int causal, VSizes* z) {
  if (Hkv < 1 || Hq < 1 || MB < 0 || NB < 1) return SFA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SFA_ERR_GQA;
  if (D < 64 || D % 64) return SFA_ERR_HEAD_DIM;
  if (kernel_dim(D) == 0) return SFA_ERR_UNSUPPORTED;
  if (!csz || (MB > 0 && (!rsz || !bmap))) return SFA_ERR_NULL;
  int64_t M = -1, N = -1;
  for (int h = 0; h < Hkv; ++h) {
    int64_t m = 0, n = 0;
    for (int i = 0; i < MB; ++i) {
      if (rsz[(int64_t)h * MB + i] < 0) return SFA_ERR_SHAPE;
      m += rsz[(int64_t)h * MB + i];
    }
    for (int j = 0; j < NB; ++j) {
      if (csz[(int64_t)h * NB + j] < 0) return SFA_ERR_SHAPE;
      n += csz[(int64_t)h * NB + j];
    }
    if ((M >= 0 && m != M) || (N >= 0 && n != N)) return SFA_ERR_SHAPE;
    M = m;
    N = n;
  }
  if (N < 1 || M > 0x7fffffffLL || N > 0x7fffffffLL) return SFA_ERR_SHAPE;
  if (causal && M > N) return SFA_ERR_CAUSAL;
  const int G = Hq / Hkv;
  int max_rows = 0;
  for (int64_t t = 0; t < (int64_t)Hkv * MB; ++t) max_rows = std::max(max_rows, rsz[t]);
  const int RS = std::max(1, std::min(max_rows, kMaxItemVectors / G));
  int64_t items = 0, nkeys = 0;
  int64_t max_keys = 0;
  for (int h = 0; h < Hkv; ++h)
    for (int i = 0; i < MB; ++i) {
      items += (rsz[(int64_t)h * MB + i] + RS - 1) / RS;
      int64_t keys = 0;
      for (int j = 0; j < NB; ++j)
        if (bmap[((int64_t)h * MB + i) * NB + j]) keys += csz[(int64_t)h * NB + j];
      nkeys += keys;
      max_keys = std::max(max_keys, keys);
    }
  if (nkeys > 0x7fffffffLL || items > 0x7fffffffLL || (int64_t)RS * G > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;
  z->M = (int)M;
  z->N = (int)N;
  z->RS = RS;
  z->items = items;
  z->nkeys = nkeys;
  z->max_keys = (int)max_keys;
  z->key_bytes = (((size_t)Hkv * MB + 1 + (size_t)nkeys) * 4 + 255) & ~(size_t)255;
  z->itab_bytes = ((size_t)items * sizeof(sfa::TopkItem) + 255) & ~(size_t)255;
  // split workspace: the larger of the plans with and without V aliasing K (decided at run)
  size_t split = 0;
  for (int alias = 0; alias < 2; ++alias) {
    const sfa::TopkPlan pl =
        sfa::plan_topk(items, RS * G, z->max_keys, kernel_dim(D), kernel_dim(D), alias != 0, sfa::device_cu_count(),
                       true);
    if (pl.WS < 1 || (int64_t)pl.grid > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;
    split = std::max(split, pl.ws_bytes);
  }
  z->split_bytes = split;
  return SFA_OK;
}

}  // namespace

extern "C" {

size_t vbsr_plan_workspace_bytes(const uint8_t* block_mask_map, const int32_t* block_row_sz,
                                 const int32_t* block_col_sz, int num_kv_heads, int MB, int NB, int num_qo_heads,
                                 int head_dim) {
  VSizes z{};
  if (validate(block_mask_map, block_row_sz, block_col_sz, num_kv_heads, MB, NB, num_qo_heads, head_dim, 0, &z) !=
      SFA_OK)
    return 0;
  return z.key_bytes + z.itab_bytes + 256;
}

size_t vbsr_plan_float_workspace_bytes(const uint8_t* block_mask_map, const int32_t* block_row_sz,
                                       const int32_t* block_col_sz, int num_kv_heads, int MB, int NB,
                                       int num_qo_heads, int head_dim) {
  VSizes z{};
  if (validate(block_mask_map, block_row_sz, block_col_sz, num_kv_heads, MB, NB, num_qo_heads, head_dim, 0, &z) !=
      SFA_OK)
    return 0;
  return z.split_bytes > 0 ? z.split_bytes + 256 : 0;
}

sfa_status vbsr_plan(vbsr_plan_t** plan, const uint8_t* block_mask_map, const int32_t* block_row_sz,
                     const int32_t* block_col_sz, int num_kv_heads, int MB, int NB, int num_qo_heads, int head_dim,
                     int causal, float sm_scale, sfa_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* float_workspace, size_t float_workspace_bytes, hipStream_t stream) {
  if (!plan) return SFA_ERR_NULL;
  *plan = nullptr;
  if (dtype != SFA_FP16 && dtype != SFA_BF16) return SFA_ERR_DTYPE;
  VSizes z{};
  const sfa_status st = validate(block_mask_map, block_row_sz, block_col_sz, num_kv_heads, MB, NB, num_qo_heads,
                                 head_dim, causal, &z);
  if (st != SFA_OK) return st;
  if (!isfinite(sm_scale)) return SFA_ERR_SCALE;
  if (!workspace || workspace_bytes < z.key_bytes + z.itab_bytes + 256) return SFA_ERR_WORKSPACE;
  if (z.split_bytes > 0 && (!float_workspace || float_workspace_bytes < z.split_bytes + 256)) return SFA_ERR_WORKSPACE;

  vbsr_plan_t* pl = (vbsr_plan_t*)calloc(1, sizeof(vbsr_plan_t));
  if (!pl) return SFA_ERR_HIP;
  // staged as one image of the device layout: key offsets + keys, padding, item table
  const size_t stage_bytes = z.key_bytes + z.itab_bytes;
  if (hipHostMalloc(&pl->pinned, stage_bytes, hipHostMallocDefault) != hipSuccess) {
    free(pl);
    return SFA_ERR_HIP;
  }
  memset(pl->pinned, 0, stage_bytes);
  const int Hkv = num_kv_heads;
  int32_t* kptr = (int32_t*)pl->pinned;
  int32_t* keys = kptr + (int64_t)Hkv * MB + 1;
  sfa::TopkItem* itab = (sfa::TopkItem*)((char*)pl->pinned + z.key_bytes);
  std::vector<int32_t> col0(NB);
  std::vector<std::pair<int, sfa::TopkItem>> pieces;  // (key count, item)
  pieces.reserve((size_t)z.items);
  int64_t nk = 0;
  kptr[0] = 0;
  for (int h = 0; h < Hkv; ++h) {
    for (int j = 0, c = 0; j < NB; c += block_col_sz[(int64_t)h * NB + j], ++j) col0[j] = c;
    for (int i = 0, r0 = 0; i < MB; r0 += block_row_sz[(int64_t)h * MB + i], ++i) {
      const int64_t list = (int64_t)h * MB + i;
      // key list of block row i: the key rows of its attended column blocks, in column order
      for (int j = 0; j < NB; ++j)
        if (block_mask_map[list * NB + j])
          for (int c = 0; c < block_col_sz[(int64_t)h * NB + j]; ++c) keys[nk++] = col0[j] + c;
      kptr[list + 1] = (int32_t)nk;
      // pieces of at most RS query rows
      const int rows = block_row_sz[list];
      for (int a = 0; a < rows; a += z.RS)
        pieces.push_back({kptr[list + 1] - kptr[list], sfa::TopkItem{r0 + a, std::min(z.RS, rows - a), h, (int)list}});
    }
  }
  // Table order = launch order: the launch deals consecutive items to one XCD (sfa::xcd_remap:
  // XCD x runs the range [start(x), start(x) + count(x)) of the table, in order).  Longest key
  // list first, so that the pieces that run last are short; the pieces of one block row (one
  // key list) go to consecutive places of one XCD's range, so they run at about the same time
  // and all but the first find the list's key rows in that XCD's L2; each list goes to the XCD
  // with the most room left (balanced ranges), a list that does not fit spills to the next.
  std::stable_sort(pieces.begin(), pieces.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
  const int64_t n = (int64_t)pieces.size(), q = n / 8, r = n % 8;
  int64_t room[8], fill[8], start[8];
  for (int x = 0; x < 8; ++x) {
    start[x] = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    room[x] = x < r ? q + 1 : q;
    fill[x] = 0;
  }
  auto roomiest = [&]() {
    int best = 0;
    for (int x = 1; x < 8; ++x)
      if (room[x] > room[best]) best = x;
    return best;
  };
  for (int64_t t = 0; t < n;) {
    int64_t e = t;
    while (e < n && pieces[(size_t)e].second.list == pieces[(size_t)t].second.list) ++e;
    int x = roomiest();
    for (; t < e; ++t) {
      if (room[x] == 0) x = roomiest();
      itab[start[x] + fill[x]++] = pieces[(size_t)t].second;
      --room[x];
    }
  }

  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  pl->d_kptr = (int32_t*)base;
  pl->d_keys = pl->d_kptr + (int64_t)Hkv * MB + 1;
  pl->d_itab = (sfa::TopkItem*)(base + z.key_bytes);
  pl->d_split = z.split_bytes > 0 ? (float*)(((uintptr_t)float_workspace + 255) & ~(uintptr_t)255) : nullptr;
  pl->split_bytes = z.split_bytes;
  if (hipEventCreateWithFlags(&pl->copied, hipEventDisableTiming) != hipSuccess ||
      hipMemcpyAsync(base, pl->pinned, stage_bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(pl->copied, stream) != hipSuccess) {
    (void)hipHostFree(pl->pinned);
    free(pl);
    return SFA_ERR_HIP;
  }
  pl->M = z.M;
  pl->N = z.N;
  pl->Hq = num_qo_heads;
  pl->Hkv = Hkv;
  pl->D = head_dim;
  pl->causal = causal ? 1 : 0;
  pl->RS = z.RS;
  pl->max_keys = z.max_keys;
  pl->items = z.items;
  pl->dtype = dtype;
  pl->scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)head_dim));
  *plan = pl;
  return SFA_OK;
}

static sfa_status vbsr_launch(const vbsr_plan_t* pl, const void* q, const void* k, const void* v, void* out,
                             float* lse, const float* fq, const float* fk, const float* fv, hipStream_t stream,
                             bool dry = false) {
  if (!pl) return SFA_ERR_PLAN;
  if (pl->M == 0 || pl->items == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if (mis & 15u) return SFA_ERR_LAYOUT;
  const bool alias = v == k;
  if (!sfa::topk_rows_addressable(pl->N, pl->D, pl->D)) return SFA_ERR_UNSUPPORTED;
  const int G = pl->Hq / pl->Hkv;
  const int KD = kernel_dim(pl->D);  // compiled head dim serving pl->D
  const sfa::TopkPlan tp = sfa::plan_topk(pl->items, pl->RS * G, pl->max_keys, KD, KD, alias,
                                          sfa::device_cu_count(), true);
  if (tp.WS < 1) return SFA_ERR_UNSUPPORTED;
  if (tp.ws_bytes > pl->split_bytes) return SFA_ERR_WORKSPACE;  // device changed since the plan
  const int64_t D = pl->D, M = pl->M, N = pl->N;

  sfa::TopkParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.idx = pl->d_keys;
  p.slot_ptr = pl->d_kptr;
  p.itab = pl->d_itab;
  p.out = (uint16_t*)out;
  p.lse = lse;
  // HND: (batch, -, query head, query row); the item table supplies the rows and KV head
  p.qs[0] = 0; p.qs[1] = 0; p.qs[2] = M * D; p.qs[3] = D;
  p.os[0] = 0; p.os[1] = 0; p.os[2] = M * D; p.os[3] = D;
  p.ls[0] = 0; p.ls[1] = 0; p.ls[2] = M; p.ls[3] = 1;
  // (batch, key row, KV head)
  p.ks[0] = 0; p.ks[1] = D; p.ks[2] = N * D;
  p.vs[0] = 0; p.vs[1] = D; p.vs[2] = N * D;
  if (tp.nsplit > 1) {
    p.ws_o = pl->d_split;
    p.ws_ml = pl->d_split + (size_t)tp.rows * tp.nsplit * KD;
  }
  p.B = 1;
  p.S1 = (int)pl->items;
  p.S2 = pl->N;
  p.N2 = 1;
  p.G = pl->RS * G;
  p.HR = G;
  p.RS = pl->RS;
  p.QROWS = pl->M;
  p.topK = pl->max_keys;
  p.dk = p.dv = pl->D;
  p.causal = pl->causal;
  p.scale_log2 = (float)((double)pl->scale * 1.4426950408889634);
  p.fq = fq;
  p.fk = fk;
  p.fv = fv;
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

sfa_status vbsr_run(const vbsr_plan_t* pl, const void* q, const void* k, const void* v, void* out, float* lse,
                    hipStream_t stream) {
  return vbsr_launch(pl, q, k, v, out, lse, nullptr, nullptr, nullptr, stream);
}

size_t vbsr_fp8_workspace_bytes(const vbsr_plan_t* pl) {
  if (!pl) return 0;
  return sfa::fp8_copies_bytes((int64_t)pl->Hq * pl->M * pl->D, (int64_t)pl->Hkv * pl->N * pl->D);
}

sfa_status vbsr_run_fp8(const vbsr_plan_t* pl, const void* q, const void* k, const void* v, sfa_fp8 q_fmt,
                        sfa_fp8 kv_fmt, const float* scale_q, const float* scale_k, const float* scale_v,
                        void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!pl) return SFA_ERR_PLAN;
  if (pl->dtype != SFA_FP16) return SFA_ERR_DTYPE;
  if ((q_fmt != SFA_FP8_E4M3 && q_fmt != SFA_FP8_E5M2) || (kv_fmt != SFA_FP8_E4M3 && kv_fmt != SFA_FP8_E5M2))
    return SFA_ERR_DTYPE;
  if (pl->M == 0 || pl->items == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)workspace) & 15u) return SFA_ERR_LAYOUT;
  if (!workspace || workspace_bytes < vbsr_fp8_workspace_bytes(pl)) return SFA_ERR_WORKSPACE;
  // the fp16 launch's own checks run before anything is enqueued (q, k, v stand in for the copies)
  const sfa_status st = vbsr_launch(pl, q, k, v == k ? k : (const void*)out, out, lse, scale_q, scale_k, scale_v,
                                    stream, true);
  if (st != SFA_OK) return st;
  void *q16, *k16, *v16;
  const hipError_t e = sfa::fp8_expand_qkv(q, k, v, (int)q_fmt, (int)kv_fmt, (int64_t)pl->Hq * pl->M * pl->D,
                                           (int64_t)pl->Hkv * pl->N * pl->D, (int64_t)pl->N * pl->D, pl->Hkv, workspace, &q16, &k16,
                                           &v16, stream);
  if (e != hipSuccess) return SFA_ERR_HIP;
  return vbsr_launch(pl, q16, k16, v16, out, lse, scale_q, scale_k, scale_v, stream);
}

sfa_status vbsr_destroy(vbsr_plan_t* pl) {
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
