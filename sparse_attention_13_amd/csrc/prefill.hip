// Dense attention of one request with an optional custom mask or bottom-right causal mask
// (flashinfer.prefill.single_prefill_with_kv_cache: q [qo_len, Hq, Dqk], k / v in NHD
// [kv_len, Hkv, D] or HND [Hkv, kv_len, D], custom_mask [qo_len, kv_len] with False =
// masked, causal applying only without a mask).
//
// Dense attention is the top-K problem whose index list is every key in order, and a block of
// query rows of one KV head shares that list: a work item is (block of RS query rows, KV head)
// with RS x (Hq / Hkv) query vectors, all items pointing at one identity key list through the
// item table.  Keys are consecutive rows, so the staging loads are whole contiguous K / V tiles
// and every staged tile serves all the item's query vectors.  The custom mask is packed on the
// GPU into the 32-slot mask words the kernels test (one word per 32 keys and query row, plus a
// flag per word where some bit is clear); causal uses the kernels' per-row limit.
#include <math.h>
#include <string.h>

#include "../../include/sfa.h"
#include "topk_launch.hpp"

namespace {

constexpr int kMaxItemVectors = 256;  // query vectors per work item (the block-sparse forms' bound)

struct PrefillLayout {
  int RS, nrb, items, W;  // rows per item, row blocks, items, mask words per query row
  size_t idx_off, ptr_off, itab_off, wptr_off, wflag_off, words_off, split_off, total;
  sfa::TopkPlan tp;
  int DK, DV;
  bool ok;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Query rows per item: as many as keep the item's query vectors within kMaxItemVectors; with a
// mask and wide values (the kernel for many query vectors has no element mask) at most 32.
PrefillLayout layout(int qo_len, int kv_len, int Hq, int Hkv, int Dqk, int Dvo, bool masked, bool alias) {
  PrefillLayout L{};
  if (!sfa::topk_kernel_dims(Dqk, Dvo, &L.DK, &L.DV)) return L;
  const int G = Hq / Hkv;
  int cap = kMaxItemVectors;
  if (masked && L.DV > 256) cap = 32;
  if (G > cap) return L;
  L.RS = std::max(1, std::min(qo_len, cap / G));
  L.nrb = (qo_len + L.RS - 1) / L.RS;
  L.items = L.nrb * Hkv;
  L.W = (kv_len + 31) / 32;
  L.tp = sfa::plan_topk(L.items, L.RS * G, kv_len, L.DK, L.DV, alias, sfa::device_cu_count());
  if (L.tp.WS < 1 || (int64_t)L.tp.grid > 0x7fffffffLL) return L;
  if (masked && L.tp.MT == sfa::kDvsHeads) return L;
  size_t o = 0;
  L.idx_off = o;   o += up256((size_t)kv_len * 4);
  L.ptr_off = o;   o += 256;
  L.itab_off = o;  o += up256((size_t)L.items * sizeof(sfa::TopkItem));
  if (masked) {
    L.wptr_off = o;  o += up256(((size_t)L.items + 1) * 4);
    L.wflag_off = o; o += up256((size_t)L.items * L.W * 4);
    L.words_off = o; o += up256((size_t)L.items * L.W * L.RS * 4);
  }
  L.split_off = o;
  o += L.tp.ws_bytes;
  L.total = o + 256;  // alignment of the caller's base
  L.ok = true;
  return L;
}

// Identity key list, its CSR offsets, the item table (item t: row block t / Hkv, KV head t % Hkv)
// and, with a mask, the first mask word of every item.
__global__ __launch_bounds__(256) void prefill_tables(int32_t* idx, int32_t* slot_ptr, sfa::TopkItem* itab,
                                                      int32_t* wptr, int kv_len, int qo_len, int RS, int Hkv,
                                                      int items, int W) {
  const int n = max(kv_len, items + 1);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    if (i < kv_len) idx[i] = i;
    if (i < items) {
      // head-major: the launch deals consecutive items to one XCD, so an XCD works on the row
      // blocks of as few KV heads as possible and their K / V rows stay in its L2
      const int nrb = items / Hkv, h = i / nrb, rb = i % nrb;
      itab[i] = sfa::TopkItem{rb * RS, min(RS, qo_len - rb * RS), h, 0};
    }
    if (wptr && i <= items) wptr[i] = i * W;
    if (i < 2) slot_ptr[i] = i * kv_len;
  }
}

// Mask words of item t, word w, query row i: bit b = mask[row0 + i][32 w + b] (keys past kv_len
// and rows past the block stay set: the kernels mask them by other means); flag[t][w] != 0 when
// some bit of the word is clear for some row.  One thread per (row block, word); the Hkv items
// of a row block get the same words.
__global__ __launch_bounds__(256) void prefill_pack_mask(const uint8_t* __restrict__ mask, int qo_len, int kv_len,
                                                         int RS, int Hkv, int nrb, int W, uint32_t* __restrict__ words,
                                                         int32_t* __restrict__ wflag) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (int64_t)nrb * W) return;
  const int rb = (int)(g / W), w = (int)(g % W);
  const int row0 = rb * RS, rows = min(RS, qo_len - row0);
  const int c0 = 32 * w, nc = min(32, kv_len - c0);
  int clear = 0;
  for (int i = 0; i < RS; ++i) {
    uint32_t bits = 0xffffffffu;
    if (i < rows) {
      const uint8_t* m = mask + (int64_t)(row0 + i) * kv_len + c0;
      for (int b = 0; b < nc; ++b)
        if (!m[b]) bits &= ~(1u << b);
    }
    clear |= bits != 0xffffffffu;
    for (int h = 0; h < Hkv; ++h) words[((int64_t)(h * nrb + rb) * W + w) * RS + i] = bits;
  }
  for (int h = 0; h < Hkv; ++h) wflag[(int64_t)(h * nrb + rb) * W + w] = clear;
}

sfa_status validate(int qo_len, int kv_len, int Hq, int Hkv, int Dqk, int Dvo, sfa_dtype dtype, sfa_kv_layout lay,
                    int causal, const void* mask) {
  if (dtype != SFA_FP16 && dtype != SFA_BF16) return SFA_ERR_DTYPE;
  if (lay != SFA_NHD && lay != SFA_HND) return SFA_ERR_LAYOUT;
  if (qo_len < 0 || kv_len < 1 || Hq < 1 || Hkv < 1) return SFA_ERR_SHAPE;
  if (Hq % Hkv) return SFA_ERR_GQA;
  if (Dqk < 64 || Dvo < 64 || Dqk % 64 || Dvo % 64 || Dvo > Dqk) return SFA_ERR_HEAD_DIM;
  if (causal && !mask && qo_len > kv_len) return SFA_ERR_CAUSAL;
  return SFA_OK;
}

}  // namespace

extern "C" {

size_t sfa_prefill_workspace_bytes(int qo_len, int kv_len, int num_qo_heads, int num_kv_heads, int head_dim_qk,
                                   int head_dim_vo, int masked) {
  if (validate(qo_len, kv_len, num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo, SFA_FP16, SFA_NHD, 0, nullptr) !=
          SFA_OK ||
      qo_len == 0)
    return 0;
  size_t most = 0;
  for (int alias = 0; alias < 2; ++alias) {
    const PrefillLayout L =
        layout(qo_len, kv_len, num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo, masked != 0, alias != 0);
    if (L.ok) most = std::max(most, L.total);
  }
  return most;
}

sfa_status sfa_prefill(int qo_len, int kv_len, int num_qo_heads, int num_kv_heads, int head_dim_qk, int head_dim_vo,
                       sfa_dtype dtype, sfa_kv_layout kv_layout, const int64_t* kv_strides, int causal,
                       float sm_scale, const void* q, const void* k, const void* v, const uint8_t* custom_mask,
                       void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int Hq = num_qo_heads, Hkv = num_kv_heads, Dqk = head_dim_qk, Dvo = head_dim_vo;
  sfa_status st = validate(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, dtype, kv_layout, causal, custom_mask);
  if (st != SFA_OK) return st;
  if (!isfinite(sm_scale) || sm_scale < 0.f) return SFA_ERR_SCALE;
  if (qo_len == 0) return SFA_OK;
  if (!q || !k || !v || !out) return SFA_ERR_NULL;
  // (row, head) element strides of k and v: the layout's contiguous ones unless given
  int64_t ks[2], vs[2];
  if (kv_strides) {
    ks[0] = kv_strides[0]; ks[1] = kv_strides[1]; vs[0] = kv_strides[2]; vs[1] = kv_strides[3];
  } else if (kv_layout == SFA_NHD) {
    ks[0] = (int64_t)Hkv * Dqk; ks[1] = Dqk; vs[0] = (int64_t)Hkv * Dvo; vs[1] = Dvo;
  } else {
    ks[0] = Dqk; ks[1] = (int64_t)kv_len * Dqk; vs[0] = Dvo; vs[1] = (int64_t)kv_len * Dvo;
  }
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return SFA_ERR_LAYOUT;
  for (int i = 0; i < 2; ++i)
    if (ks[i] < 0 || vs[i] < 0 || ks[i] % 8 || vs[i] % 8) return SFA_ERR_LAYOUT;
  if (!sfa::topk_rows_addressable(kv_len, ks[0], Dqk) || !sfa::topk_rows_addressable(kv_len, vs[0], Dvo))
    return SFA_ERR_UNSUPPORTED;
  const bool alias = v == k && vs[0] == ks[0] && vs[1] == ks[1];
  const bool masked = custom_mask != nullptr;
  const PrefillLayout L = layout(qo_len, kv_len, Hq, Hkv, Dqk, Dvo, masked, alias);
  if (!L.ok) return SFA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < L.total) return SFA_ERR_WORKSPACE;

  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  int32_t* d_idx = (int32_t*)(base + L.idx_off);
  int32_t* d_ptr = (int32_t*)(base + L.ptr_off);
  sfa::TopkItem* d_itab = (sfa::TopkItem*)(base + L.itab_off);
  int32_t* d_wptr = masked ? (int32_t*)(base + L.wptr_off) : nullptr;
  {
    const int n = std::max(kv_len, L.items + 1);
    hipLaunchKernelGGL(prefill_tables, dim3(std::min((n + 255) / 256, 1024)), dim3(256), 0, stream, d_idx, d_ptr,
                       d_itab, d_wptr, kv_len, qo_len, L.RS, Hkv, L.items, L.W);
    if (hipGetLastError() != hipSuccess) return SFA_ERR_HIP;
  }
  if (masked) {
    const int64_t n = (int64_t)L.nrb * L.W;
    hipLaunchKernelGGL(prefill_pack_mask, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, custom_mask,
                       qo_len, kv_len, L.RS, Hkv, L.nrb, L.W, (uint32_t*)(base + L.words_off),
                       (int32_t*)(base + L.wflag_off));
    if (hipGetLastError() != hipSuccess) return SFA_ERR_HIP;
  }

  sfa::TopkParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.idx = d_idx;
  p.slot_ptr = d_ptr;
  p.itab = d_itab;
  p.out = (uint16_t*)out;
  p.lse = lse;
  // query vectors through the item table: head stride st[2], row stride st[3]
  p.qs[2] = Dqk; p.qs[3] = (int64_t)Hq * Dqk;
  p.os[2] = Dvo; p.os[3] = (int64_t)Hq * Dvo;
  p.ls[2] = 1;   p.ls[3] = Hq;
  p.ks[0] = 0; p.ks[1] = ks[0]; p.ks[2] = ks[1];
  p.vs[0] = 0; p.vs[1] = vs[0]; p.vs[2] = vs[1];
  if (L.tp.nsplit > 1) {
    p.ws_o = (float*)(base + L.split_off);
    p.ws_ml = p.ws_o + (size_t)L.tp.rows * L.tp.nsplit * L.DV;
  }
  p.B = 1;
  p.S1 = L.items;
  p.S2 = kv_len;
  p.N2 = 1;
  p.G = L.RS * (Hq / Hkv);
  p.HR = Hq / Hkv;
  p.RS = L.RS;
  p.QROWS = qo_len;
  p.topK = kv_len;
  p.causal = (causal && !masked) ? 1 : 0;  // the page: causal applies only without a custom mask
  p.dense = 1;  // the identity key list: a causal item stops at its last row's limit
  p.dk = Dqk;
  p.dv = Dvo;
  p.scale_log2 = (float)((double)(sm_scale > 0.f ? sm_scale : 1.0 / sqrt((double)Dqk)) * 1.4426950408889634);
  if (masked) {
    p.bm_words = (const uint32_t*)(base + L.words_off);
    p.bm_wptr = d_wptr;
    p.bm_wflag = (const int32_t*)(base + L.wflag_off);
  }
  p.nsplit = L.tp.nsplit;
  p.split_len = L.tp.split_len;
  p.HB = L.tp.HB;
  p.n_items = L.tp.grid;
  bool found = false;
  const hipError_t e = sfa::launch_topk(dtype == SFA_FP16, alias, L.DK, L.DV, L.tp, p, stream, &found);
  if (!found) return SFA_ERR_UNSUPPORTED;
  return e == hipSuccess ? SFA_OK : SFA_ERR_HIP;
}

}  // extern "C"
