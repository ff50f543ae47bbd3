// C-ABI entry points of libsfa: argument validation (the rules of the
// SparseFlashAttention operator page, section 3, and of the BSR wrapper's
// plan()), stride normalisation, launch configuration and kernel launch.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/sfa.h"
#include "topk_launch.hpp"

namespace {

using sfa::TopkParams;
using sfa::TopkPlan;

bool log_enabled() {
  static const bool on = getenv("SFA_LOG") != nullptr;
  return on;
}

sfa_status validate_shape(const sfa_shape* s, sfa_dtype dtype, int causal) {
  if (!s) return SFA_ERR_NULL;
  if (dtype != SFA_FP16 && dtype != SFA_BF16) return SFA_ERR_DTYPE;
  if (s->B < 0 || s->S1 < 0 || s->S2 < 1 || s->N1 < 1 || s->N2 < 1) return SFA_ERR_SHAPE;
  if (s->N1 % s->N2 != 0) return SFA_ERR_GQA;
  if (s->Dk < 64 || s->Dv < 64 || s->Dk % 64 || s->Dv % 64 || s->Dv > s->Dk) return SFA_ERR_HEAD_DIM;
  if (s->topK < 1 || s->topK > s->S2) return SFA_ERR_TOPK;
  if (causal && s->S1 > s->S2) return SFA_ERR_CAUSAL;
  return SFA_OK;
}

// Launch plan on the compiled head-dim pair that serves (Dk, Dv); WS == 0 when there is none.
TopkPlan plan_topk(const sfa_shape* s, bool alias) {
  int DK = 0, DV = 0;
  if (!sfa::topk_kernel_dims(s->Dk, s->Dv, &DK, &DV)) return TopkPlan{};
  return sfa::plan_topk((int64_t)s->B * s->S1 * s->N2, s->N1 / s->N2, s->topK, DK, DV, alias,
                        sfa::device_cu_count());
}

void contiguous_strides(const sfa_shape* s, sfa_layout layout, sfa_strides* st) {
  // layout-order strides of contiguous tensors
  auto fill = [&](int64_t* o, int64_t S, int64_t N, int64_t D) {
    if (layout == SFA_BSND) {
      o[0] = S * N * D; o[1] = N * D; o[2] = D;
    } else {
      o[0] = N * S * D; o[1] = S * D; o[2] = D;
    }
  };
  fill(st->q, s->S1, s->N1, s->Dk);
  fill(st->k, s->S2, s->N2, s->Dk);
  fill(st->v, s->S2, s->N2, s->Dv);
  fill(st->idx, s->S1, s->N2, s->topK);
  fill(st->out, s->S1, s->N1, s->Dv);
}

// layout-order (b, x, y) -> canonical (batch, seq, head)
void canon(const int64_t* in, sfa_layout layout, int64_t* out) {
  out[0] = in[0];
  if (layout == SFA_BSND) {
    out[1] = in[1]; out[2] = in[2];
  } else {
    out[1] = in[2]; out[2] = in[1];
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool strides_ok(const int64_t* st, int64_t mult) {
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % mult) return false;
  return true;
}

}  // namespace

extern "C" {

const char* sfa_status_str(sfa_status status) {
  switch (status) {
    case SFA_OK: return "ok";
    case SFA_ERR_NULL: return "a required pointer is NULL";
    case SFA_ERR_DTYPE: return "dtype must be fp16 or bf16";
    case SFA_ERR_LAYOUT: return "layout must be BSND or BNSD with 16-byte aligned rows";
    case SFA_ERR_SHAPE: return "invalid problem size";
    case SFA_ERR_GQA: return "query heads must be a multiple of key/value heads";
    case SFA_ERR_HEAD_DIM: return "head dims must be positive multiples of 64 with Dv <= Dk";
    case SFA_ERR_TOPK: return "topK must lie in [1, S2]";
    case SFA_ERR_CAUSAL: return "causal attention requires S1 <= S2";
    case SFA_ERR_SCALE: return "scale must be finite and > 0";
    case SFA_ERR_WORKSPACE: return "workspace missing or too small";
    case SFA_ERR_PLAN: return "missing plan or malformed block-sparse pattern";
    case SFA_ERR_INDEX: return "block column index out of range or repeated";
    case SFA_ERR_UNSUPPORTED: return "head dim above 576 or a size beyond the kernels' addressing";
    case SFA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t sfa_workspace_bytes(const sfa_shape* shape, sfa_dtype dtype, int causal) {
  if (validate_shape(shape, dtype, causal) != SFA_OK) return 0;
  if (shape->B == 0 || shape->S1 == 0) return 0;
  // the alias decision does not change the split (it only changes WS for large dims): take the larger need
  const TopkPlan a = plan_topk(shape, true), b = plan_topk(shape, false);
  return a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
}

sfa_status sfa_run(const sfa_shape* shape, const sfa_strides* strides, sfa_dtype dtype, sfa_layout layout,
                   int causal, float scale, const void* q, const void* k, const void* v,
                   const int32_t* sparse_indices, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  sfa_status st = validate_shape(shape, dtype, causal);
  if (st != SFA_OK) return st;
  if (layout != SFA_BSND && layout != SFA_BNSD) return SFA_ERR_LAYOUT;
  if (!(scale > 0.f) || !isfinite(scale)) return SFA_ERR_SCALE;
  if (shape->B == 0 || shape->S1 == 0) return SFA_OK;
  if (!q || !k || !v || !sparse_indices || !out) return SFA_ERR_NULL;
  int DK = 0, DV = 0;  // compiled head dims of the kernels that serve this call
  if (!sfa::topk_kernel_dims(shape->Dk, shape->Dv, &DK, &DV)) return SFA_ERR_UNSUPPORTED;

  sfa_strides sd;
  if (strides) sd = *strides;
  else contiguous_strides(shape, layout, &sd);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sparse_indices) || !aligned16(out))
    return SFA_ERR_LAYOUT;
  if (!strides_ok(sd.q, 8) || !strides_ok(sd.k, 8) || !strides_ok(sd.v, 8) || !strides_ok(sd.out, 8) ||
      !strides_ok(sd.idx, 1))
    return SFA_ERR_LAYOUT;

  const bool alias = v == k && sd.v[0] == sd.k[0] && sd.v[1] == sd.k[1] && sd.v[2] == sd.k[2];
  {
    int64_t ks[3], vs[3];
    canon(sd.k, layout, ks);
    canon(sd.v, layout, vs);
    if (!sfa::topk_rows_addressable(shape->S2, ks[1], shape->Dk) ||
        !sfa::topk_rows_addressable(shape->S2, vs[1], shape->Dv))
      return SFA_ERR_UNSUPPORTED;
  }
  const TopkPlan pl = plan_topk(shape, alias);
  if (pl.WS < 1) return SFA_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return SFA_ERR_WORKSPACE;
  if ((int64_t)pl.grid > 0x7fffffffLL) return SFA_ERR_UNSUPPORTED;

  TopkParams p;
  memset(&p, 0, sizeof p);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.idx = sparse_indices;
  p.out = (uint16_t*)out;
  p.lse = lse;
  canon(sd.q, layout, p.qs);
  canon(sd.k, layout, p.ks);
  canon(sd.v, layout, p.vs);
  canon(sd.idx, layout, p.is);
  canon(sd.out, layout, p.os);
  {
    const int64_t S1 = shape->S1, N1 = shape->N1;
    if (layout == SFA_BSND) {
      p.ls[0] = S1 * N1; p.ls[1] = N1; p.ls[2] = 1;
    } else {
      p.ls[0] = N1 * S1; p.ls[1] = 1; p.ls[2] = S1;
    }
  }
  p.qs[3] = p.os[3] = p.ls[3] = 0;  // one query row per item row
  if (pl.nsplit > 1) {
    float* ws = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    p.ws_o = ws;
    p.ws_ml = ws + (size_t)pl.rows * pl.nsplit * DV;
  }
  p.B = shape->B;
  p.S1 = shape->S1;
  p.S2 = shape->S2;
  p.N2 = shape->N2;
  p.G = shape->N1 / shape->N2;
  p.HR = p.G;
  p.RS = 1;
  p.QROWS = shape->S1;
  p.topK = shape->topK;
  p.causal = causal ? 1 : 0;
  p.dk = shape->Dk;
  p.dv = shape->Dv;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.nsplit = pl.nsplit;
  p.split_len = pl.split_len;
  p.HB = pl.HB;
  p.n_items = pl.grid;

  bool found = false;
  hipError_t e = sfa::launch_topk(dtype == SFA_FP16, alias, DK, DV, pl, p, stream, &found);
  if (!found) return SFA_ERR_UNSUPPORTED;
  if (e != hipSuccess) {
    if (log_enabled()) fprintf(stderr, "sfa_run: %s\n", hipGetErrorString(e));
    return SFA_ERR_HIP;
  }
  if (log_enabled())
    fprintf(stderr, "sfa_run: kernel dims %dx%d MT=%d WH=%d WS=%d HB=%d nsplit=%d split_len=%d grid=%d alias=%d\n",
            DK, DV, pl.MT, pl.WH, pl.WS, pl.HB, pl.nsplit, pl.split_len, pl.grid, (int)alias);
  return SFA_OK;
}

}  // extern "C"
