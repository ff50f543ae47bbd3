// FP8 inputs of the block-sparse run calls (flashinfer.sparse page: run() of
// BlockSparseAttentionWrapper and VariableBlockSparseAttentionWrapper takes scale_q
// [num_qo_heads], scale_k and scale_v [num_kv_heads], per-head factors of FP8 q, k, v).
// The FP8 tensors are expanded once per call into fp16 copies in the caller's workspace,
// each decoded exactly (every E4M3 / E5M2 value is an fp16 value).  The kernels apply the
// factors in fp32: scale * scale_q[h] * scale_k[hk] to each logit, and scale_v[hk] to the
// accumulated output rows (the softmax-weighted sum is linear in v).  The fp16 kernels then
// run on the copies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfa {

// One tensor to expand: n elements (a multiple of 16, 16-byte aligned source and
// destination); element e belongs to head (e / inner) % heads, which selects scale[head]
// (scale NULL: factor 1).  fmt 0 = E4M3, 1 = E5M2 (OCP 8-bit formats).
struct Fp8Job {
  const uint8_t* src;
  uint16_t* dst;
  const float* scale;
  int64_t n, inner;
  int heads, fmt;
};

// Expands up to three tensors in one launch on stream s.
hipError_t launch_fp8_expand(const Fp8Job* jobs, int njobs, hipStream_t s);

// Workspace bytes of the fp16 copies of q (nq elements) and k, v (nkv elements each).
inline size_t fp8_copies_bytes(int64_t nq, int64_t nkv) {
  const auto up = [](int64_t n) { return ((size_t)n * 2 + 255) & ~(size_t)255; };
  return up(nq) + 2 * up(nkv);
}

// Expands q, k and v exactly into the workspace (no factors: the kernels apply them; v reuses
// k's copy when v == k).  kv_inner and Hkv describe the head layout of k and v.  On return
// q16 / k16 / v16 point at the copies.
hipError_t fp8_expand_qkv(const void* q, const void* k, const void* v, int q_fmt, int kv_fmt, int64_t nq,
                          int64_t nkv, int64_t kv_inner, int Hkv, void* workspace, void** q16, void** k16,
                          void** v16, hipStream_t s);

}  // namespace sfa
