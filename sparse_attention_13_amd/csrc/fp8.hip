// Expansion of FP8 (OCP E4M3 / E5M2) tensors with per-head factors into fp16.
//
// Memory-bound elementwise pass: every lane reads 16 codes (one 16-byte load, lanes of
// a wave cover 1 KB contiguously) and writes 16 fp16 values (two 16-byte stores).  The
// decode is exact (every E4M3 / E5M2 value is an fp16 value); a job with a factor applies
// it in fp32 and rounds the product once more to fp16 (the attention calls pass none).
#include "fp8.hpp"

#include "common.hpp"
#include "topk_launch.hpp"

namespace sfa {
namespace {

struct Fp8Args {
  Fp8Job job[3];
};

// Value of one code.  E4M3: bias 7, exponent field 15 with mantissa 7 is NaN, no
// infinities.  E5M2: bias 15, exponent field 31 is infinity (mantissa 0) or NaN.
// Normal codes become the float whose exponent field is e - bias + 127 and whose top
// mantissa bits are the code's; subnormal codes are m * 2^(1 - bias - mantissa bits).
__device__ __forceinline__ float fp8_value(uint32_t b, int fmt) {
  const uint32_t sign = (b & 0x80u) << 24;
  uint32_t bits;
  if (fmt == 0) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return __builtin_bit_cast(float, sign | 0x7fc00000u);
    if (e == 0u) return __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, (float)m * 0x1p-9f));
    bits = ((e + 120u) << 23) | (m << 20);
  } else {
    const uint32_t e = (b >> 2) & 31u, m = b & 3u;
    if (e == 31u) return __builtin_bit_cast(float, sign | (m ? 0x7fc00000u : 0x7f800000u));
    if (e == 0u) return __builtin_bit_cast(float, sign | __builtin_bit_cast(uint32_t, (float)m * 0x1p-16f));
    bits = ((e + 112u) << 23) | (m << 21);
  }
  return __builtin_bit_cast(float, sign | bits);
}

__global__ __launch_bounds__(256) void fp8_expand(Fp8Args a) {
  const Fp8Job& j = a.job[blockIdx.y];
  const int64_t n16 = j.n >> 4;
  const u32x4* src = (const u32x4*)j.src;
  u32x4* dst = (u32x4*)j.dst;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 w = __builtin_nontemporal_load(&src[i]);
    const float f = j.scale ? j.scale[((i << 4) / j.inner) % j.heads] : 1.f;
    float x[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) x[c] = fp8_value((w[c >> 2] >> (8 * (c & 3))) & 0xffu, j.fmt) * f;
    dst[2 * i] = pack8<half_t>(x);
    dst[2 * i + 1] = pack8<half_t>(x + 8);
  }
}

}  // namespace

hipError_t launch_fp8_expand(const Fp8Job* jobs, int njobs, hipStream_t s) {
  if (njobs < 1 || njobs > 3) return hipErrorInvalidValue;
  Fp8Args a;
  int64_t most = 0;
  for (int i = 0; i < njobs; ++i) {
    a.job[i] = jobs[i];
    if (jobs[i].n > most) most = jobs[i].n;
  }
  if (most == 0) return hipSuccess;
  // enough workgroups to keep every CU streaming, each lane a few 16-code groups
  const int64_t want = (most / 16 + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int gx = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL(fp8_expand, dim3(gx, njobs), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t fp8_expand_qkv(const void* q, const void* k, const void* v, int q_fmt, int kv_fmt, int64_t nq,
                          int64_t nkv, int64_t kv_inner, int Hkv, void* workspace, void** q16, void** k16,
                          void** v16, hipStream_t s) {
  uint8_t* w = (uint8_t*)workspace;
  const size_t qb = ((size_t)nq * 2 + 255) & ~(size_t)255, kb = ((size_t)nkv * 2 + 255) & ~(size_t)255;
  *q16 = w;
  *k16 = w + qb;
  const bool shared = v == k;
  *v16 = shared ? *k16 : (void*)(w + qb + kb);
  Fp8Job jobs[3] = {
      {(const uint8_t*)q, (uint16_t*)*q16, nullptr, nq, nq, 1, q_fmt},
      {(const uint8_t*)k, (uint16_t*)*k16, nullptr, nkv, nkv, 1, kv_fmt},
      {(const uint8_t*)v, (uint16_t*)*v16, nullptr, nkv, kv_inner, Hkv, kv_fmt},
  };
  return launch_fp8_expand(jobs, shared ? 2 : 3, s);
}

}  // namespace sfa
