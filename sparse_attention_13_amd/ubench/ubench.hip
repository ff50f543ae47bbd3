// Microbenchmarks that measure the practical ceilings the attention kernels are judged
// against on one MI355X: streaming copy (HBM), random-row gather of the selected K rows
// (into LDS by direct global->LDS loads, as the attention kernels do, and into registers),
// dense MFMA throughput, and whether one SIMD overlaps MFMA and VALU work.  Built as libsfa_ubench.so and driven by bench.py --ceilings;
// no attention arithmetic lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../csrc/common.hpp"

namespace {

using sfa::u32x4;

// Streaming copy, 16 bytes per lane per access, four accesses in flight per lane.
__global__ __launch_bounds__(256) void ub_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Gather of item `blockIdx.x`'s rows into an LDS ring, as the attention kernels stage them, with
// no compute.  Item t reads rows idx[t * slots .. + slots) of the K slice of batch t / per_batch
// and KV head (t / head_div) % heads: base + batch * batch_bytes + head * head_bytes; a row is RB
// bytes at a pitch of `pitch` bytes.  The
// ring holds NBUF chunks of CH rows; a workgroup of W waves issues one 16-byte piece per lane
// per load.  Every wave waits for its own loads of a chunk, then the workgroup barrier; one word
// of every staged chunk is folded into a checksum written per workgroup (so nothing is idle).
template <int RB, int CH, int NBUF, int W>
__global__ __launch_bounds__(64 * W) void ub_gather_lds(const uint8_t* __restrict__ base, const int32_t* __restrict__ idx,
                                                       int slots, int per_batch, int head_div, int heads,
                                                       int64_t batch_bytes, int64_t head_bytes, int pitch,
                                                       uint32_t* __restrict__ out) {
  constexpr int PIECES = RB / 16;           // 16-byte pieces per row
  constexpr int POS = CH * PIECES;          // pieces per chunk
  constexpr int NT = 64 * W;
  static_assert(POS % NT == 0, "whole rounds");
  constexpr int LPT = POS / NT;             // loads per thread per chunk
  constexpr int BUF = POS * 16;
  extern __shared__ __align__(16) char smem[];
  int* idxl = (int*)(smem + NBUF * BUF);
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* kb = sfa::uniform_ptr(base + (int64_t)(t / per_batch) * batch_bytes +
                                       (int64_t)((t / head_div) % heads) * head_bytes);
  for (int i = tid; i < slots; i += NT) idxl[i] = idx[(int64_t)t * slots + i];
  __syncthreads();
  const uint32_t lds0 = sfa::lds_addr_of(smem);
  const int nchunks = slots / CH;
  auto issue = [&](int c) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int pos = u * NT + tid;
      const int row = idxl[c * CH + pos / PIECES];
      const uint32_t voff = (uint32_t)row * (uint32_t)pitch + (uint32_t)(pos % PIECES) * 16u;
      sfa::lds_dma16_at(kb, voff, lds0 + (c % NBUF) * BUF + (u * NT + wave * 64) * 16);
    }
  };
  uint32_t sum = 0;
  for (int c = 0; c < NBUF - 1 && c < nchunks; ++c) issue(c);
  for (int c = 0; c < nchunks; ++c) {
    // chunk c has landed once at most the later chunks' loads are outstanding
    if (c + NBUF - 2 < nchunks && NBUF > 2) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LPT * (NBUF > 2 ? NBUF - 2 : 0)) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    sum += *(const uint32_t*)(smem + (c % NBUF) * BUF + (tid % (BUF / 4)) * 4);
    __syncthreads();  // everyone read chunk c's buffer before it is refilled
    if (c + NBUF - 1 < nchunks) issue(c + NBUF - 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tid == 0) out[t] = sum;
}

// The same rows gathered into registers with ordinary 16-byte loads (U loads in flight per lane),
// folded into a per-thread checksum.
template <int RB, int W, int U>
__global__ __launch_bounds__(64 * W) void ub_gather_reg(const uint8_t* __restrict__ base, const int32_t* __restrict__ idx,
                                                       int slots, int per_batch, int head_div, int heads,
                                                       int64_t batch_bytes, int64_t head_bytes, int pitch,
                                                       uint32_t* __restrict__ out) {
  constexpr int PIECES = RB / 16;
  constexpr int NT = 64 * W;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t* kb = base + (int64_t)(t / per_batch) * batch_bytes + (int64_t)((t / head_div) % heads) * head_bytes;
  const int32_t* ig = idx + (int64_t)t * slots;
  const int npos = slots * PIECES;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int p0 = tid; p0 < npos; p0 += NT * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = p0 + u * NT;
      v[u] = pos < npos ? *(const u32x4*)(kb + (int64_t)ig[pos / PIECES] * pitch + (pos % PIECES) * 16) : acc;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  out[(int64_t)t * NT + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Dense MFMA throughput: every wave runs CH independent chains of 32x32x16 products.
template <typename T, int CH>
__global__ __launch_bounds__(256) void ub_mfma(float* out, int iters) {
  using vec8 = typename T::vec8;
  sfa::u32x4 ra = {threadIdx.x, threadIdx.x * 3u, 7u, 11u}, rb = {blockIdx.x, 5u, threadIdx.x, 1u};
  ra &= 0x3bff3bffu;  // finite 16-bit values
  rb &= 0x3bff3bffu;
  const vec8 a = sfa::as<vec8>(ra), b = sfa::as<vec8>(rb);
  sfa::f32x16 acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if constexpr (__is_same(T, sfa::half_t))
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Co-execution of MFMA and VALU work on one SIMD.  Eight-wave workgroups, one per CU, so that
// waves w and w + 4 share a SIMD; per iteration a wave runs the MFMA part (8 products of
// 32x32x16 f16 over 4 accumulators), the VALU part (64 fp32 FMAs over 8 chains), or both:
//   mode 0: every wave MFMA;  1: every wave VALU;  2: waves 0-3 MFMA, waves 4-7 VALU (one of
//   each per SIMD);  3: every wave both.
// Overlap across waves would make mode 2 take max(mode 0, mode 1) / 2; none makes it the sum.
template <int MODE>
__global__ __launch_bounds__(512) void ub_coexec(float* out, int iters, float seed) {
  using vec8 = sfa::half_t::vec8;
  const int wave = threadIdx.x >> 6;
  const bool do_mfma = MODE == 0 || MODE == 3 || (MODE == 2 && wave < 4);
  const bool do_valu = MODE == 1 || MODE == 3 || (MODE == 2 && wave >= 4);
  sfa::u32x4 ra = {threadIdx.x, threadIdx.x * 3u, 7u, 11u}, rb = {blockIdx.x, 5u, threadIdx.x, 1u};
  ra &= 0x3bff3bffu;  // finite 16-bit values
  rb &= 0x3bff3bffu;
  const vec8 a = sfa::as<vec8>(ra), b = sfa::as<vec8>(rb);
  sfa::f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = seed * (j + 1) + (float)threadIdx.x;
  for (int i = 0; i < iters; ++i) {
    if (do_mfma) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k & 3], 0, 0, 0);
    }
    if (do_valu) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf(v[j], 0.999f, seed);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
#pragma unroll
  for (int j = 0; j < 8; ++j) s += v[j];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int RB, int CH, int NBUF, int W>
hipError_t launch_lds(const void* base, const int32_t* idx, int items, int slots, int per_batch, int head_div, int heads,
                      int64_t batch_bytes, int64_t head_bytes, int pitch, uint32_t* out, hipStream_t s) {
  constexpr int BUF = CH * RB;
  const int lds = NBUF * BUF + slots * 4;
  if (lds > 160 * 1024 || slots % CH) return hipErrorInvalidValue;
  auto kern = ub_gather_lds<RB, CH, NBUF, W>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(items), dim3(64 * W), lds, s, (const uint8_t*)base, idx, slots, per_batch, head_div,
                     heads, batch_bytes, head_bytes, pitch, out);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16, 16-byte aligned buffers) from src to dst.
int ub_copy_run(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  if (bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) & 15u) return 1;
  int cus = 256;
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0);
  hipLaunchKernelGGL(ub_copy, dim3(cus * 8), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Gathers the rows of `items` work items into LDS (mode 0) or registers (mode 1).  Geometry:
// row bytes rb (256, 384 or 1152), slots per item (a multiple of the chunk), the K slice of item
// t at base + (t / per_batch) * batch_bytes + ((t / head_div) % heads) * head_bytes, rows `pitch`
// bytes apart; idx int32 [items][slots] with values in [0, rows) -- the caller guarantees every
// row lies inside the buffer.  out: uint32 [items] (mode 0) or [items][threads] (mode 1, threads
// = ub_gather_reg_threads(rb)).
int ub_gather_run(int mode, int rb, const void* base, const int32_t* idx, int items, int slots, int per_batch,
                  int head_div, int heads, int64_t batch_bytes, int64_t head_bytes, int pitch, uint32_t* out,
                  hipStream_t s) {
  if (items < 1 || slots < 1 || per_batch < 1 || head_div < 1 || heads < 1) return 1;
  hipError_t e = hipErrorInvalidValue;
  if (mode == 0) {
    // one loader workgroup per item, the ring shapes of the attention kernels' decode forms
    if (rb == 256) e = launch_lds<256, 128, 3, 8>(base, idx, items, slots, per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out, s);
    if (rb == 384) e = launch_lds<384, 32, 2, 2>(base, idx, items, slots, per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out, s);
    if (rb == 1152) e = launch_lds<1152, 32, 3, 4>(base, idx, items, slots, per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out, s);
  } else {
    if (rb == 256) {
      hipLaunchKernelGGL((ub_gather_reg<256, 8, 4>), dim3(items), dim3(512), 0, s, (const uint8_t*)base, idx, slots,
                         per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out);
      e = hipGetLastError();
    } else if (rb == 384) {
      hipLaunchKernelGGL((ub_gather_reg<384, 2, 4>), dim3(items), dim3(128), 0, s, (const uint8_t*)base, idx, slots,
                         per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out);
      e = hipGetLastError();
    } else if (rb == 1152) {
      hipLaunchKernelGGL((ub_gather_reg<1152, 8, 4>), dim3(items), dim3(512), 0, s, (const uint8_t*)base, idx, slots,
                         per_batch, head_div, heads, batch_bytes, head_bytes, pitch, out);
      e = hipGetLastError();
    }
  }
  return e == hipSuccess ? 0 : 2;
}

// Threads per workgroup of the register gather for row bytes rb (sizes its out buffer).
int ub_gather_reg_threads(int rb) { return rb == 384 ? 128 : 512; }

// Dense 32x32x16 MFMA (dtype 0 fp16, 1 bf16): `blocks` workgroups of 4 waves, each wave `iters`
// rounds of 4 independent products.  out: float [blocks * 256].  Flops = blocks * 4 * iters * 4
// * 32768.
int ub_mfma_run(int dtype, int blocks, int iters, float* out, hipStream_t s) {
  if (dtype == 0) hipLaunchKernelGGL((ub_mfma<sfa::half_t, 4>), dim3(blocks), dim3(256), 0, s, out, iters);
  else hipLaunchKernelGGL((ub_mfma<sfa::bfloat_t, 4>), dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// MFMA / VALU co-execution (ub_coexec, modes 0-3): `blocks` workgroups of 8 waves, `iters`
// iterations each.  out: float [blocks * 512].
int ub_coexec_run(int mode, int blocks, int iters, float* out, hipStream_t s) {
  switch (mode) {
    case 0: hipLaunchKernelGGL(ub_coexec<0>, dim3(blocks), dim3(512), 0, s, out, iters, 1e-3f); break;
    case 1: hipLaunchKernelGGL(ub_coexec<1>, dim3(blocks), dim3(512), 0, s, out, iters, 1e-3f); break;
    case 2: hipLaunchKernelGGL(ub_coexec<2>, dim3(blocks), dim3(512), 0, s, out, iters, 1e-3f); break;
    case 3: hipLaunchKernelGGL(ub_coexec<3>, dim3(blocks), dim3(512), 0, s, out, iters, 1e-3f); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
