// Device-side building blocks shared by the gfx950 kernels of libsfa:
// vector types, the 16x16x32 MFMA wrappers, fp16/bf16 conversions, the LDS
// transpose read and the XOR swizzle of staged K/V rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element type tags.  Storage is always 16-bit; the MFMA operand type differs.
struct half_t {
  using vec8 = f16x8;
  static __device__ __forceinline__ float to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

struct bfloat_t {
  using vec8 = bf16x8;
  static __device__ __forceinline__ float to_float(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
  }
  static __device__ __forceinline__ uint16_t from_float(float x) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename V>
__device__ __forceinline__ V as(u32x4 x) {
  return __builtin_bit_cast(V, x);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as two 16-bit T in one word (round to nearest even; one v_cvt_pk_*_f32).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (__is_same(T, half_t)) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Packs 8 fp32 values as the 16-bit type T (round to nearest even).
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float* x) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack2<T>(x[2 * i], x[2 * i + 1]);
  return r;
}

// The two 16-bit halves of a pair of fp32 values, hi = round(x), lo = round(x - hi) (x - hi is
// exact in fp32): the pair carries about twice the significand bits of T into a T x T
// contraction.  fp16: lo comes from mixed-precision FMAs (x - hi from the fp16 hi and the fp32
// x, rounded to fp16 in the same instruction); bf16: hi is widened by a shift or a mask.
template <typename T>
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2<T>(a, b);
  if constexpr (__is_same(T, half_t)) {
    uint32_t l;
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=&v"(l)
        : "v"(hi), "v"(a), "v"(b));
    lo = l;
  } else {
    lo = pack2<T>(a - __builtin_bit_cast(float, hi << 16), b - __builtin_bit_cast(float, hi & 0xffff0000u));
  }
}

template <typename T>
__device__ __forceinline__ void split_hi_lo(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h, l;
    split2<T>(x[2 * i], x[2 * i + 1], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// Staged-row layout of the top-K kernels.  A row of CPR 16-byte chunks occupies
// staged_stride(CPR) chunk positions, with stride = 4 * odd (mod 16) in chunks, and
// chunk cc of row r sits at position r * stride + (cc & ~3) + ((cc & 3) ^ stage_xor(r)).
// With 64 LDS banks of 4 bytes this keeps conflict-free:
//  * 16 lanes reading the same chunk of 16 consecutive rows (MFMA K operand), and
//  * the transpose reads of 4 consecutive rows x 64 bytes, or of 8 rows x 32 bytes.
// The XOR only touches the low two chunk bits, so operand addresses of successive
// k-steps / dv tiles differ by compile-time offsets.
constexpr int staged_stride(int cpr) {
  int s = cpr;
  while (s % 16 != 4 && s % 16 != 12) ++s;
  return s;
}

__device__ __forceinline__ int stage_xor(int r) { return ((r >> 1) & 2) | ((r >> 3) & 1); }

// chunk position of chunk (cc_hi + cc_lo) of row r; cc_hi a multiple of 4, cc_lo in [0, 4)
template <int STRIDE>
__device__ __forceinline__ int stage_pos(int r, int cc_hi, int cc_lo) {
  return r * STRIDE + cc_hi + (cc_lo ^ stage_xor(r));
}

// Pad-free staged layouts for 16-wide head tiles: a row of KCPR chunks occupies exactly KCPR
// chunk positions, and chunk cc of row r sits at r * KCPR + (cc & ~(S - 1)) +
// ((cc ^ stage_xor_pf<S>(r)) & (S - 1)), with swizzle group S = 8 for KCPR = 8 mod 16 and
// S = 16 for KCPR = 0 mod 16.  The reads are the K operand (16 consecutive rows, one chunk,
// ds_read_b128) and the transposes (rows 4m .. 4m + 3, two adjacent chunks,
// ds_read_b64_tr_b16).  The LDS does not serve a 16-byte read as 16 lanes over 256 bytes in
// lane order (a probe replaying these patterns against the bank-conflict counter shows
// two-way conflicts for layouts that meet that rule), so the XOR values come from that
// measurement:
//  * S = 8: 0, 1, 5, 4, 3, 2, 6, 7 for r mod 8 -- both reads conflict-free for every chunk
//    offset and whole 8-row offsets (the prefill kernel's LDS conflict cycles went from 0.39
//    of its active LDS cycles to 0, its time by ~1%);
//  * S = 16: 2 (r mod 8) + (r / 8 mod 2) -- transposes conflict-free, K operand reads two-way.
//    (9 r mod 16) ^ (4 if r mod 16 >= 8) measured conflict-free for both but was not faster
//    on the decode kernel (20.6 against 20.5 us), which keeps this one.
template <int S>
__device__ __forceinline__ int stage_xor_pf(int r) {
  if constexpr (S == 8) {
    return (0x76234510 >> (4 * (r & 7))) & 7;
  } else {
    static_assert(S == 16, "swizzle group");
    return 2 * (r & 7) + ((r >> 3) & 1);
  }
}

// XOR of the wide-value kernel's staged rows (padded stride, chunk cc of row r at position
// r * stride + (cc & ~7) + ((cc ^ stage_xor_w(r)) & 7)), over groups of 8 chunks: [0, 1, 7, 6]
// by r mod 4, complemented when r mod 16 >= 8.  Chosen by measurement like stage_xor_pf: the
// K operand reads (16 consecutive rows, one chunk) and the transposes (rows 4m .. 4m + 3, two
// adjacent chunks) are conflict-free at the 1216- and 1088-byte row pitches of Dk = 576 and
// 512 for every chunk and ring-buffer offset, where the 2-bit stage_xor gave two-way conflicts
// for both.
__device__ __forceinline__ int stage_xor_w(int r) {
  return ((0x6710 >> (4 * (r & 3))) & 7) ^ (((r >> 3) & 1) * 7);
}

// LDS transpose read of four 16-bit values (gfx950 ds_read_b64_tr_b16).  Inside
// each group of 16 lanes, lane i receives element (i % 4) of the 8-byte words
// addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in that order.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(void*)lds_ptr);
  return __builtin_bit_cast(u32x2, v);
}

// DPP row_ror:8 inside each row of 16 lanes (lane l <- lane l ^ 8), written only to the
// 4-lane banks of a row selected by BANKS (bit i: lanes 4i .. 4i + 3); other lanes keep x.
template <int BANKS>
__device__ __forceinline__ uint32_t ror8_into(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xF, BANKS, false);
}
__device__ __forceinline__ float xor8_lane(float x) {
  return __uint_as_float(ror8_into<0xF>(__float_as_uint(x)));
}

// Reductions over the lanes that share an MFMA output column: lanes l, l + MT, ...
// Done with the gfx950 lane swaps (VALU, no LDS round trip): permlane16_swap of a value with
// itself leaves x[l] in one result and x[l ^ 16] in the other, permlane32_swap the same for
// l ^ 32, so combining the two results reduces over that lane pair in every lane.  (With
// ds_bpermute each step was an LDS round trip on the softmax's dependent chain: GQA prefill
// 273 -> 254 us.)
// MT = 8 (packed 16-wide tiles) also reduces over lanes l and l ^ 8 (a DPP row rotation).
template <int MT>
__device__ __forceinline__ float wave_max_lanes(float x) {
  if constexpr (MT <= 8) x = fmaxf(x, xor8_lane(x));
  if constexpr (MT <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int MT>
__device__ __forceinline__ float wave_sum_lanes(float x) {
  if constexpr (MT <= 8) x += xor8_lane(x);
  if constexpr (MT <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max_across_groups(float x) { return wave_max_lanes<16>(x); }
__device__ __forceinline__ float wave_sum_across_groups(float x) { return wave_sum_lanes<16>(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The online softmax keeps its reference max until a chunk exceeds it by more than this
// (log2 units), so probabilities stay <= 2^8 (well inside fp16 range) and the O
// accumulators are rescaled only when the reference moves.
constexpr float kLazyRescale = 8.f;

// Multiplies MFMA accumulators in place by s.  The library is built with the MFMA operands
// and results in ordinary VGPRs (gfx950 allows both forms), so this is a plain multiply.
template <int N, typename V>
__device__ __forceinline__ void scale_acc(V& acc, float s) {
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] *= s;
}

// 16-byte global -> LDS load (gfx950 global_load_lds_dwordx4).  lds_addr (an LDS byte
// address, see lds_addr_of) must be the same for all lanes of the wave; lane i's 16 bytes
// land at lds_addr + 16 * i.  Completion is tracked by vmcnt, and the caller owns the wait:
// the instruction is issued from inline asm so that the compiler's wait tracking does not
// see an LDS write in flight.  (Seen, it makes every later LDS read that lacks alias
// information -- the transposing ds_read_b64_tr_b16 among them -- wait for vmcnt(0), that
// is for the whole prefetch ring.)  The caller makes the data visible with an explicit
// s_waitcnt vmcnt + s_barrier.
// Wait states: the compiler cannot see that the asm holds a memory instruction, so it does
// not pad the hazards before it.  A vector-memory instruction that reads an SGPR (M0, or the
// base pair of lds_dma16_at) needs 5 wait states after a VALU instruction that wrote it
// (v_readfirstlane, or v_readlane restoring a spilled SGPR -- the compiler emits both right
// before these loads under register pressure), 1 after a SALU write of M0.  With fewer the
// load can take the register's previous value: a wild address.  SFA_DMA_NOPS provides the 5.
#define SFA_DMA_NOPS "s_nop 4\n\t"
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile(SFA_DMA_NOPS "global_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// 4-byte global -> LDS load (global_load_lds_dword): lane i's word lands at lds_addr + 4 * i.
// Same contract as lds_dma16.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile(SFA_DMA_NOPS "global_load_lds_dword %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// The same 16-byte load with the address split into a wave-uniform 64-bit base (SGPRs) and
// a per-lane 32-bit byte offset: address = base + voff (global_load_lds_dwordx4 v, s[:]).
// The offset arithmetic stays 32-bit (full-rate VALU) instead of a 64-bit multiply-add.
// A pointer whose value is the same in every lane, held in SGPRs.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (P*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// base must be wave-uniform; it is re-read from the first lane so the asm operand is an SGPR
// pair wherever the compiler kept the value.
__device__ __forceinline__ void lds_dma16_at(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile(SFA_DMA_NOPS "global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(base)), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// LDS byte address of a pointer into a __shared__ array (as a constant offset from it).
template <typename P>
__device__ __forceinline__ uint32_t lds_addr_of(P* shared_array) {
  typedef __attribute__((address_space(3))) P lds_p;
  return (uint32_t)(uintptr_t)(lds_p*)shared_array;
}

// Maps a launch index to a work item so that consecutive work items land on the
// same XCD (blocks are dealt round-robin to the 8 XCDs of an MI355X).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int x = bid % kXcd, k = bid / kXcd;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return start + k;
}

}  // namespace sfa
