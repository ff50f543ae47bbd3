// Block-sparse (BSR) attention kernel for gfx950.
//
// Operator (flashinfer.sparse, BlockSparseAttentionWrapper): q [M, Hq, D] attends
// to k, v [N, Hkv, D] under the boolean mask of a BSR matrix with R x C blocks:
// query row r may see key c iff block (r / R, c / C) is stored.  Each stored
// block's keys are contiguous rows, so the "gather" is a coalesced block load.
//
// Work item: (kv head, block row, query tile).  The R x G query vectors of a block
// row and kv head (G = Hq / Hkv) share the same key list; a workgroup of 4 waves
// takes 64*NQ of them, each wave NQ tiles of 16 (the N dim of the 16x16x32 MFMA),
// and all four waves sweep the same staged 64-key chunks:
//   S^T[32 keys x 16 queries] = K Q^T        (K from LDS, Q in VGPRs)
//   online softmax (fp32, log2 units)
//   O^T[D x 16 queries] += V^T (P_hi + P_lo)^T (V^T by LDS transpose reads)
// Optional bottom-right causal mask: key c is masked for row r when c > r + N - M.
#pragma once

#include "common.hpp"

namespace sfa {

struct BsrParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const int32_t* indptr;   // [MB + 1]
  const int32_t* indices;  // [nnz]
  const int32_t* order;    // [MB] block rows, longest first
  int M, N, R, C, Hq, Hkv, G, causal;
  float scale_log2;
  int MB;
  int QV;  // R * G query vectors per block row
  int QT;  // query tiles (of 64 * NQ) per block row
  int n_items;
};

constexpr int kBsrMaxBlocks = 4096;  // column blocks of one block row staged in LDS

template <typename T, int D, int NQ>
struct BsrCfg {
  static constexpr int NT = 256;
  static constexpr int CH = 64;  // keys per staged chunk
  static constexpr int RB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int LD = CH * CPR / NT;  // 16-byte loads per thread per chunk, per tensor
  static constexpr int KSTEPS = D / 32;
  static constexpr int DT = D / 16;
  static constexpr int BUF = CH * RB;
  static constexpr int LDS_BYTES = 4 * BUF + CH * 4 * 3 + kBsrMaxBlocks * 4;
  static_assert(D % 64 == 0, "head dim");
  static_assert((CH * CPR) % NT == 0, "load split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int NQ>
__global__ __launch_bounds__(256) void bsr_fwd(BsrParams p) {
  using C = BsrCfg<T, D, NQ>;
  using vec8 = typename T::vec8;
  extern __shared__ __align__(16) char smem[];
  char* const kbuf0 = smem;
  char* const kbuf1 = smem + C::BUF;
  char* const vbuf0 = smem + 2 * C::BUF;
  char* const vbuf1 = smem + 3 * C::BUF;
  int* keyl = (int*)(smem + 4 * C::BUF);  // [3][CH] key row of each chunk slot, -1 = none
  int* blkl = keyl + 3 * C::CH;           // [kBsrMaxBlocks] column blocks of this block row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  int item = xcd_remap(blockIdx.x, p.n_items);
  const int qt = item % p.QT;
  item /= p.QT;
  const int bi = item % p.MB;
  const int hk = item / p.MB;
  const int br = p.order[bi];

  const int b0 = p.indptr[br];
  const int nblk = p.indptr[br + 1] - b0;
  const int nkeys = nblk * p.C;
  const int nchunks = (nkeys + C::CH - 1) / C::CH;
  for (int i = tid; i < nblk; i += C::NT) blkl[i] = p.indices[b0 + i];

  // this lane's query vectors (one per query tile)
  int qrow[NQ], qhead[NQ];
  bool qok[NQ];
  int64_t climit[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const int qv = qt * 64 * NQ + (wave * NQ + qi) * 16 + c16;
    const int r = br * p.R + qv / p.G;
    qok[qi] = qv < p.QV && r < p.M;
    qrow[qi] = qok[qi] ? r : 0;
    qhead[qi] = hk * p.G + qv % p.G;
    climit[qi] = p.causal ? (int64_t)qrow[qi] + (p.N - p.M) : (int64_t)0x7fffffffffffLL;
  }
  u32x4 qreg[NQ][C::KSTEPS];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const uint16_t* qp = p.q + ((int64_t)qrow[qi] * p.Hq + qhead[qi]) * D;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[qi][ks] = qok[qi] ? *(const u32x4*)(qp + ks * 32 + g4 * 8) : z;
    }
  }
  __syncthreads();  // blkl visible

  const int64_t kv_row_stride = (int64_t)p.Hkv * D;
  const uint16_t* kg = p.k + (int64_t)hk * D;
  const uint16_t* vg = p.v + (int64_t)hk * D;

  auto key_of = [&](int t) -> int {  // key row of slot t of this block row, -1 past the end
    if (t >= nkeys) return -1;
    const int blk = blkl[t / p.C];
    return blk * p.C + t % p.C;
  };

  u32x4 kst[C::LD], vst[C::LD];
  // key rows of chunk c go to keyl[c % 3]: written before the barrier that precedes the
  // chunk's loads, and not overwritten until every wave is done with chunk c
  auto stage_keys = [&](int c) {
    if (tid < C::CH) keyl[(c % 3) * C::CH + tid] = key_of(c * C::CH + tid);
  };
  auto issue = [&](int c) {
#pragma unroll
    for (int u = 0; u < C::LD; ++u) {
      const int pos = u * C::NT + tid;
      const int r = pos / C::CPR, x = pos % C::CPR;
      const int key = keyl[(c % 3) * C::CH + r];
      const int cc = swz<C::RB>(r, x);
      const int64_t off = (int64_t)(key < 0 ? 0 : key) * kv_row_stride + cc * 8;
      kst[u] = *(const u32x4*)(kg + off);
      vst[u] = *(const u32x4*)(vg + off);
    }
  };
  auto write_staged = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::LD; ++u) {
      *(u32x4*)((buf ? kbuf1 : kbuf0) + (u * C::NT + tid) * 16) = kst[u];
      *(u32x4*)((buf ? vbuf1 : vbuf0) + (u * C::NT + tid) * 16) = vst[u];
    }
  };

  f32x4 acc[NQ][C::DT];
  float m_run[NQ], l_run[NQ];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m_run[qi] = -INFINITY;
    l_run[qi] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[qi][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (nchunks > 0) stage_keys(0);
  if (nchunks > 1) stage_keys(1);
  __syncthreads();
  if (nchunks > 0) {
    issue(0);
    write_staged(0);
    if (nchunks > 1) issue(1);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const char* kb = buf ? kbuf1 : kbuf0;
    const char* vb = buf ? vbuf1 : vbuf0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // two 32-key halves of the chunk
      const int sb = half * 32;
      int kv8[8];
      {
        const int4 j0 = *(const int4*)(keyl + (c % 3) * C::CH + sb + 4 * g4);
        const int4 j1 = *(const int4*)(keyl + (c % 3) * C::CH + sb + 16 + 4 * g4);
        kv8[0] = j0.x; kv8[1] = j0.y; kv8[2] = j0.z; kv8[3] = j0.w;
        kv8[4] = j1.x; kv8[5] = j1.y; kv8[6] = j1.z; kv8[7] = j1.w;
      }
      f32x4 s[NQ][2];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) s[qi][0] = s[qi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r = sb + 16 * t + c16;
          const u32x4 a = *(const u32x4*)(kb + r * C::RB + swz<C::RB>(r, 4 * ks + g4) * 16);
#pragma unroll
          for (int qi = 0; qi < NQ; ++qi) s[qi][t] = T::mfma(as<vec8>(a), as<vec8>(qreg[qi][ks]), s[qi][t]);
        }
      }
      u32x4 phi[NQ], plo[NQ];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        float x[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int key = kv8[i];
          const bool ok = key >= 0 && (int64_t)key <= climit[qi];
          x[i] = ok ? s[qi][i >> 2][i & 3] * p.scale_log2 : -INFINITY;
          cmax = fmaxf(cmax, x[i]);
        }
        cmax = wave_max_across_groups(cmax);
        const bool bump = cmax > m_run[qi] + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(bump)) {
          const float m_new = bump ? cmax : m_run[qi];
          const float alpha = fast_exp2(m_run[qi] - m_new);
          l_run[qi] *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) scale_acc<4>(acc[qi][dt], alpha);
          m_run[qi] = m_new;
        }
        const float m_use = m_run[qi] == -INFINITY ? 0.f : m_run[qi];
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = fast_exp2(x[i] - m_use);
          psum += pv[i];
        }
        l_run[qi] += psum;
        split_hi_lo<T>(pv, phi[qi], plo[qi]);
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        u32x2 lo_half, hi_half;
        {
          const int r = sb + 4 * g4 + (c16 >> 2);
          const int cc = 2 * dt + ((c16 & 3) >> 1);
          lo_half = lds_read_tr16(vb + r * C::RB + swz<C::RB>(r, cc) * 16 + (c16 & 1) * 8);
        }
        {
          const int r = sb + 16 + 4 * g4 + (c16 >> 2);
          const int cc = 2 * dt + ((c16 & 3) >> 1);
          hi_half = lds_read_tr16(vb + r * C::RB + swz<C::RB>(r, cc) * 16 + (c16 & 1) * 8);
        }
        const u32x4 a = {lo_half[0], lo_half[1], hi_half[0], hi_half[1]};
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
          acc[qi][dt] = T::mfma(as<vec8>(a), as<vec8>(phi[qi]), acc[qi][dt]);
          acc[qi][dt] = T::mfma(as<vec8>(a), as<vec8>(plo[qi]), acc[qi][dt]);
        }
      }
    }
    if (c + 1 < nchunks) write_staged(buf ^ 1);
    if (c + 2 < nchunks) stage_keys(c + 2);
    __syncthreads();
    if (c + 2 < nchunks) issue(c + 2);
  }

#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float l_tot = wave_sum_across_groups(l_run[qi]);
    if (!qok[qi]) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.out + ((int64_t)qrow[qi] * p.Hq + qhead[qi]) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      u32x2 w;
      w[0] = (uint32_t)T::from_float(acc[qi][dt][0] * inv) | ((uint32_t)T::from_float(acc[qi][dt][1] * inv) << 16);
      w[1] = (uint32_t)T::from_float(acc[qi][dt][2] * inv) | ((uint32_t)T::from_float(acc[qi][dt][3] * inv) << 16);
      *(u32x2*)(orow + dt * 16 + 4 * g4) = w;
    }
    if (p.lse && g4 == 0)
      p.lse[(int64_t)qrow[qi] * p.Hq + qhead[qi]] =
          l_tot > 0.f ? (m_run[qi] + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace sfa
