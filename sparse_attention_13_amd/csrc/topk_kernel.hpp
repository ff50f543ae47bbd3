// Top-K sparse flash attention kernels for gfx950.
//
// Operator (SparseFlashAttention operator page, section 2): for each query row
// (b, s1, n1), gather the topK key/value rows named by the index row of its
// KV-head group (b, s1, n2 = n1 / G), take softmax(q K_sel^T * scale) over the
// topK axis after the optional bottom-right causal mask, and multiply by V_sel.
//
// Work decomposition.  A work item is (group (b, n2, s1), head block, split):
// the G query heads of a group share one index row, so one gathered K/V tile
// in LDS serves all of them.  A workgroup has WH x WS waves: WH head tiles of 16
// heads each (the N dim of the 16x16x32 MFMAs) times WS waves that take
// disjoint 32-slot parts of each staged chunk of CH = 32*WS slots.
//
// Per chunk:  registers <- gathered 16-byte pieces of the CH selected rows
// (global loads issued one chunk ahead), then LDS (XOR-swizzled rows), then per
// wave:
//   S^T[32 slots x 16 heads] = K_sel Q^T        (MFMA, K from LDS, Q in VGPRs)
//   online softmax in fp32, log2 domain          (one head per lane column)
//   O^T[Dv x 16 heads] += V_sel^T (P_hi + P_lo)^T (MFMA, V^T by LDS transpose reads)
// P enters the PV product as two 16-bit parts (hi = round(P), lo = round(P - hi))
// so the product carries about 16 (bf16) / 22 (fp16) significand bits of P.
//
// A split of the topK axis (decode shapes with few groups) writes the partial
// (O, running max, running sum) to the float workspace; topk_merge combines the
// splits with the log-sum-exp rule.
#pragma once

#include "common.hpp"

namespace sfa {

struct TopkParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  float* lse;
  float* ws_o;   // [rows, nsplit, Dv] partial outputs (unnormalised)
  float* ws_ml;  // [rows, nsplit, 2] (running max in log2 units, running sum)
  // element strides of (batch, seq, head) for each tensor
  int64_t qs[3], ks[3], vs[3], is[3], os[3], ls[3];
  int B, S1, S2, N1, N2, G, topK, causal;
  float scale_log2;  // scale * log2(e)
  int nsplit, split_len, HB;
  int n_items;
};

constexpr int kMaxSplitLen = 2048;  // index slots staged in LDS per work item

template <typename T, int DK, int DV, bool ALIAS, int WH, int WS>
struct TopkCfg {
  static constexpr int NT = 64 * WH * WS;  // threads
  static constexpr int CH = 32 * WS;       // slots per staged chunk
  static constexpr int KB = DK * 2;        // bytes per staged K row
  static constexpr int VB = ALIAS ? KB : DV * 2;
  static constexpr int KCPR = DK / 8;  // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;
  static constexpr int KLD = CH * KCPR / NT;  // 16-byte loads per thread per chunk
  static constexpr int VLD = ALIAS ? 0 : CH * VCPR / NT;
  static constexpr int KSTEPS = DK / 32;
  static constexpr int DT = DV / 16;
  static constexpr int KBUF = CH * KB;
  static constexpr int VBUF = ALIAS ? 0 : CH * VB;
  static constexpr int LDS_BYTES = 2 * (KBUF + VBUF) + kMaxSplitLen * 4;
  static_assert(DK % 64 == 0 && DV % 64 == 0 && DV <= DK, "head dims");
  static_assert((CH * KCPR) % NT == 0 && (ALIAS || (CH * VCPR) % NT == 0), "load split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // cross-wave merge of WS slot parts reuses the chunk buffers
  static_assert(WS == 1 || WS * WH * 16 * (DV + 2) * 4 <= 2 * (KBUF + VBUF), "merge scratch");
};

template <typename T, int DK, int DV, bool ALIAS, int WH, int WS>
__global__ __launch_bounds__(64 * WH * WS) void topk_fwd(TopkParams p) {
  using C = TopkCfg<T, DK, DV, ALIAS, WH, WS>;
  using vec8 = typename T::vec8;
  extern __shared__ __align__(16) char smem[];
  char* kbuf0 = smem;
  char* kbuf1 = smem + C::KBUF;
  char* vbuf0 = smem + 2 * C::KBUF;
  char* vbuf1 = vbuf0 + C::VBUF;
  int* idxl = (int*)(smem + 2 * (C::KBUF + C::VBUF));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wh = wave % WH;
  const int wsl = wave / WH;
  const int g4 = lane >> 4;  // lane group 0..3
  const int c16 = lane & 15;

  // ---- work item
  int item = xcd_remap(blockIdx.x, p.n_items);
  const int hb = item % p.HB;
  item /= p.HB;
  const int split = item % p.nsplit;
  item /= p.nsplit;
  const int s1 = item % p.S1;
  item /= p.S1;
  const int n2 = item % p.N2;
  const int b = item / p.N2;

  const int slot0 = split * p.split_len;
  const int nslots = min(p.split_len, p.topK - slot0);
  const int nchunks = (nslots + C::CH - 1) / C::CH;

  const int head = hb * 16 * WH + wh * 16 + c16;  // head within the group (this lane's column)
  const bool head_ok = head < p.G;
  const int n1 = n2 * p.G + (head_ok ? head : 0);

  const uint16_t* kg = p.k + (int64_t)b * p.ks[0] + (int64_t)n2 * p.ks[2];
  const uint16_t* vg = p.v + (int64_t)b * p.vs[0] + (int64_t)n2 * p.vs[2];

  // ---- stage this split's indices: row index, or -1 for a masked / padded / out-of-range slot
  {
    const int32_t* ig = p.idx + (int64_t)b * p.is[0] + (int64_t)s1 * p.is[1] + (int64_t)n2 * p.is[2];
    const int64_t climit = (int64_t)s1 + (p.S2 - p.S1);
    for (int i = tid; i < nchunks * C::CH; i += C::NT) {
      int j = -1;
      if (i < nslots) {
        j = ig[slot0 + i];
        if (j < 0 || j >= p.S2 || (p.causal && j > climit)) j = -1;
      }
      idxl[i] = j;
    }
  }

  // ---- Q^T operand: lane holds q[head][32*ks + 8*g4 .. +7]
  u32x4 qreg[C::KSTEPS];
  {
    const uint16_t* qrow = p.q + (int64_t)b * p.qs[0] + (int64_t)s1 * p.qs[1] + (int64_t)n1 * p.qs[2];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qreg[ks] = head_ok ? *(const u32x4*)(qrow + ks * 32 + g4 * 8) : z;
    }
  }
  __syncthreads();

  // ---- gather: registers <- global, then LDS (swizzled)
  u32x4 kst[C::KLD];
  u32x4 vst[C::VLD > 0 ? C::VLD : 1];
  auto issue_gather = [&](int c) {
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) {
      const int pos = u * C::NT + tid;
      const int r = pos / C::KCPR, x = pos % C::KCPR;
      const int j = idxl[c * C::CH + r];
      const int cc = swz<C::KB>(r, x);
      kst[u] = *(const u32x4*)(kg + (int64_t)(j < 0 ? 0 : j) * p.ks[1] + cc * 8);
    }
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < C::VLD; ++u) {
        const int pos = u * C::NT + tid;
        const int r = pos / C::VCPR, x = pos % C::VCPR;
        const int j = idxl[c * C::CH + r];
        const int cc = swz<C::VB>(r, x);
        vst[u] = *(const u32x4*)(vg + (int64_t)(j < 0 ? 0 : j) * p.vs[1] + cc * 8);
      }
    }
  };
  auto write_staged = [&](char* kb, char* vb) {
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) *(u32x4*)(kb + (u * C::NT + tid) * 16) = kst[u];
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < C::VLD; ++u) *(u32x4*)(vb + (u * C::NT + tid) * 16) = vst[u];
    }
  };

  // ---- running state (per lane: head = c16; O^T rows dv = 16*dt + 4*g4 + e)
  f32x4 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (nchunks > 0) {
    issue_gather(0);
    write_staged(kbuf0, vbuf0);
    if (nchunks > 1) issue_gather(1);
  }
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const char* kb = (c & 1) ? kbuf1 : kbuf0;
    const char* vb = ALIAS ? kb : ((c & 1) ? vbuf1 : vbuf0);
    const int sb = wsl * 32;  // this wave's 32 slots inside the chunk

    // S^T = K Q^T for two 16-slot tiles
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = sb + 16 * t + c16;
        const int cc = 4 * ks + g4;
        const u32x4 a = *(const u32x4*)(kb + r * C::KB + swz<C::KB>(r, cc) * 16);
        s[t] = T::mfma(as<vec8>(a), as<vec8>(qreg[ks]), s[t]);
      }
    }

    // mask, scale (log2 units), chunk max
    float x[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int4 jj = *(const int4*)(idxl + c * C::CH + sb + 16 * t + 4 * g4);
      const int jv[4] = {jj.x, jj.y, jj.z, jj.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = jv[e] >= 0 ? s[t][e] * p.scale_log2 : -INFINITY;
        x[4 * t + e] = xv;
        cmax = fmaxf(cmax, xv);
      }
    }
    cmax = wave_max_across_groups(cmax);
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while nothing has been seen
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = fast_exp2(x[i] - m_use);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] *= alpha;

    u32x4 phi, plo;
    split_hi_lo<T>(pv, phi, plo);

    // O^T += V^T P^T.  MFMA k index 8*g4 + e maps to slot 16*(e/4) + 4*g4 + e%4,
    // matching where the S tiles left P.
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      u32x2 lo_half, hi_half;
      {
        const int r = sb + 4 * g4 + (c16 >> 2);
        const int cc = 2 * dt + ((c16 & 3) >> 1);
        lo_half = lds_read_tr16(vb + r * C::VB + swz<C::VB>(r, cc) * 16 + (c16 & 1) * 8);
      }
      {
        const int r = sb + 16 + 4 * g4 + (c16 >> 2);
        const int cc = 2 * dt + ((c16 & 3) >> 1);
        hi_half = lds_read_tr16(vb + r * C::VB + swz<C::VB>(r, cc) * 16 + (c16 & 1) * 8);
      }
      const u32x4 a = {lo_half[0], lo_half[1], hi_half[0], hi_half[1]};
      acc[dt] = T::mfma(as<vec8>(a), as<vec8>(phi), acc[dt]);
      acc[dt] = T::mfma(as<vec8>(a), as<vec8>(plo), acc[dt]);
    }

    if (c + 1 < nchunks) write_staged((c & 1) ? kbuf0 : kbuf1, (c & 1) ? vbuf0 : vbuf1);
    __syncthreads();
    if (c + 2 < nchunks) issue_gather(c + 2);
  }

  // ---- epilogue
  const float l_tot = wave_sum_across_groups(l_run);
  const int64_t row = ((int64_t)b * p.S1 + s1) * p.N1 + n1;  // flat (b, s1, n1)

  if constexpr (WS == 1) {
    if (p.nsplit == 1) {
      if (head_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = p.out + (int64_t)b * p.os[0] + (int64_t)s1 * p.os[1] + (int64_t)n1 * p.os[2];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          u32x2 w;
          w[0] = (uint32_t)T::from_float(acc[dt][0] * inv) | ((uint32_t)T::from_float(acc[dt][1] * inv) << 16);
          w[1] = (uint32_t)T::from_float(acc[dt][2] * inv) | ((uint32_t)T::from_float(acc[dt][3] * inv) << 16);
          *(u32x2*)(orow + dt * 16 + 4 * g4) = w;
        }
        if (p.lse && g4 == 0)
          p.lse[(int64_t)b * p.ls[0] + (int64_t)s1 * p.ls[1] + (int64_t)n1 * p.ls[2]] =
              l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      }
    } else {
      if (head_ok) {
        float* po = p.ws_o + (row * p.nsplit + split) * DV;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) *(f32x4*)(po + dt * 16 + 4 * g4) = acc[dt];
        if (g4 == 0) {
          float* pm = p.ws_ml + (row * p.nsplit + split) * 2;
          pm[0] = m_run;
          pm[1] = l_tot;
        }
      }
    }
  } else {
    // merge the WS slot parts of each head tile through LDS
    float* mo = (float*)smem;                       // [WS][WH][16][DV]
    float* mml = mo + WS * WH * 16 * DV;            // [WS][WH][16][2]
    // every wave finished its last chunk (loop ends with a barrier)
    {
      float* o = mo + ((wsl * WH + wh) * 16 + c16) * DV;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) *(f32x4*)(o + dt * 16 + 4 * g4) = acc[dt];
      if (g4 == 0) {
        float* ml = mml + ((wsl * WH + wh) * 16 + c16) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    __syncthreads();
    // thread -> (head tile, head, 4 dv values)
    constexpr int PER_ROW = DV / 4;
    for (int w = tid; w < WH * 16 * PER_ROW; w += C::NT) {
      const int hrow = w / PER_ROW;  // wh*16 + head column
      const int d4 = w % PER_ROW;
      const int hh = hb * 16 * WH + hrow;
      if (hh >= p.G) continue;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < WS; ++q) M = fmaxf(M, mml[(q * WH * 16 + hrow) * 2]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float L = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < WS; ++q) {
        const float wq = fast_exp2(mml[(q * WH * 16 + hrow) * 2] - Mu);
        L += mml[(q * WH * 16 + hrow) * 2 + 1] * wq;
        o += *(const f32x4*)(mo + (q * WH * 16 + hrow) * DV + 4 * d4) * wq;
      }
      const int nn1 = n2 * p.G + hh;
      const int64_t rr = ((int64_t)b * p.S1 + s1) * p.N1 + nn1;
      if (p.nsplit == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t* orow = p.out + (int64_t)b * p.os[0] + (int64_t)s1 * p.os[1] + (int64_t)nn1 * p.os[2];
        u32x2 wv;
        wv[0] = (uint32_t)T::from_float(o[0] * inv) | ((uint32_t)T::from_float(o[1] * inv) << 16);
        wv[1] = (uint32_t)T::from_float(o[2] * inv) | ((uint32_t)T::from_float(o[3] * inv) << 16);
        *(u32x2*)(orow + 4 * d4) = wv;
        if (p.lse && d4 == 0)
          p.lse[(int64_t)b * p.ls[0] + (int64_t)s1 * p.ls[1] + (int64_t)nn1 * p.ls[2]] =
              L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
      } else {
        *(f32x4*)(p.ws_o + (rr * p.nsplit + split) * DV + 4 * d4) = o;
        if (d4 == 0) {
          float* pm = p.ws_ml + (rr * p.nsplit + split) * 2;
          pm[0] = M;
          pm[1] = L;
        }
      }
    }
  }
}

// Combines the nsplit partials of every row: M = max m_j, L = sum l_j 2^(m_j - M),
// y = sum O_j 2^(m_j - M) / L, lse = (M + log2 L) ln 2; a row with L == 0 gets y = 0,
// lse = -inf.  One thread per 4 output values.
template <typename T, int DV>
__global__ __launch_bounds__(256) void topk_merge(TopkParams p, int64_t nrows) {
  constexpr int PER_ROW = DV / 4;
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = w / PER_ROW;
  const int d4 = (int)(w % PER_ROW);
  if (row >= nrows) return;
  const float* ml = p.ws_ml + row * p.nsplit * 2;
  float M = -INFINITY;
  for (int j = 0; j < p.nsplit; ++j) M = fmaxf(M, ml[2 * j]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  const float* po = p.ws_o + row * p.nsplit * DV + 4 * d4;
  for (int j = 0; j < p.nsplit; ++j) {
    const float wj = fast_exp2(ml[2 * j] - Mu);
    L += ml[2 * j + 1] * wj;
    o += *(const f32x4*)(po + (int64_t)j * DV) * wj;
  }
  const int n1 = (int)(row % p.N1);
  const int s1 = (int)((row / p.N1) % p.S1);
  const int b = (int)(row / ((int64_t)p.N1 * p.S1));
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = p.out + (int64_t)b * p.os[0] + (int64_t)s1 * p.os[1] + (int64_t)n1 * p.os[2];
  u32x2 wv;
  wv[0] = (uint32_t)T::from_float(o[0] * inv) | ((uint32_t)T::from_float(o[1] * inv) << 16);
  wv[1] = (uint32_t)T::from_float(o[2] * inv) | ((uint32_t)T::from_float(o[3] * inv) << 16);
  *(u32x2*)(orow + 4 * d4) = wv;
  if (p.lse && d4 == 0)
    p.lse[(int64_t)b * p.ls[0] + (int64_t)s1 * p.ls[1] + (int64_t)n1 * p.ls[2]] =
        L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace sfa
