// Top-K kernel for many query vectors per index list with wide value heads (the MLA
// decode shape of the SparseFlashAttention operator page: 128 heads on one latent KV
// head, Dk = 576, Dv = 512, value = key[..., :512]).
//
// A workgroup has 8 waves (two per SIMD) and 64 query vectors ("heads") of one work item;
// the gathered rows are staged in chunks of 32 slots as in topk_fwd.  Per chunk:
//  * S^T = K_sel Q^T is split over (head tile of 16, slot half of 16): wave w computes the
//    16 x 16 scores of head tile w % 4 over slots 16 (w / 4) .. +15, Q^T in VGPRs.
//  * Softmax: each head's two slot halves live in two waves.  Both keep the same running
//    reference max; while neither half exceeds it by more than kLazyRescale (the common
//    case after the first chunk) each wave turns its scores into P on its own.  When one
//    must move it, the half-chunk maxima go through LDS, both waves take the same new max
//    and P is recomputed (one extra barrier).  P goes to LDS as hi/lo 16-bit parts.
//  * O^T = V_sel^T P^T is split over dv: wave w accumulates dv columns [w Dv/8, (w+1) Dv/8)
//    for all 64 heads, with P^T read from LDS.
// Against splitting only the heads (topk_fwd), a staged V row is read from LDS once per
// workgroup instead of once per head tile, the softmax work per wave is a quarter, and the
// O accumulators (Dv x 64 fp32) are spread over 8 waves, leaving room for two waves per
// SIMD so one wave's LDS reads and softmax overlap the other's MFMAs.
#pragma once

#include "topk_kernel.hpp"

namespace sfa {

constexpr int kDvsHeads = 64;  // query vectors per workgroup
constexpr int kDvsWaves = 8;
constexpr int kDvsPRow = 40;   // P row stride in 16-bit elements: 32 slots + pad (80 B, conflict-free reads)

// LDS bytes besides the ring and the index slots: P hi + lo, half maxima / half sums
// [2][64], alpha / final max [64], mask flags and bump flags [kMaxSplitLen / 32] each.
constexpr int dvs_misc_bytes() {
  return 2 * kDvsHeads * kDvsPRow * 2 + 2 * kDvsHeads * 4 + kDvsHeads * 4 + 2 * kFlagBytes;
}

// Ring depth: the deepest ring (at most 4) that leaves kIdxReserve bytes for index slots.
constexpr int dvs_nbuf(int DK, int DV, bool alias) {
  const int buf = topk_chunk_bytes(DK, DV, alias, 1);
  for (int n = 4; n >= 2; --n)
    if (n * buf + dvs_misc_bytes() + kIdxReserve <= 160 * 1024) return n;
  return 0;
}

// Shapes this kernel is built for: Dv a multiple of 256 (an even number of 16-wide dv tiles
// per wave) and a ring of at least two chunks.
constexpr bool dvs_supported(int DK, int DV, bool alias) {
  return DV % 256 == 0 && DK % 64 == 0 && DV <= DK && dvs_nbuf(DK, DV, alias) >= 2;
}

inline int dvs_max_split_len(int DK, int DV, bool alias) {
  const int nbuf = dvs_nbuf(DK, DV, alias);
  if (nbuf < 2) return 0;
  int len = (160 * 1024 - nbuf * topk_chunk_bytes(DK, DV, alias, 1) - dvs_misc_bytes()) / 4;
  len = len / 32 * 32;
  return len < kMaxSplitLen ? len : kMaxSplitLen;
}

template <typename T, int DK, int DV, bool ALIAS, int NBUF>
struct DvsCfg {
  static constexpr int NT = 64 * kDvsWaves;
  static constexpr int CH = 32;
  static constexpr int KCPR = DK / 8;
  static constexpr int VCPR = DV / 8;
  static constexpr int KS = staged_stride(KCPR);
  static constexpr int VS = ALIAS ? KS : staged_stride(VCPR);
  static constexpr int KPOS = CH * KS;
  static constexpr int VPOS = ALIAS ? 0 : CH * VS;
  static constexpr int KLD = (KPOS + NT - 1) / NT;
  static constexpr int VLD = (VPOS + NT - 1) / NT;
  static constexpr int rounds_all(int pos, int ld) {
    int n = 0;
    for (int u = 0; u < ld; ++u) n += (u * NT + 64 * (kDvsWaves - 1) < pos) ? 1 : 0;
    return n;
  }
  static constexpr int CNT = rounds_all(KPOS, KLD) + rounds_all(VPOS, VLD);
  // the 64 query rows, piece-major, in ring buffers 1.. before the loop starts
  static constexpr int QPOS = kDvsHeads * KCPR;
  static constexpr int QLD = QPOS / NT;  // every wave issues every round
  static constexpr int QCNT = QLD;
  static constexpr bool QSTAGE = QPOS * 16 <= (NBUF - 1) * (KPOS + VPOS) * 16;
  static_assert(QPOS % NT == 0, "whole query copy rounds");
  static constexpr int KSTEPS = DK / 32;       // 16x16x32 k-steps of one score tile
  static constexpr int DTW = DV / kDvsWaves / 16;  // 16-wide dv tiles per wave
  static constexpr int KBUF = KPOS * 16;
  static constexpr int VBUF = VPOS * 16;
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int P_BYTES = kDvsHeads * kDvsPRow * 2;
  static constexpr int OFF_P = NBUF * BUF;                     // P hi [64][kDvsPRow], then P lo
  static constexpr int OFF_HM = OFF_P + 2 * P_BYTES;           // [2][64] f32
  static constexpr int OFF_AL = OFF_HM + 2 * kDvsHeads * 4;    // [64] f32
  static constexpr int OFF_CF = OFF_AL + kDvsHeads * 4;        // mask flags [64] i32
  static constexpr int OFF_BF = OFF_CF + kFlagBytes;           // bump flags [64] i32
  static constexpr int LDS_FIXED = OFF_BF + kFlagBytes;        // index slots follow
  static_assert(BUF == topk_chunk_bytes(DK, DV, ALIAS, 1), "layout");
  static_assert(LDS_FIXED == NBUF * BUF + dvs_misc_bytes(), "layout");
  static_assert(DV % 256 == 0 && DK % 64 == 0 && DV <= DK, "head dims");
  static_assert(KPOS % 128 == 0 && VPOS % 128 == 0, "whole-wave rounds");
  static_assert(LDS_FIXED + kIdxReserve <= 160 * 1024, "LDS budget");
  static_assert(NBUF >= 2 && (NBUF - 2) * CNT < 64, "vmcnt range");
};

// LDS writes of this wave done, then the workgroup barrier (no wait on the gathers in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int DK, int DV, bool ALIAS, int NBUF>
__global__ __launch_bounds__(512) void topk_fwd_dvs(TopkParams p) {
  using C = DvsCfg<T, DK, DV, ALIAS, NBUF>;
  using vec8 = typename T::vec8;
  extern __shared__ __align__(16) char smem[];
  char* p_hi = smem + C::OFF_P;
  char* p_lo = smem + C::OFF_P + C::P_BYTES;
  float* hmax = (float*)(smem + C::OFF_HM);
  float* alph = (float*)(smem + C::OFF_AL);
  int* cflag = (int*)(smem + C::OFF_CF);
  int* bflag = (int*)(smem + C::OFF_BF);
  int* idxl = (int*)(smem + C::LDS_FIXED);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qt = wave & 3;   // score role: head tile
  const int sh = wave >> 2;  // score role: slot half
  const int kg = lane >> 4;  // k-group of this lane in MFMA operands
  const int col = lane & 15;

  // ---- work item (same decomposition as topk_fwd; head blocks of 64)
  int item = xcd_remap(blockIdx.x, p.n_items);
  const int hb = item % p.HB;
  item /= p.HB;
  const int split = item % p.nsplit;
  item /= p.nsplit;
  const int s1 = item % p.S1;
  item /= p.S1;
  const int n2 = item % p.N2;
  const int b = item / p.N2;

  const int32_t* ig;
  int nslots_all;
  if (p.slot_ptr) {
    const int s0 = p.slot_ptr[s1];
    ig = p.idx + s0;
    nslots_all = p.slot_ptr[s1 + 1] - s0;
  } else {
    ig = p.idx + (int64_t)b * p.is[0] + (int64_t)s1 * p.is[1] + (int64_t)n2 * p.is[2];
    nslots_all = p.topK;
  }
  const int slot0 = split * p.split_len;
  const int nslots = max(0, min(p.split_len, nslots_all - slot0));
  const int nchunks = (nslots + C::CH - 1) / C::CH;

  const int h0 = hb * kDvsHeads;
  // score role: virtual head h0 + 16 qt + col
  const int head = h0 + 16 * qt + col;
  const int qrow_idx = s1 * p.RS + head / p.HR;
  const bool head_ok = head < p.G && qrow_idx < p.QROWS;
  const int hv = head_ok ? head : 0;

  const uint16_t* kg_ptr = uniform_ptr(p.k + (int64_t)b * p.ks[0] + (int64_t)n2 * p.ks[2]);
  const uint16_t* vg_ptr = uniform_ptr(p.v + (int64_t)b * p.vs[0] + (int64_t)n2 * p.vs[2]);
  const uint32_t krow_bytes = (uint32_t)p.ks[1] * 2u, vrow_bytes = (uint32_t)p.vs[1] * 2u;

  const uint32_t smem_lds = lds_addr_of(smem);
  const uint32_t jrows = (uint32_t)p.S2;
  const uint32_t jend = (uint32_t)(p.causal ? max(0, min(p.S2, qrow_idx + (p.S2 - p.QROWS) + 1)) : p.S2);
  auto clamp_row = [&](int j) -> int { return min(max(j, 0), (int)jrows - 1); };
  auto selects = [&](int j) -> bool { return (uint32_t)j < jend; };

  // ---- gather rounds (see topk_fwd): thread tid loads position u * NT + tid of a chunk
  auto pack_pos = [&](int pos, int stride, int cpr) -> int {
    const int r = pos / stride, x = pos % stride;
    const int cc = x < cpr ? ((x & ~3) | ((x & 3) ^ stage_xor(r))) : (x & 3);
    return r | (cc << 8);
  };
  auto round_in = [&](int u, int npos) -> bool {
    if (u * C::NT + C::NT <= npos) return true;
    return u * C::NT + wave_u * 64 < npos;
  };

  // ---- prologue.  The split's raw row indices and (when the ring buffers after the first can
  // hold them) the workgroup's 64 query rows are copied to LDS together; chunk 0 of the gather
  // is issued as soon as the indices have landed, and the query rows are read into registers
  // while it is in flight.  Query rows are staged piece-major: 16-byte piece cc of row r at
  // position 64 cc + r, so lane i of a copy round always loads row i (its row offset is
  // computed once) and the Q^T operand reads (16 rows, one piece) are conflict-free.
  u32x4 qreg[C::KSTEPS];  // k-step ks: q[head][32 ks + 8 kg .. + 7]
  {
    for (int i0 = wave_u * 64; i0 < nslots; i0 += C::NT)
      if (i0 + lane < nslots) lds_dma4(ig + slot0 + i0 + lane, smem_lds + C::LDS_FIXED + i0 * 4);
  }
  if constexpr (C::QSTAGE) {
    const int h = h0 + lane;
    const bool ok = h < p.G && s1 * p.RS + h / p.HR < p.QROWS;  // else any valid row: head 0
    const uint16_t* qrow = p.q + qv_offset(p, p.qs, b, s1, n2, ok ? h : 0);
#pragma unroll
    for (int u = 0; u < C::QLD; ++u) {
      const int cc = u * kDvsWaves + wave_u;  // piece of this round (wave-uniform)
      lds_dma16(qrow + cc * 8, smem_lds + C::BUF + (u * C::NT + wave_u * 64) * 16);
    }
  } else {
    const uint16_t* qrow = p.q + qv_offset(p, p.qs, b, s1, n2, hv);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qreg[ks] = *(const u32x4*)(qrow + 32 * ks + 8 * kg);
  }
  for (int i = nslots + tid; i < nchunks * C::CH; i += C::NT) idxl[i] = -1;
  for (int i = tid; i < 2 * kFlagBytes / 4; i += C::NT) cflag[i] = 0;  // mask and bump flags
  if constexpr (C::QSTAGE) wait_vm_barrier<C::QCNT>();  // indices landed (query rows may not have)
  else {
    wait_vm_all();
    __syncthreads();
  }
  {
    const uint32_t jend_lo =
        (uint32_t)(p.causal ? max(0, min(p.S2, s1 * p.RS + h0 / p.HR + (p.S2 - p.QROWS) + 1)) : p.S2);
    for (int i = tid; i < nslots; i += C::NT)
      if (!((uint32_t)idxl[i] < jend_lo)) cflag[i / C::CH] = 1;
    if (tid == 0 && nslots % C::CH != 0) cflag[nslots / C::CH] = 1;
  }

  int kpk[C::KLD];
#pragma unroll
  for (int u = 0; u < C::KLD; ++u) {
    const int pos = u * C::NT + tid;
    kpk[u] = pos < C::KPOS ? pack_pos(pos, C::KS, C::KCPR) : 0;
  }
  int vpk[C::VLD > 0 ? C::VLD : 1];
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int pos = u * C::NT + tid;
    vpk[u] = pos < C::VPOS ? pack_pos(pos, C::VS, C::VCPR) : 0;
  }
  // Gather of chunk c in NR rounds (K rounds, then V rounds): read_rows fetches the row
  // indices of all rounds (one batch of LDS reads), issue_round issues one load.
  constexpr int NR = C::KLD + (ALIAS ? 0 : C::VLD);
  int jrow[NR];
  auto read_rows = [&](int c) {
    const int* irow = idxl + c * C::CH;
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) jrow[u] = irow[kpk[u] & 255];
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < C::VLD; ++u) jrow[C::KLD + u] = irow[vpk[u] & 255];
    }
  };
  auto issue_round = [&](int c, int r) {
    const uint32_t kb_lds = smem_lds + (c % NBUF) * C::BUF;
    if (r < C::KLD) {
      if (round_in(r, C::KPOS))
        lds_dma16_at(kg_ptr, __umul24((uint32_t)clamp_row(jrow[r]), krow_bytes) + ((uint32_t)kpk[r] >> 8) * 16u,
                     kb_lds + (r * C::NT + wave_u * 64) * 16);
    } else if constexpr (!ALIAS) {
      const int u = r - C::KLD;
      if (round_in(u, C::VPOS))
        lds_dma16_at(vg_ptr, __umul24((uint32_t)clamp_row(jrow[r]), vrow_bytes) + ((uint32_t)vpk[u] >> 8) * 16u,
                     kb_lds + C::KBUF + (u * C::NT + wave_u * 64) * 16);
    }
  };
  auto issue_gather = [&](int c) {
    read_rows(c);
#pragma unroll
    for (int r = 0; r < NR; ++r) issue_round(c, r);
  };

  if (nchunks > 0) issue_gather(0);
  if constexpr (C::QSTAGE) {
    // the query rows were issued before chunk 0: at most chunk 0's loads may be outstanding
    if (nchunks > 0) wait_vm_barrier<C::CNT>();
    else wait_vm_barrier<0>();
    const char* qb = smem + C::BUF + (kg * kDvsHeads + 16 * qt + col) * 16;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qreg[ks] = *(const u32x4*)(qb + ks * 4 * kDvsHeads * 16);
    lds_barrier();  // every wave has its Q^T before ring buffers 1.. are reused
  }
#pragma unroll
  for (int i = 1; i < NBUF - 1; ++i)
    if (i < nchunks) issue_gather(i);

  // ---- per-lane LDS byte offsets of the operands
  //  K (score A operand), k-step ks: row 16 sh + col, 16-byte chunk 4 ks + kg
  const int rk = 16 * sh + col;
  const int lane_k = (rk * C::KS + (kg ^ stage_xor(rk))) * 16;
  //  V^T (PV A operand), dv tile dt of this wave (global 16-wide tile g = wave * DTW + dt), half
  //  hh: lane c16 of k-group kg reads row 8 kg + 4 hh + c16 / 4 at dv 16 g + 4 (c16 % 4), so it
  //  receives dv 16 g + c16 of slots 8 kg + 4 hh .. + 3 (MFMA k index = slot)
  const int c16 = lane & 15;
  int lane_v[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * kg + 4 * hh + (c16 >> 2);
#pragma unroll
    for (int par = 0; par < 2; ++par)
      lane_v[hh][par] = (r * C::VS + ((2 * par + ((c16 & 3) >> 1)) ^ stage_xor(r))) * 16 + 8 * (c16 & 1);
  }
  const int vwave = wave_u * C::DTW * 2 * 16;  // byte offset of this wave's first dv chunk (2 chunks per tile)
  auto v_off = [&](int dt, int hh) -> int { return lane_v[hh][dt & 1] + vwave + 64 * (dt >> 1); };
  //  P^T (PV B operand), head tile ht: P[16 ht + col][8 kg .. + 7]
  const int lane_p = (col * kDvsPRow + 8 * kg) * 2;
  //  P writes (score role): P[16 qt + col][16 sh + 4 kg .. + 3]
  const int lane_pw = ((16 * qt + col) * kDvsPRow + 16 * sh + 4 * kg) * 2;

  f32x4 acc[C::DTW][4];  // O^T: dv 16 (wave DTW + dt) + 4 kg + e, head 16 ht + col
#pragma unroll
  for (int dt = 0; dt < C::DTW; ++dt)
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max of this lane's head (log2 units), same in both halves
  float l_run = 0.f;        // this lane's share of the half sum

  auto wait_chunk = [&](int ahead) {
    switch (ahead) {
#define SFA_WAIT_CASE(k) \
  case k:                \
    if constexpr (k <= NBUF - 2) wait_vm_barrier<k * C::CNT>(); \
    break;
      SFA_WAIT_CASE(0)
      SFA_WAIT_CASE(1)
      SFA_WAIT_CASE(2)
#undef SFA_WAIT_CASE
      default:
        wait_vm_barrier<0>();
    }
  };

  for (int c = 0; c < nchunks; ++c) {
    // chunk c has landed and every wave is done with chunk c - 1 (its ring buffer and P)
    wait_chunk(min(NBUF - 2, nchunks - 1 - c));
    // chunk c + NBUF - 1 goes into the buffer of chunk c - 1 (free: every wave passed the
    // barrier above); its loads are issued between the PV MFMAs below
    const int gc = c + NBUF - 1 < nchunks ? c + NBUF - 1 : -1;
    if (gc >= 0) read_rows(gc);
    const char* kb = smem + (c % NBUF) * C::BUF;
    const char* vb = ALIAS ? kb : kb + C::KBUF;

    // scores of 16 slots x 16 heads, two accumulation chains
    f32x4 s;
    {
      f32x4 s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      constexpr int KG = 6;
#pragma unroll
      for (int k0 = 0; k0 < C::KSTEPS; k0 += KG) {
        u32x4 a[KG];
#pragma unroll
        for (int g = 0; g < KG; ++g)
          if (k0 + g < C::KSTEPS) a[g] = *(const u32x4*)(kb + lane_k + 64 * (k0 + g));
#pragma unroll
        for (int g = 0; g < KG; ++g)
          if (k0 + g < C::KSTEPS)
            s2[(k0 + g) & 1] = T::mfma(as<vec8>(a[g]), as<vec8>(qreg[k0 + g < C::KSTEPS ? k0 + g : 0]),
                                       s2[(k0 + g) & 1]);
      }
      s = s2[0] + s2[1];
    }

    // mask; half-chunk max (element e: slot 16 sh + 4 kg + e)
    float x[4];
    if (__builtin_amdgcn_readfirstlane(cflag[c])) {
      const u32x4 jj = *(const u32x4*)(idxl + c * C::CH + 16 * sh + 4 * kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = selects((int)jj[e]) ? s[e] : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = s[e];
    }
    // Only a wave where some lane exceeds the reference by more than kLazyRescale reduces its
    // half maxima across lanes; the others publish -inf (nothing to move).
    const float mx4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])) * p.scale_log2;
    float hm_pub = -INFINITY;
    if (__builtin_amdgcn_ballot_w64(mx4 > m_run + kLazyRescale)) {
      const float hm = wave_max_lanes<16>(mx4);
      const bool need = hm > m_run + kLazyRescale;
      hm_pub = need ? hm : -INFINITY;
      if (need) bflag[c] = 1;
    }
    if (kg == 0) hmax[sh * kDvsHeads + 16 * qt + col] = hm_pub;
    // P against the current reference (rewritten below if some head moves it)
    auto make_p = [&](float m_use, float& psum) {
      float pr[4];
      psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr[e] = fast_exp2(__builtin_fmaf(x[e], p.scale_log2, -m_use));
        psum += pr[e];
      }
      u32x2 hi, lo;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint16_t h0v = T::from_float(pr[2 * i]), h1v = T::from_float(pr[2 * i + 1]);
        hi[i] = (uint32_t)h0v | ((uint32_t)h1v << 16);
        lo[i] = (uint32_t)T::from_float(pr[2 * i] - T::to_float(h0v)) |
                ((uint32_t)T::from_float(pr[2 * i + 1] - T::to_float(h1v)) << 16);
      }
      *(u32x2*)(p_hi + lane_pw) = hi;
      *(u32x2*)(p_lo + lane_pw) = lo;
    };
    float psum;
    make_p(m_run == -INFINITY ? 0.f : m_run, psum);
    lds_barrier();  // P, half maxima and bump flag visible

    if (__builtin_amdgcn_readfirstlane(bflag[c])) {
      // some head moves its reference: both halves take max(needing half maxima)
      const float hx = fmaxf(hmax[16 * qt + col], hmax[kDvsHeads + 16 * qt + col]);
      float alpha = 1.f;
      if (hx > m_run + kLazyRescale) {
        alpha = fast_exp2(m_run - hx);  // 0 when nothing was seen yet
        m_run = hx;
        l_run *= alpha;
      }
      make_p(m_run == -INFINITY ? 0.f : m_run, psum);
      if (sh == 0 && kg == 0) alph[16 * qt + col] = alpha;
      lds_barrier();
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float a = alph[16 * ht + col];
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt) acc[dt][ht] *= a;  // accumulators stay in VGPRs
      }
    }
    l_run += psum;

    // O^T += V^T (P_hi + P_lo)^T over the 32 slots of the chunk
    u32x4 bh[4], bl[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      bh[ht] = *(const u32x4*)(p_hi + lane_p + ht * 16 * kDvsPRow * 2);
      bl[ht] = *(const u32x4*)(p_lo + lane_p + ht * 16 * kDvsPRow * 2);
    }
#pragma unroll
    for (int dt = 0; dt < C::DTW; ++dt) {
      if (gc >= 0) {
#pragma unroll
        for (int r = dt * NR / C::DTW; r < (dt + 1) * NR / C::DTW; ++r) issue_round(gc, r);
      }
      const u32x2 v0 = lds_read_tr16(vb + v_off(dt, 0));
      const u32x2 v1 = lds_read_tr16(vb + v_off(dt, 1));
      const u32x4 a = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = T::mfma(as<vec8>(a), as<vec8>(bh[ht]), acc[dt][ht]);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = T::mfma(as<vec8>(a), as<vec8>(bl[ht]), acc[dt][ht]);
    }
  }
  __syncthreads();  // every wave is done with the last chunk's P

  // ---- epilogue: head totals through LDS (half sums [2][64], reference max [64])
  {
    const float l_half = wave_sum_lanes<16>(l_run);
    if (kg == 0) {
      hmax[sh * kDvsHeads + 16 * qt + col] = l_half;
      if (sh == 0) alph[16 * qt + col] = m_run;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int hh = h0 + 16 * ht + col;
    if (hh >= p.G || s1 * p.RS + hh / p.HR >= p.QROWS) continue;
    const float L = hmax[16 * ht + col] + hmax[kDvsHeads + 16 * ht + col];
    const float M = alph[16 * ht + col];
    const int dv0 = wave * C::DTW * 16 + 4 * kg;
    if (p.nsplit == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      uint16_t* orow = p.out + qv_offset(p, p.os, b, s1, n2, hh);
#pragma unroll
      for (int dt = 0; dt < C::DTW; ++dt) {
        u32x2 w;
        w[0] = (uint32_t)T::from_float(acc[dt][ht][0] * inv) | ((uint32_t)T::from_float(acc[dt][ht][1] * inv) << 16);
        w[1] = (uint32_t)T::from_float(acc[dt][ht][2] * inv) | ((uint32_t)T::from_float(acc[dt][ht][3] * inv) << 16);
        *(u32x2*)(orow + dv0 + 16 * dt) = w;
      }
      if (p.lse && wave == 0 && kg == 0)
        p.lse[qv_offset(p, p.ls, b, s1, n2, hh)] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
    } else {
      const int64_t row = ws_row(p, b, s1, n2, hh);
      float* po = p.ws_o + (row * p.nsplit + split) * DV + dv0;
#pragma unroll
      for (int dt = 0; dt < C::DTW; ++dt) *(f32x4*)(po + 16 * dt) = acc[dt][ht];
      if (wave == 0 && kg == 0) {
        float* pm = p.ws_ml + (row * p.nsplit + split) * 2;
        pm[0] = M;
        pm[1] = L;
      }
    }
  }
}

}  // namespace sfa
