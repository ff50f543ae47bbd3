// Top-K kernel for many query vectors per index list with wide value heads (the MLA
// decode shape of the SparseFlashAttention operator page: 128 heads on one latent KV
// head, Dk = 576, Dv = 512, value = key[..., :512]).
//
// A workgroup has 8 waves and 64 query vectors ("heads") of one work item; the gathered rows
// are staged in chunks of 32 slots as in topk_fwd.  The waves take two roles, one wave of
// each on every SIMD, and work on consecutive chunks at once:
//  * score waves (0..3): wave w computes S^T = K_sel Q^T for 32 heads (h0 + 32 (w % 2) ..)
//    over 16 slots (16 (w / 2) ..) of chunk c -- one K operand read feeds two MFMAs, Q^T in
//    VGPRs -- then the online softmax of those heads over its slots, and writes P (hi/lo
//    16-bit parts) and the reference max it used to LDS;
//  * value waves (4..7): wave 4 + w issues the gather of chunk c + NBUF - 2 and accumulates
//    O^T = V_sel^T P^T of chunk c - 1 for dv columns [w Dv/4, (w+1) Dv/4) of all 64 heads,
//    P^T read from LDS.
// One barrier per step separates the chunks; P and the references are double-buffered.
// Each head's 32 slots are scored by two waves that share a reference max.  A half whose
// scores exceed it by more than kLazyRescale uses its own new maximum for that chunk; the
// value waves then bring both halves' P and the accumulators to the larger reference (in
// registers, only for head tiles flagged in that chunk) and the two score waves adopt it at
// the next step.
// Against splitting only the heads (topk_fwd), a staged V row is read from LDS once per
// workgroup instead of once per head tile, and the O accumulators (Dv x 64 fp32) live in the
// value waves only, which leaves room for two waves per SIMD: a score wave's LDS reads and
// exponentials overlap the value wave's MFMAs.
#pragma once

#include "topk_kernel.hpp"

namespace sfa {

constexpr int kDvsHeads = 64;  // query vectors per workgroup
constexpr int kDvsWaves = 8;   // 4 score waves, then 4 value waves
constexpr int kDvsPRow = 40;   // P row stride in 16-bit elements: 32 slots + pad (80 B, conflict-free reads)
constexpr int kDvsPBytes = kDvsHeads * kDvsPRow * 2;

// LDS bytes besides the ring and the index slots: P hi + lo, double-buffered; references
// [2][2 halves][64]; mask flags [kMaxSplitLen / 32]; moved-reference flags [kMaxSplitLen / 32][4].
constexpr int dvs_misc_bytes() { return 4 * kDvsPBytes + 4 * kDvsHeads * 4 + kFlagBytes + 4 * kFlagBytes; }

// Ring depth: the deepest ring (at most 4) that leaves kIdxReserve bytes for index slots.
constexpr int dvs_nbuf(int DK, int DV, bool alias) {
  const int buf = topk_chunk_bytes(DK, DV, alias, 1, kDvsHeads);
  for (int n = 4; n >= 2; --n)
    if (n * buf + dvs_misc_bytes() + kIdxReserve <= 160 * 1024) return n;
  return 0;
}

// Shapes this kernel is built for: Dv a multiple of 256 (an even number of 16-wide dv tiles
// per value wave) and a ring of at least three chunks (one being scored, one in the PV
// product, one or more landing).
constexpr bool dvs_supported(int DK, int DV, bool alias) {
  return DV % 256 == 0 && DK % 64 == 0 && DV <= DK && dvs_nbuf(DK, DV, alias) >= 3;
}

inline int dvs_max_split_len(int DK, int DV, bool alias) {
  const int nbuf = dvs_nbuf(DK, DV, alias);
  if (nbuf < 3) return 0;
  int len = (160 * 1024 - nbuf * topk_chunk_bytes(DK, DV, alias, 1, kDvsHeads) - dvs_misc_bytes()) / 4;
  len = len / 32 * 32;
  return len < kMaxSplitLen ? len : kMaxSplitLen;
}

template <typename T, int DK, int DV, bool ALIAS, int NBUF>
struct DvsCfg {
  static constexpr int NT = 64 * kDvsWaves;
  static constexpr int NG = NT / 2;  // threads of the value waves (they issue the gathers)
  static constexpr int CH = 32;
  static constexpr int KCPR = DK / 8;
  static constexpr int VCPR = DV / 8;
  static constexpr int KS = staged_stride(KCPR);
  static constexpr int VS = ALIAS ? KS : staged_stride(VCPR);
  static constexpr int KPOS = CH * KS;
  static constexpr int VPOS = ALIAS ? 0 : CH * VS;
  static constexpr int KLD = (KPOS + NG - 1) / NG;  // gather rounds per value thread
  static constexpr int VLD = (VPOS + NG - 1) / NG;
  static constexpr int rounds_all(int pos, int ld) {
    int n = 0;
    for (int u = 0; u < ld; ++u) n += (u * NG + 64 * (kDvsWaves / 2 - 1) < pos) ? 1 : 0;
    return n;
  }
  static constexpr int CNT = rounds_all(KPOS, KLD) + rounds_all(VPOS, VLD);
  // the 64 query rows, piece-major, in ring buffers 1.. before the loop starts (the 4 score
  // waves copy them)
  static constexpr int QPOS = kDvsHeads * KCPR;
  static constexpr int QLD = QPOS / (NT / 2);
  static_assert(QPOS % (NT / 2) == 0, "whole query copy rounds");
  static_assert(QPOS * 16 <= (NBUF - 1) * (KPOS + VPOS) * 16, "query rows fit the idle buffers");
  static constexpr int KSTEPS = DK / 32;           // 16x16x32 k-steps of one score tile
  static constexpr int DTW = DV / (kDvsWaves / 2) / 16;  // 16-wide dv tiles per value wave
  static constexpr int KBUF = KPOS * 16;
  static constexpr int VBUF = VPOS * 16;
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int OFF_P = NBUF * BUF;                      // [2][hi, lo][64][kDvsPRow]
  static constexpr int OFF_RF = OFF_P + 4 * kDvsPBytes;         // references [2][2][64] f32
  static constexpr int OFF_CF = OFF_RF + 4 * kDvsHeads * 4;     // mask flags [64] i32
  static constexpr int OFF_BF = OFF_CF + kFlagBytes;            // moved-reference flags [64][4] i32
  static constexpr int LDS_FIXED = OFF_BF + 4 * kFlagBytes;     // index slots follow
  static_assert(BUF == topk_chunk_bytes(DK, DV, ALIAS, 1, kDvsHeads), "layout");
  static_assert(LDS_FIXED == NBUF * BUF + dvs_misc_bytes(), "layout");
  static_assert(DV % 256 == 0 && DK % 64 == 0 && DV <= DK, "head dims");
  static_assert(DTW % 4 == 0 && KCPR % 8 == 0 && VCPR % 8 == 0, "8-piece swizzle groups");
  static_assert(KPOS % 128 == 0 && VPOS % 128 == 0, "whole-wave rounds");
  static_assert(LDS_FIXED + kIdxReserve <= 160 * 1024, "LDS budget");
  static_assert(NBUF >= 3 && (NBUF - 3) * CNT < 64, "ring depth / vmcnt range");
};

// LDS writes of this wave done, then the workgroup barrier (no wait on the gathers in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int DK, int DV, bool ALIAS, int NBUF>
__global__ __launch_bounds__(512) void topk_fwd_dvs(TopkParams p) {
  using C = DvsCfg<T, DK, DV, ALIAS, NBUF>;
  using vec8 = typename T::vec8;
  extern __shared__ __align__(16) char smem[];
  float* refs = (float*)(smem + C::OFF_RF);  // [chunk parity][half][head]
  int* cflag = (int*)(smem + C::OFF_CF);
  int* bflag = (int*)(smem + C::OFF_BF);
  int* idxl = (int*)(smem + C::LDS_FIXED);
  auto p_buf = [&](int c, int lo) -> char* { return smem + C::OFF_P + ((c & 1) * 2 + lo) * kDvsPBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool score_wave = wave_u < kDvsWaves / 2;
  const int wr = wave_u & 3;  // head tile (score wave) or dv quarter (value wave)
  const int kg = lane >> 4;   // k-group of this lane in MFMA operands
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
  if (!item_has(p, s1, hb * kDvsHeads)) return;  // head block past a partial block row

  const int32_t* ig;
  int nslots_all;
  if (p.slot_ptr) {
    const int list = item_list(p, s1);
    const int s0 = p.slot_ptr[list];
    ig = p.idx + s0;
    nslots_all = p.slot_ptr[list + 1] - s0;
  } else {
    ig = p.idx + (int64_t)b * p.is[0] + (int64_t)s1 * p.is[1] + (int64_t)n2 * p.is[2];
    nslots_all = p.topK;
  }
  nslots_all = item_slots(p, s1, nslots_all);
  const int item_splits = item_split_count(p, nslots_all);  // as in topk_fwd
  if (split >= item_splits) return;
  const bool direct = item_splits == 1;
  const int slot0 = split * p.split_len;
  const int nslots = max(0, min(p.split_len, nslots_all - slot0));
  const int nchunks = (nslots + C::CH - 1) / C::CH;
  const int h0 = hb * kDvsHeads;

  const int kvh = item_kvh(p, s1, n2);
  const uint16_t* kg_ptr = uniform_ptr(p.k + (int64_t)b * p.ks[0] + (int64_t)kvh * p.ks[2]);
  const uint16_t* vg_ptr = uniform_ptr(p.v + (int64_t)b * p.vs[0] + (int64_t)kvh * p.vs[2]);
  const uint32_t krow_bytes = (uint32_t)p.ks[1] * 2u, vrow_bytes = (uint32_t)p.vs[1] * 2u;
  const uint32_t smem_lds = lds_addr_of(smem);
  const uint32_t jrows = (uint32_t)p.S2;
  auto clamp_row = [&](int j) -> int { return min(max(j, 0), (int)jrows - 1); };

  // ---- prologue.  The split's raw row indices are copied to LDS first; once they have landed
  // the value waves issue chunk 0 of the gather and the score waves copy the workgroup's 64
  // query rows into ring buffers 1.. behind it (every workgroup starts at once, and chunk 0
  // is on the critical path while the query rows are needed only after it has landed).  Query
  // rows are staged piece-major: 16-byte piece cc of row r at position 64 cc + r, so lane i of a
  // copy round always loads row i and the Q^T operand reads (16 rows, one piece) are
  // conflict-free.
  for (int i0 = wave_u * 64; i0 < nslots; i0 += C::NT)
    if (i0 + lane < nslots) lds_dma4(ig + slot0 + i0 + lane, smem_lds + C::LDS_FIXED + i0 * 4);
  for (int i = nslots + tid; i < nchunks * C::CH; i += C::NT) idxl[i] = -1;
  for (int i = tid; i < 5 * kFlagBytes / 4; i += C::NT) cflag[i] = 0;  // mask and rescale flags
  wait_vm_barrier<0>();  // indices landed
  {
    const uint32_t jend_lo =
        (uint32_t)(p.causal ? max(0, min(p.S2, item_row0(p, s1) + h0 / p.HR + (p.S2 - p.QROWS) + 1)) : p.S2);
    for (int i = tid; i < nslots; i += C::NT)
      if (!((uint32_t)idxl[i] < jend_lo)) cflag[i / C::CH] = 1;
    if (tid == 0 && nslots % C::CH != 0) cflag[nslots / C::CH] = 1;
  }

  // ---- gather (value waves): thread g = tid - NG loads position u * NG + g of a chunk in round
  // u (see topk_fwd for the position packing and the whole-wave rounds)
  const int gt = tid - C::NG;
  const int gw = wave_u - kDvsWaves / 2;
  auto pack_pos = [&](int pos, int stride, int cpr) -> int {
    const int r = pos / stride, x = pos % stride;
    const int cc = x < cpr ? ((x & ~7) | ((x ^ stage_xor_w(r)) & 7)) : (x & 3);
    return r | (cc << 8);
  };
  auto round_in = [&](int u, int npos) -> bool {
    if (u * C::NG + C::NG <= npos) return true;
    return u * C::NG + gw * 64 < npos;
  };
  constexpr int NR = C::KLD + (ALIAS ? 0 : C::VLD);
  // pieces past the call's head dims load a piece of the same row (finite values that meet q
  // zeros in QK or fill output columns that are not stored)
  auto clamp_piece = [&](int pk, int cpr) -> int {
    const int cc = pk >> 8;
    return cc < cpr ? pk : (pk & 255) | ((cc % cpr) << 8);
  };
  // (row, piece) of every round, the same for every chunk: computed once by the value waves
  int pk[NR];
#pragma unroll
  for (int u = 0; u < C::KLD; ++u) {
    const int pos = u * C::NG + gt;
    pk[u] = (!score_wave && pos < C::KPOS) ? pack_pos(pos, C::KS, C::KCPR) : 0;
    if (C::KCPR != p.dk / 8) pk[u] = clamp_piece(pk[u], p.dk / 8);
  }
  if constexpr (!ALIAS) {
#pragma unroll
    for (int u = 0; u < C::VLD; ++u) {
      const int pos = u * C::NG + gt;
      pk[C::KLD + u] = (!score_wave && pos < C::VPOS) ? pack_pos(pos, C::VS, C::VCPR) : 0;
      if (C::VCPR != p.dv / 8) pk[C::KLD + u] = clamp_piece(pk[C::KLD + u], p.dv / 8);
    }
  }
  auto issue_gather = [&](int c) {
    const int* irow = idxl + c * C::CH;
    int jrow[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) jrow[r] = irow[pk[r] & 255];
    const uint32_t kb_lds = smem_lds + (c % NBUF) * C::BUF;
#pragma unroll
    for (int u = 0; u < C::KLD; ++u)
      if (round_in(u, C::KPOS))
        lds_dma16_at(kg_ptr, __umul24((uint32_t)clamp_row(jrow[u]), krow_bytes) + ((uint32_t)pk[u] >> 8) * 16u,
                     kb_lds + (u * C::NG + gw * 64) * 16);
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < C::VLD; ++u)
        if (round_in(u, C::VPOS))
          lds_dma16_at(vg_ptr,
                       __umul24((uint32_t)clamp_row(jrow[C::KLD + u]), vrow_bytes) +
                           ((uint32_t)pk[C::KLD + u] >> 8) * 16u,
                       kb_lds + C::KBUF + (u * C::NG + gw * 64) * 16);
    }
  };
  // chunks issued before step 0: 0 .. NBUF - 3 (buffer 0 first; the others once Q^T is read)
  if (!score_wave && nchunks > 0) issue_gather(0);
  if (score_wave) {
    const int h = h0 + lane;
    const bool ok = item_has(p, s1, h);  // else any valid row: head 0
    const uint16_t* qrow = p.q + qv_offset(p, p.qs, b, s1, n2, ok ? h : 0);
#pragma unroll
    for (int u = 0; u < C::QLD; ++u) {
      // piece of this round (wave-uniform); pieces past the call's dk copy an in-row piece, and
      // the score waves zero their Q^T there
      const int pc = u * (kDvsWaves / 2) + wave_u;
      lds_dma16(qrow + (pc % (p.dk / 8)) * 8, smem_lds + C::BUF + pc * 64 * 16);
    }
  }

  // Step t (t = 0 .. nchunks) starts with one barrier, after which chunk t has landed, the
  // softmax of chunk t - 1 is published and the PV product of chunk t - 2 is done everywhere.
  // Then score waves: QK + softmax of chunk t; value waves: gather of chunk t + NBUF - 2 into
  // the buffer of chunk t - 2, PV of chunk t - 1.
  // wait at step t: value waves may leave the chunks after t (issued up to t + NBUF - 3)
  auto step_barrier = [&](int t) {
    if (score_wave) {
      wait_vm_barrier<0>();
    } else {
      switch (min(NBUF - 3, nchunks - 1 - t)) {
        case 1:
          if constexpr (NBUF >= 4) wait_vm_barrier<C::CNT>();
          break;
        default:
          wait_vm_barrier<0>();
      }
    }
  };

  if (score_wave) {
    // ====== score waves: heads h0 + 32 hg .. + 31 (two 16-wide tiles), slots 16 sh .. + 15 ======
    const int hg = wr & 1, sh = wr >> 1;
    uint32_t jend[2];
    float sl2[2];  // logit scale of tile ht's head in log2 units (with per-head factors, if any)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int head = h0 + 32 * hg + 16 * ht + col;
      const int qrow_idx = item_row0(p, s1) + head / p.HR;
      jend[ht] = (uint32_t)(p.causal ? max(0, min(p.S2, qrow_idx + (p.S2 - p.QROWS) + 1)) : p.S2);
      sl2[ht] = p.scale_log2;
      if (p.fq) sl2[ht] *= p.fq[kvh * p.HR + head % p.HR];
      if (p.fk) sl2[ht] *= p.fk[kvh];
    }
    // Q^T of tile ht: k-step ks holds q[head][32 ks + 8 kg .. + 7]
    u32x4 qreg[C::KSTEPS][2];
    wait_vm_barrier<0>();  // query rows landed (this wave's copies; the barrier: everyone's)
    {
      const char* qb = smem + C::BUF + (kg * kDvsHeads + 32 * hg + col) * 16;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          qreg[ks][ht] = *(const u32x4*)(qb + ks * 4 * kDvsHeads * 16 + ht * 16 * 16);
          if (32 * ks + 8 * kg >= p.dk) qreg[ks][ht] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    lds_barrier();  // every score wave has its Q^T before ring buffers 1.. are reused
    // K operand, k-step ks: row 16 sh + col, piece 4 ks + kg, at lane_k[ks % 2] + 128 (ks / 2)
    // (the XOR spans groups of 8 pieces, two k-steps)
    const int rk = 16 * sh + col;
    int lane_k[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) lane_k[p] = (rk * C::KS + ((4 * p + kg) ^ stage_xor_w(rk))) * 16;
    const int hl0 = 32 * hg + col;  // local head of tile 0 (tile 1: + 16)
    float m_run[2] = {-INFINITY, -INFINITY};  // reference agreed by both halves (log2 units)
    float l_run[2] = {0.f, 0.f};              // this lane's share of its half's sum
    float ref[2] = {-INFINITY, -INFINITY};    // reference this half used for the last chunk
    for (int t = 0; t <= nchunks; ++t) {
      step_barrier(t);
      if (t > 0) {
        // adopt the larger of the two halves' references of chunk t - 1
        const float* other = refs + ((t - 1) & 1) * 2 * kDvsHeads + (1 - sh) * kDvsHeads + hl0;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const float M = fmaxf(ref[ht], other[16 * ht]);
          if (M > ref[ht]) l_run[ht] *= fast_exp2(ref[ht] - M);
          m_run[ht] = M;
        }
      }
      if (t == nchunks) break;
      const char* kb = smem + (t % NBUF) * C::BUF;
      const int masked = __builtin_amdgcn_readfirstlane(cflag[t]);  // read ahead of the MFMAs
      f32x4 s[2];
      {
        f32x4 s2[2][2] = {};
        constexpr int KG = 3;
#pragma unroll
        for (int k0 = 0; k0 < C::KSTEPS; k0 += KG) {
          u32x4 a[KG];
#pragma unroll
          for (int g = 0; g < KG; ++g)
            if (k0 + g < C::KSTEPS) a[g] = *(const u32x4*)(kb + lane_k[(k0 + g) & 1] + 128 * ((k0 + g) >> 1));
#pragma unroll
          for (int g = 0; g < KG; ++g)
            if (k0 + g < C::KSTEPS) {
              const int ks = k0 + g < C::KSTEPS ? k0 + g : 0;
#pragma unroll
              for (int ht = 0; ht < 2; ++ht)
                s2[ht][ks & 1] = T::mfma(as<vec8>(a[g]), as<vec8>(qreg[ks][ht]), s2[ht][ks & 1]);
            }
        }
        s[0] = s2[0][0] + s2[0][1];
        s[1] = s2[1][0] + s2[1][1];
      }
      // mask (element e: slot 16 sh + 4 kg + e)
      float x[2][4];
      if (masked) {
        const u32x4 jj = *(const u32x4*)(idxl + t * C::CH + 16 * sh + 4 * kg);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[ht][e] = (uint32_t)jj[e] < jend[ht] ? s[ht][e] : -INFINITY;
      } else {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[ht][e] = s[ht][e];
      }
      float mx[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
        mx[ht] = fmaxf(fmaxf(x[ht][0], x[ht][1]), fmaxf(x[ht][2], x[ht][3])) * sl2[ht];
      ref[0] = m_run[0];
      ref[1] = m_run[1];
      // a half moves its reference only where it exceeds the agreed one by more than kLazyRescale
      if (__builtin_amdgcn_ballot_w64(mx[0] > m_run[0] + kLazyRescale || mx[1] > m_run[1] + kLazyRescale)) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const float hm = wave_max_lanes<16>(mx[ht]);
          if (hm > m_run[ht] + kLazyRescale) {
            l_run[ht] *= fast_exp2(m_run[ht] - hm);  // 0 when nothing was seen yet
            ref[ht] = hm;
          }
          if (__builtin_amdgcn_ballot_w64(ref[ht] != m_run[ht]) && lane == 0) bflag[t * 4 + 2 * hg + ht] = 1;
        }
      }
      if (kg == 0) {
        float* mine = refs + (t & 1) * 2 * kDvsHeads + sh * kDvsHeads + hl0;
        mine[0] = ref[0];
        mine[16] = ref[1];
      }
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float m_use = ref[ht] == -INFINITY ? 0.f : ref[ht];
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[e] = fast_exp2(__builtin_fmaf(x[ht][e], sl2[ht], -m_use));
          l_run[ht] += pr[e];
        }
        u32x2 hi, lo;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint32_t h, l;
          split2<T>(pr[2 * i], pr[2 * i + 1], h, l);
          hi[i] = h;
          lo[i] = l;
        }
        const int off = ((hl0 + 16 * ht) * kDvsPRow + 16 * sh + 4 * kg) * 2;
        *(u32x2*)(p_buf(t, 0) + off) = hi;
        *(u32x2*)(p_buf(t, 1) + off) = lo;
      }
    }
    // head totals for the value waves: agreed reference and the two half sums, in the P buffer
    // that the last step leaves free (the value waves still read the last chunk's P)
    float* tot = (float*)p_buf(nchunks, 0);  // [max][64], then [half][64] sums
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const float l_half = wave_sum_lanes<16>(l_run[ht]);
      if (kg == 0) {
        if (sh == 0) tot[hl0 + 16 * ht] = m_run[ht];
        tot[kDvsHeads + sh * kDvsHeads + hl0 + 16 * ht] = l_half;
      }
    }
    lds_barrier();
  } else {
    // ================= value waves: dv columns [wr Dv/4, (wr+1) Dv/4) of all 64 heads =================
    // the score waves' query rows landed (the barrier); this wave's chunk 0 may be in flight
    if (nchunks > 0) wait_vm_barrier<C::CNT>();
    else wait_vm_barrier<0>();
    lds_barrier();  // the score waves have read their Q^T
#pragma unroll
    for (int i = 1; i < NBUF - 2; ++i)
      if (i < nchunks) issue_gather(i);
    // V^T operand, dv tile dt (global 16-wide tile g = wr * DTW + dt), half hh: lane c16 of
    // k-group kg reads row 8 kg + 4 hh + c16 / 4 at dv 16 g + 4 (c16 % 4), so it receives dv
    // 16 g + c16 of slots 8 kg + 4 hh .. + 3 (MFMA k index = slot)
    // (the XOR spans groups of 8 pieces, four dv tiles: tile g at lane_v[hh][g % 4] + 128 (g / 4))
    int lane_v[2][4];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 8 * kg + 4 * hh + (col >> 2);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lane_v[hh][j] = (r * C::VS + ((2 * j + ((col & 3) >> 1)) ^ stage_xor_w(r))) * 16 + 8 * (col & 1);
    }
    const int vwave = wr * C::DTW * 2 * 16;  // byte offset of this wave's first dv piece (2 per tile)
    // P^T operand, head tile ht: P[16 ht + col][8 kg .. + 7]
    const int lane_p = (col * kDvsPRow + 8 * kg) * 2;
    f32x4 acc[C::DTW][4];  // O^T: dv 16 (wr DTW + dt) + 4 kg + e, head 16 ht + col
    float m_acc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // reference of acc[.][ht]
#pragma unroll
    for (int dt = 0; dt < C::DTW; ++dt)
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t <= nchunks; ++t) {
      step_barrier(t);
      if (t + NBUF - 2 < nchunks) issue_gather(t + NBUF - 2);
      if (t == 0) continue;
      const int c = t - 1;
      const char* kb = smem + (c % NBUF) * C::BUF;
      const char* vb = ALIAS ? kb : kb + C::KBUF;
      u32x4 bh[4], bl[4];
      const char* phi = p_buf(c, 0) + lane_p;
      const char* plo = p_buf(c, 1) + lane_p;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        bh[ht] = *(const u32x4*)(phi + ht * 16 * kDvsPRow * 2);
        bl[ht] = *(const u32x4*)(plo + ht * 16 * kDvsPRow * 2);
      }
      // where a half moved its reference in chunk c (flags of the 4 head tiles): bring the
      // accumulators and both halves' P to the larger reference (the P^T operand of this lane
      // holds slots 8 kg .. + 7: half kg / 2)
      const u32x4 bf = *(const u32x4*)(bflag + c * 4);
      if (__builtin_amdgcn_readfirstlane(bf[0] | bf[1] | bf[2] | bf[3])) {
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          if (__builtin_amdgcn_readfirstlane(bf[ht])) {
            const float* rc = refs + (c & 1) * 2 * kDvsHeads + 16 * ht + col;
            const float r0 = rc[0], r1 = rc[kDvsHeads];
            const float M = fmaxf(r0, r1);
            if (M != -INFINITY) {
              const float a = fast_exp2(m_acc[ht] - M);  // 0 while nothing was accumulated
#pragma unroll
              for (int dt = 0; dt < C::DTW; ++dt) acc[dt][ht] *= a;  // accumulators stay in VGPRs
              m_acc[ht] = M;
              const float f = fast_exp2((kg < 2 ? r0 : r1) - M);
              if (f != 1.f) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  v[2 * i] = (T::to_float((uint16_t)bh[ht][i]) + T::to_float((uint16_t)bl[ht][i])) * f;
                  v[2 * i + 1] = (T::to_float((uint16_t)(bh[ht][i] >> 16)) + T::to_float((uint16_t)(bl[ht][i] >> 16))) * f;
                }
                split_hi_lo<T>(v, bh[ht], bl[ht]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int dt = 0; dt < C::DTW; ++dt) {
        const int off = vwave + 128 * (dt >> 2);
        const u32x2 v0 = lds_read_tr16(vb + lane_v[0][dt & 3] + off);
        const u32x2 v1 = lds_read_tr16(vb + lane_v[1][dt & 3] + off);
        const u32x4 a = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = T::mfma(as<vec8>(a), as<vec8>(bh[ht]), acc[dt][ht]);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = T::mfma(as<vec8>(a), as<vec8>(bl[ht]), acc[dt][ht]);
      }
    }
    lds_barrier();  // the score waves published the head totals
    const float* tot = (const float*)p_buf(nchunks, 0);
    if (p.fv) {
      const float f = p.fv[kvh];
#pragma unroll
      for (int dt = 0; dt < C::DTW; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) acc[dt][ht] *= f;
    }
    // ---- epilogue
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int hh = h0 + 16 * ht + col;
      if (!item_has(p, s1, hh)) continue;
      const float M = tot[16 * ht + col];
      const float L = tot[kDvsHeads + 16 * ht + col] + tot[2 * kDvsHeads + 16 * ht + col];
      const int dv0 = wr * C::DTW * 16 + 4 * kg;
      if (direct) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t* orow = p.out + qv_offset(p, p.os, b, s1, n2, hh);
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt) {
          if (dv0 + 16 * dt >= p.dv) continue;
          u32x2 w;
          w[0] = (uint32_t)T::from_float(acc[dt][ht][0] * inv) | ((uint32_t)T::from_float(acc[dt][ht][1] * inv) << 16);
          w[1] = (uint32_t)T::from_float(acc[dt][ht][2] * inv) | ((uint32_t)T::from_float(acc[dt][ht][3] * inv) << 16);
          *(u32x2*)(orow + dv0 + 16 * dt) = w;
        }
        if (p.lse && wr == 0 && kg == 0)
          p.lse[qv_offset(p, p.ls, b, s1, n2, hh)] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
      } else {
        const int64_t row = ws_row(p, b, s1, n2, hh);
        float* po = p.ws_o + (row * p.nsplit + split) * DV + dv0;
#pragma unroll
        for (int dt = 0; dt < C::DTW; ++dt) *(f32x4*)(po + 16 * dt) = acc[dt][ht];
        if (wr == 0 && kg == 0) {
          float* pm = p.ws_ml + (row * p.nsplit + split) * 2;
          pm[0] = M;
          pm[1] = L;
        }
      }
    }
  }
}

}  // namespace sfa
