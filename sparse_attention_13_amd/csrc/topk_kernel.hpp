// Top-K sparse flash attention kernels for gfx950.
//
// Operator (SparseFlashAttention operator page, section 2): for each query row
// (b, s1, n1), gather the topK key/value rows named by the index row of its
// KV-head group (b, s1, n2 = n1 / G), take softmax(q K_sel^T * scale) over the
// topK axis after the optional bottom-right causal mask, and multiply by V_sel.
//
// Work decomposition.  A work item is (group (b, n2, s1), head block, split):
// the G query heads of a group share one index row, so one gathered K/V tile
// in LDS serves all of them.  A workgroup has WH x WS waves: WH head tiles of MT
// heads each (MT = 16 or 32, the N dim of the 16x16x32 / 32x32x16 MFMAs) times
// WS waves that take disjoint 32-slot parts of each staged chunk of CH = 32*WS
// slots.
//
// Per chunk:  the 16-byte pieces of the CH selected rows are loaded straight into
// LDS (XOR-swizzled rows, issued one chunk ahead of their use), then per wave:
//   S^T[32 slots x MT heads] = K_sel Q^T          (MFMA, K from LDS, Q in VGPRs)
//   online softmax in fp32, log2 domain            (one head per lane column)
//   O^T[Dv x MT heads] += V_sel^T (P_hi + P_lo)^T  (MFMA, V^T by LDS transpose reads)
// P enters the PV product as two 16-bit parts (hi = round(P), lo = round(P - hi))
// so the product carries about 16 (bf16) / 22 (fp16) significand bits of P.
//
// A split of the topK axis (decode shapes with few groups) writes the partial
// (O, running max, running sum) to the float workspace; topk_merge combines the
// splits with the log-sum-exp rule.
#pragma once

#include "common.hpp"

namespace sfa {

// A work item is (b, s1, n2, head block, split).  Its G "heads" are the query vectors that
// share one index list: query head h of the KV group for top-K attention; for block-sparse
// attention, query row s1 * RS + h / HR of block row s1 with query head n2 * HR + h % HR;
// with an item table (variable block sizes), query row row0 + h / HR of the entry's rows,
// query head kvh * HR + h % HR.

// One entry of the item table: query rows row0 .. row0 + nrows - 1 (nrows <= RS) of KV head
// kvh, whose key list is idx[slot_ptr[list] .. slot_ptr[list + 1]).
struct TopkItem {
  int row0, nrows, kvh, list;
};
struct TopkParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  // null: item (b, s1, n2) has topK slots at idx + b * is[0] + s1 * is[1] + n2 * is[2];
  // else: its slots are idx[slot_ptr[s1] .. slot_ptr[s1 + 1])
  const int32_t* slot_ptr;
  uint16_t* out;
  float* lse;
  float* ws_o;   // [rows, nsplit, Dv] partial outputs (unnormalised)
  float* ws_ml;  // [rows, nsplit, 2] (running max in log2 units, running sum)
  // element strides: (batch, seq, head, query row inside an item) for q, out and lse;
  // (batch, seq, head) for k, v and idx
  int64_t qs[4], ks[3], vs[3], is[3], os[4], ls[4];
  int B, S1, S2, N2, G, topK, causal;
  // head dims of the call (multiples of 64, dk <= DK and dv <= DV of the kernel): q columns past
  // dk enter the products as zeros, output columns past dv are not stored
  int dk, dv;
  int HR;     // query heads per KV head
  int RS;     // query rows per item row s1
  int QROWS;  // query rows in all (sets the bottom-right causal limit)
  float scale_log2;  // scale * log2(e)
  // Optional per-head logit factors (null: 1): the logit of query vector h is further
  // multiplied by fq[query head] * fk[KV head] (positive; FP8 inputs decoded without them)
  const float* fq;
  const float* fk;
  // Optional per-KV-head output factor (null: 1): the output row (and its split partials) of
  // every query vector of KV head hk is multiplied by fv[hk] (the factor of FP8 values)
  const float* fv;
  int nsplit, split_len, HB;
  int n_items;
  // Optional element mask of block-sparse items (null: none).  The slots of item row s1 are
  // cut into 32-slot words bm_wptr[s1] .. bm_wptr[s1 + 1] - 1; word w holds, for query row i
  // of the item row (i < RS), the bits bm_words[w * RS + i] (bit b: slot 32 (w - bm_wptr[s1])
  // + b is attended) and bm_wflag[w] != 0 when some bit of the word is clear.
  const uint32_t* bm_words;
  const int32_t* bm_wptr;
  const int32_t* bm_wflag;
  // Optional item table (null: none), one entry per item row s1; with a table N2 = 1, B = 1
  // and the per-item rows, KV head and key list come from the entry (q / out / lse use the
  // head stride st[2] and the row stride st[3]; st[1] is not used).
  const TopkItem* itab;
  // Every key list is the keys 0, 1, 2, ... in order (dense attention): with causal, an item
  // then needs only the keys below the causal limit of its last query row.
  int dense;
};

// Element offset of the query vector (b, s1, n2, virtual head h) in q, out (st = qs / os) or
// lse (st = ls), and its flat row in the split workspace.
__device__ __forceinline__ int64_t qv_offset(const TopkParams& p, const int64_t* st, int b, int s1, int n2, int h) {
  if (p.itab) {
    const TopkItem t = p.itab[s1];
    return (int64_t)(t.row0 + h / p.HR) * st[3] + (int64_t)(t.kvh * p.HR + h % p.HR) * st[2];
  }
  return (int64_t)b * st[0] + (int64_t)s1 * st[1] + (int64_t)(h / p.HR) * st[3] +
         (int64_t)(n2 * p.HR + h % p.HR) * st[2];
}
// First query row of item row s1, and whether its virtual head h is a query that exists (the
// last block row may be partial; table entries hold nrows rows).
__device__ __forceinline__ int item_row0(const TopkParams& p, int s1) {
  return p.itab ? p.itab[s1].row0 : s1 * p.RS;
}
__device__ __forceinline__ bool item_has(const TopkParams& p, int s1, int h) {
  return h < p.G && (p.itab ? h / p.HR < p.itab[s1].nrows : s1 * p.RS + h / p.HR < p.QROWS);
}
// KV head and key list of item (s1, n2)
__device__ __forceinline__ int item_kvh(const TopkParams& p, int s1, int n2) { return p.itab ? p.itab[s1].kvh : n2; }
__device__ __forceinline__ int item_list(const TopkParams& p, int s1) { return p.itab ? p.itab[s1].list : s1; }

// Index slots of item row s1 that can be attended, of its n_all: all of them, except that a
// causal item of a dense list stops at the limit of its last query row (the keys past it are
// masked for every row of the item).
__device__ __forceinline__ int item_slots(const TopkParams& p, int s1, int n_all) {
  if (!(p.dense && p.causal)) return n_all;
  const int rows = p.itab ? p.itab[s1].nrows : min(p.RS, p.QROWS - s1 * p.RS);
  const int last = item_row0(p, s1) + rows - 1;
  return min(n_all, max(0, min(p.S2, last + (p.S2 - p.QROWS) + 1)));
}

// Splits an item with n index slots takes (at least one).
__device__ __forceinline__ int item_split_count(const TopkParams& p, int n) {
  return max(1, (n + p.split_len - 1) / p.split_len);
}

__device__ __forceinline__ int64_t ws_row(const TopkParams& p, int b, int s1, int n2, int h) {
  return (((int64_t)b * p.S1 + s1) * p.N2 + n2) * p.G + h;
}

constexpr int kMaxSplitLen = 2048;  // index slots staged in LDS per work item (topk_fwd_dvs)
constexpr int kTopkMaxSplitLen = 4096;  // the same for topk_fwd

// MFMA tile geometry.  MT x MT output tile, K = 512 / MT per instruction; every
// lane feeds 8 consecutive k values of row (lane % MT) of each operand, and holds
// NACC outputs: column lane % MT, rows row_of(E) for E < NACC.
template <typename T, int MT>
struct Tile;

template <typename T>
struct Tile<T, 16> {
  using acc_t = f32x4;
  static constexpr int NACC = 4;
  static constexpr int KSTEP = 32;
  static __device__ __forceinline__ acc_t mfma(typename T::vec8 a, typename T::vec8 b, acc_t c) {
    return T::mfma(a, b, c);
  }
};

template <>
struct Tile<half_t, 32> {
  using acc_t = f32x16;
  static constexpr int NACC = 16;
  static constexpr int KSTEP = 16;
  static __device__ __forceinline__ acc_t mfma(f16x8 a, f16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Tile<bfloat_t, 32> {
  using acc_t = f32x16;
  static constexpr int NACC = 16;
  static constexpr int KSTEP = 16;
  static __device__ __forceinline__ acc_t mfma(bf16x8 a, bf16x8 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// MFMA tile width (N dim) of a head tile of MT heads.  MT = 8 is the packed form of the
// 16-wide tile: its columns c and c + 8 both belong to head c, column c scoring the first 16
// slots of each 32-slot part and column c + 8 the other 16, so groups of G <= 8 query vectors
// leave no tile column idle in the softmax.
constexpr int topk_tile_n(int MT) { return MT == 8 ? 16 : MT; }

// Output row of accumulator element E for a lane in k-group kg = lane / MT.
template <int MT>
__device__ __forceinline__ int acc_row(int E, int kg) {
  return (E >> 2) * (256 / MT) + 4 * kg + (E & 3);
}

// Q^T k-steps kept in VGPRs (the rest is read from LDS): for the widest head dims Q plus
// the O accumulators would otherwise overflow the register file.
constexpr int topk_qreg(int DK, int DV, int MT) {
  const int ksteps = DK * topk_tile_n(MT) / 512;
  const int acc_regs = DV * topk_tile_n(MT) / 64;
  const int fit = (364 - acc_regs) / 4;
  const int q = fit < ksteps / 2 ? ksteps / 2 : fit;
  return q < ksteps ? q : ksteps;
}

constexpr int kIdxReserve = 4096;  // LDS bytes reserved for flags + index slots when sizing the ring
constexpr int kFlagBytes = 256;    // per-chunk "needs the mask" flags (kMaxSplitLen / 32 chunks at most)
// topk_fwd keeps one byte per chunk (kTopkMaxSplitLen / 32 chunks): the flag area also
// bounds the workgroups per CU of LDS-bound shapes (six single-wave GQA prefill workgroups)
constexpr int kTopkFlagBytes = 128;
static_assert(kFlagBytes < kIdxReserve && kTopkFlagBytes < kIdxReserve, "flags come out of the index reserve");
static_assert(kTopkFlagBytes * 32 == kTopkMaxSplitLen, "one flag byte per 32-slot chunk");

// Staged K rows are pad-free (stage_xor_pf) for 16-wide head tiles with V a view of K and
// KCPR a multiple of 8; the swizzle group (8 or 16 chunks) is returned, 0 for padded rows.
constexpr int topk_pad_free(int DK, bool alias, int MT) {
  return (topk_tile_n(MT) == 16 && alias && (DK / 8) % 8 == 0) ? ((DK / 8) % 16 == 8 ? 8 : 16) : 0;
}
constexpr int topk_kstride(int DK, bool alias, int MT) {
  return topk_pad_free(DK, alias, MT) ? DK / 8 : staged_stride(DK / 8);
}

// LDS bytes of one staged chunk (K rows, plus V rows when V is not a view of K).
constexpr int topk_chunk_bytes(int DK, int DV, bool alias, int WS, int MT) {
  const int ch = 32 * WS;
  return ch * topk_kstride(DK, alias, MT) * 16 + (alias ? 0 : ch * staged_stride(DV / 8) * 16);
}

constexpr int topk_qlds_bytes(int DK, int DV, int MT, int WH) {
  return (DK * topk_tile_n(MT) / 512 - topk_qreg(DK, DV, MT)) * 1024 * WH;
}

// Row stride (floats) of the slot-part merge through LDS: one head row per lane column; a
// stride of 4 floats past Dv puts the 16-byte stores of adjacent columns on different banks
// (with a stride of Dv, 8 adjacent columns of a store hit the same banks).
constexpr int topk_merge_stride(int DV) { return DV + 4; }

// Workgroup shape and ring depth: WS slot-parallel waves and NBUF chunk buffers, chosen to
// maximise the bytes of gathered rows in flight per CU (NBUF - 1 chunks per workgroup times
// the workgroups that fit in 160 KB of LDS), preferring shapes that keep at least 4 waves
// per CU.  The wide form (chosen by the host for launches with many more work items than
// CUs) is one wave and a two-chunk ring, the most workgroups per CU: there each wave's
// serial gather -> QK -> softmax -> PV chain is hidden by the other waves rather than by a
// deeper ring.  Returns WS * 16 + NBUF, or 0 if nothing fits.
constexpr int topk_pick(int DK, int DV, bool alias, int MT, int WH, bool wide) {
  int best = 0;
  long best_score = -1;
  for (int ws = (wide || WH >= 4) ? 1 : 4 / WH; ws >= 1; ws /= 2) {
    const int buf = topk_chunk_bytes(DK, DV, alias, ws, MT);
    const int merge = ws == 1 ? 0 : ws * WH * MT * (topk_merge_stride(DV) + 2) * 4;
    // 16-wide tiles (memory-bound shapes) stop at 3 buffers: on GQA decode a fourth made the
    // kernel 7-9% slower, with or without the pipelined loop
    for (int nbuf = 2; nbuf <= (wide ? 2 : (MT <= 16 ? 3 : 8)); ++nbuf) {
      const int fixed = nbuf * buf + topk_qlds_bytes(DK, DV, MT, WH);
      const int lds = fixed + kIdxReserve;
      if (lds > 160 * 1024 || merge > nbuf * buf) continue;
      // loads per thread per chunk must keep (nbuf - 2) chunks countable in vmcnt (< 64)
      const int nt = 64 * WH * ws;
      const int per_chunk = buf / 16 / nt + 2;
      if ((nbuf - 2) * per_chunk >= 64) continue;
      const int wgs = (160 * 1024) / lds;
      const int waves = wgs * WH * ws;
      long score = (waves >= 4 ? (1L << 40) : 0) + (long)wgs * (nbuf - 1) * buf;
      // 16-wide tiles: decode-like launches have about one work item per CU, so several
      // workgroups per CU would only come from splitting the index lists (and merging them
      // again); they count the bytes in flight of one workgroup of >= 4 waves instead
      if (MT <= 16) score = (WH * ws >= 4 ? (1L << 40) : 0) + (long)(nbuf - 1) * buf;
      if (score > best_score) {
        best_score = score;
        best = ws * 16 + nbuf;
      }
    }
  }
  return best;
}

// Loader waves: waves that only issue gathers.  Gathers into LDS are bound by the loads in
// flight per wave, not only per CU, so the same bytes in flight land sooner from more waves.
// 16-wide single-tile workgroups of four slot parts (the decode shapes, one workgroup per CU)
// add four, so eight waves share each chunk's loads; the single-wave form (prefill shapes,
// many workgroups per CU) adds one.  Only where the registers leave room (Dv <= 192).
constexpr int topk_loader_waves(int DV, int MT, int WH, int WS) {
  if (topk_tile_n(MT) != 16 || WH != 1 || DV > 192) return 0;
  return WS == 4 ? 4 : (WS == 1 ? 1 : 0);
}

template <typename T, int DK, int DV, bool ALIAS, int MT, int WH, int WS, int NBUF>
struct TopkCfg {
  static constexpr bool PK = MT == 8;          // packed 16-wide tile (8 heads x 2 slot groups)
  static constexpr int MN = topk_tile_n(MT);   // MFMA tile width
  static constexpr int NCW = WH * WS;  // compute waves
  static constexpr int LW = topk_loader_waves(DV, MT, WH, WS);
  static constexpr int NWAVES = NCW + LW;
  static constexpr int NT = 64 * NWAVES;  // threads
  static constexpr int CH = 32 * WS;       // slots per staged chunk
  static constexpr int KCPR = DK / 8;  // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;
  static constexpr int PF = topk_pad_free(DK, ALIAS, MT);   // pad-free K rows: swizzle group, or 0
  static constexpr int KS = topk_kstride(DK, ALIAS, MT);  // staged K row stride, in chunks
  static constexpr int VS = ALIAS ? KS : staged_stride(VCPR);
  static constexpr int KPOS = CH * KS;                   // staged positions per chunk (with pads)
  static constexpr int VPOS = ALIAS ? 0 : CH * VS;
  // threads that issue the gathers: the loader waves where there are any (the compute waves
  // then never stall on a gather issue), else every wave
  static constexpr int GT = LW > 0 ? 64 * LW : NT;
  static constexpr int GW = GT / 64;
  static constexpr int KLD = (KPOS + GT - 1) / GT;       // load rounds per gathering thread per chunk
  static constexpr int VLD = (VPOS + GT - 1) / GT;
  // load instructions per chunk that every gathering wave issues (rounds where even the last one
  // has an active lane); the vmcnt waits count with this lower bound (waves that issue none have
  // nothing outstanding)
  static constexpr int rounds_all(int pos, int ld) {
    int n = 0;
    for (int u = 0; u < ld; ++u) n += (u * GT + 64 * (GW - 1) < pos) ? 1 : 0;
    return n;
  }
  static constexpr int CNT = rounds_all(KPOS, KLD) + rounds_all(VPOS, VLD);
  static constexpr int KSTEPS = DK / Tile<T, MN>::KSTEP;  // QK MFMAs per S tile (per slot group if PK)
  static constexpr int NST = PK ? 1 : 32 / MN;             // S tiles per 32-slot part
  static constexpr int PVK = 32 / Tile<T, MN>::KSTEP;      // PV k-steps per 32-slot part
  static constexpr int DT = DV / MN;                       // dv tiles
  static constexpr int KBUF = KPOS * 16;
  static constexpr int VBUF = VPOS * 16;
  static constexpr int BUF = KBUF + VBUF;
  static constexpr int QREG = topk_qreg(DK, DV, MT);
  static constexpr int QLDS = topk_qlds_bytes(DK, DV, MT, WH);  // [WH][KSTEPS - QREG][64 lanes][16 B]
  static constexpr int LDS_FIXED = NBUF * BUF + QLDS + kTopkFlagBytes;  // index slots follow (4 B each)
  // element-mask words (only with a block-sparse mask): [NBUF][WS][MW] after the index slots,
  // MW >= the query rows of a workgroup's heads, whole 64-word DMA rounds
  static constexpr int MW = (MT * WH + 63) / 64 * 64;
  static constexpr int MASK_BYTES = NBUF * WS * MW * 4;
  static_assert(BUF == topk_chunk_bytes(DK, DV, ALIAS, WS, MT), "layout");
  static_assert(DK % 64 == 0 && DV % 64 == 0 && DV <= DK, "head dims");
  static_assert(!PK || (QREG == KSTEPS && WH == 1), "packed tiles keep Q in registers, one head tile");
  static_assert(LDS_FIXED - kTopkFlagBytes + kIdxReserve <= 160 * 1024, "LDS budget");
  static_assert(NBUF >= 2 && (NBUF - 2) * CNT < 64, "vmcnt range");
  // cross-wave merge of WS slot parts reuses the chunk buffers
  static_assert(WS == 1 || WS * WH * MT * (topk_merge_stride(DV) + 2) * 4 <= NBUF * BUF, "merge scratch");
};

// Wait until at most N vector-memory operations of this wave are outstanding (and its LDS
// operations are done), then join the workgroup barrier.  Also a compiler memory barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(0), as a builtin the compiler's wait tracking accounts for
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; others at maximum).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// HF: the launch may carry per-head logit factors (p.fq / p.fk); without it the logit scale
// stays one wave-uniform value.
template <typename T, int DK, int DV, bool ALIAS, int MT, int WH, int WS, int NBUF, bool HF = false>
__global__ __launch_bounds__(64 * (WH * WS + topk_loader_waves(DV, MT, WH, WS))) void topk_fwd(TopkParams p) {
  using C = TopkCfg<T, DK, DV, ALIAS, MT, WH, WS, NBUF>;
  constexpr bool PK = C::PK;
  constexpr int MN = C::MN;
  using TL = Tile<T, MN>;
  using acc_t = typename TL::acc_t;
  using vec8 = typename T::vec8;
  constexpr int NACC = TL::NACC;
  extern __shared__ __align__(16) char smem[];
  // ring of NBUF chunk buffers, each [K rows][V rows]; then Q^T k-steps; then index slots
  char* qlds = smem + NBUF * C::BUF;
  int* idxl = (int*)(smem + C::LDS_FIXED);
  uint8_t* cflag = (uint8_t*)(smem + C::LDS_FIXED - kTopkFlagBytes);  // [chunk]: some slot needs the mask

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wh = wave % WH;
  const int wsl = wave / WH;
  const bool loader = C::LW > 0 && wave >= C::NCW;  // issues gathers only (wave-uniform)
  const bool gwave = C::LW == 0 || loader;          // issues gathers (all of them, with loaders)
  const int gt = C::LW > 0 ? tid - 64 * C::NCW : tid;  // gathering thread index (when gwave)
  const int kg = lane / MN;     // k-group of this lane in MFMA operands
  const int col = lane % MN;    // MFMA column of this lane
  const int hcol = PK ? col % 8 : col;  // its head column (packed tiles: columns c, c + 8 -> c)
  const int grp = PK ? col / 8 : 0;     // packed tiles: the 16-slot group this column scores
  const int q16 = lane >> 4;    // 16-lane group (transpose reads)
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
  // a head block with no query (past a partial block row) has nothing to do
  if (!item_has(p, s1, hb * MT * WH)) return;

  const int32_t* ig;  // this item's index slots
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
  // splits of this item: a list shorter than the longest may need fewer, and a list with one
  // split writes its output directly (no partials to merge)
  const int item_splits = item_split_count(p, nslots_all);
  if (split >= item_splits) return;
  const bool direct = item_splits == 1;
  const int slot0 = split * p.split_len;
  const int nslots = max(0, min(p.split_len, nslots_all - slot0));
  const int nchunks = (nslots + C::CH - 1) / C::CH;

  // element mask (block-sparse items): first word of this split, end of the item row's words,
  // and the query rows of the item row that this workgroup's heads belong to
  int bm_w0 = 0, bm_wend = 1, bm_row0 = 0, bm_nrows = 1;
  if (p.bm_words) {
    bm_w0 = p.bm_wptr[s1] + slot0 / 32;
    bm_wend = p.bm_wptr[s1 + 1];
    bm_row0 = hb * MT * WH / p.HR;
    bm_nrows = min(p.RS - bm_row0, (hb * MT * WH + MT * WH - 1) / p.HR - bm_row0 + 1);
  }

  const int head = hb * MT * WH + wh * MT + hcol;  // virtual head of this lane's column
  const int qrow_idx = item_row0(p, s1) + head / p.HR;  // its query row
  const bool head_ok = item_has(p, s1, head);
  const int hv = head_ok ? head : 0;

  // K / V rows of this (b, n2): row j at byte j * krow_bytes (the host checks that every row
  // of the slice lies within 4 GiB of its base and that S2 and the row pitch fit in 24 bits)
  const int kvh = item_kvh(p, s1, n2);
  // logit scale of this lane's head in log2 units (with the per-head factors, if any)
  float sl2 = p.scale_log2;
  if constexpr (HF) {
    if (p.fq) sl2 *= p.fq[kvh * p.HR + hv % p.HR];
    if (p.fk) sl2 *= p.fk[kvh];
  }
  const uint16_t* kg_ptr = uniform_ptr(p.k + (int64_t)b * p.ks[0] + (int64_t)kvh * p.ks[2]);
  const uint16_t* vg_ptr = uniform_ptr(p.v + (int64_t)b * p.vs[0] + (int64_t)kvh * p.vs[2]);
  const uint32_t krow_bytes = (uint32_t)p.ks[1] * 2u, vrow_bytes = (uint32_t)p.vs[1] * 2u;

  // ---- Q^T operand: lane holds q[head][KSTEP*ks + 8*kg .. +7]; k-steps >= QREG live in LDS.
  // All Q loads are issued first so that their latency overlaps the index staging below.
  constexpr int QL = C::KSTEPS - C::QREG;  // k-steps staged through LDS
  // Packed tiles keep two copies, [group][k-step]: group g's copy holds q in the columns of
  // group g and zeros in the others, so the products of the two slot groups land in their
  // own columns of one tile.
  u32x4 qreg[C::QREG * (PK ? 2 : 1)];
  u32x4 qstage[QL > 0 ? QL : 1];
  {
    const uint16_t* qrow = p.q + qv_offset(p, p.qs, b, s1, n2, hv);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < C::QREG; ++ks) {
      const u32x4 qv = head_ok && !loader && ks * TL::KSTEP + kg * 8 < p.dk
                           ? *(const u32x4*)(qrow + ks * TL::KSTEP + kg * 8) : z;
      if constexpr (PK) {
        qreg[ks] = grp == 0 ? qv : z;
        qreg[C::QREG + ks] = grp == 1 ? qv : z;
      } else {
        qreg[ks] = qv;
      }
    }
    if (wsl == 0) {
#pragma unroll
      for (int i = 0; i < QL; ++i)
        qstage[i] = head_ok && (C::QREG + i) * TL::KSTEP + kg * 8 < p.dk
                        ? *(const u32x4*)(qrow + (C::QREG + i) * TL::KSTEP + kg * 8)
                        : z;
    }
  }

  // ---- stage this split's raw row indices in LDS (straight from global memory, 256 B per wave
  // instruction); the slots of the last chunk past nslots hold -1.  Whether a slot selects a
  // row is decided at use: slot value j is a row iff 0 <= j < S2 (else the gather reads row 0),
  // and this lane's query attends to it iff also j < jend, the bottom-right causal limit
  // qrow + (S2 - QROWS) + 1 when causal.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t smem_lds = lds_addr_of(smem);
  {
    for (int i0 = wave_u * 64; i0 < nslots; i0 += C::NT)
      if (i0 + lane < nslots) lds_dma4(ig + slot0 + i0 + lane, smem_lds + C::LDS_FIXED + i0 * 4);
    for (int i = nslots + tid; i < nchunks * C::CH; i += C::NT) idxl[i] = -1;
  }
  const uint32_t jrows = (uint32_t)p.S2;
  const uint32_t jend = (uint32_t)(p.causal ? max(0, min(p.S2, qrow_idx + (p.S2 - p.QROWS) + 1)) : p.S2);
  // a slot that is no row is gathered from a row in range (it is masked in the softmax)
  auto clamp_row = [&](int j) -> int { return min(max(j, 0), (int)jrows - 1); };
  auto selects = [&](int j) -> bool { return (uint32_t)j < jend; };

  // Q loads and index copies complete (a wait the compiler sees: the ring's own vmcnt waits
  // are inline asm it cannot read, so it would otherwise wait for vmcnt(0) -- every gather
  // load in flight -- before the first use of Q inside the loop).
  for (int i = tid; i < kTopkFlagBytes / 4; i += C::NT) ((int*)cflag)[i] = 0;
  wait_vm_all();
  if (wsl == 0) {
#pragma unroll
    for (int i = 0; i < QL; ++i) *(u32x4*)(qlds + ((wh * QL + i) * 64 + lane) * 16) = qstage[i];
  }
  __syncthreads();
  // ---- gather: 16-byte pieces of the selected rows go straight from HBM to LDS (swizzled
  // positions); each wave instruction fills 1 KB of LDS, lane i at byte 16*i.
  // DMA rounds: the (row, chunk) each thread loads in round u is the same for every chunk;
  // precompute it once, packed as row | chunk << 8.  A chunk holds CH rows of KS (VS)
  // positions, a multiple of 128, so a wave's 64 positions of a round are either all inside
  // the chunk or all past its end: the skip is wave-uniform and no lane is masked off.  The
  // pad positions of a row (KCPR <= x < KS, never read) load chunk x & 3 of their own row,
  // a line the same instruction fetches anyway.
  static_assert(C::KPOS % 128 == 0 && C::VPOS % 128 == 0, "whole-wave rounds");
  auto pack_pos = [&](int pos, int stride, int cpr) -> int __attribute__((always_inline)) {
    const int r = pos / stride, x = pos % stride;
    const int cc = x < cpr ? ((x & ~3) | ((x & 3) ^ stage_xor(r))) : (x & 3);
    return r | (cc << 8);
  };
  auto pack_pos_pf = [&](int pos) -> int {  // pad-free K rows
    constexpr int S = C::PF ? C::PF : 8;
    const int r = pos / C::KS, x = pos % C::KS;
    return r | (((x & ~(S - 1)) | ((x ^ stage_xor_pf<S>(r)) & (S - 1))) << 8);
  };
  // pieces past the call's head dim load a piece of the same row (finite values: they meet q
  // zeros in QK and fill output columns that are not stored)
  auto clamp_piece = [&](int pk, int cpr) -> int __attribute__((always_inline)) {
    const int cc = pk >> 8;
    return cc < cpr ? pk : (pk & 255) | ((cc % cpr) << 8);
  };
  const int kcpr = p.dk / 8, vcpr = p.dv / 8;
  int kpk[C::KLD];
#pragma unroll
  for (int u = 0; u < C::KLD; ++u) {
    const int pos = u * C::GT + gt;
    if constexpr (C::PF) kpk[u] = pos < C::KPOS ? pack_pos_pf(pos) : 0;
    else kpk[u] = pos < C::KPOS ? pack_pos(pos, C::KS, C::KCPR) : 0;
    if (C::KCPR != kcpr) kpk[u] = clamp_piece(kpk[u], kcpr);
  }
  int vpk[C::VLD > 0 ? C::VLD : 1];
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int pos = u * C::GT + gt;
    vpk[u] = pos < C::VPOS ? pack_pos(pos, C::VS, C::VCPR) : 0;
    if (C::VCPR != vcpr) vpk[u] = clamp_piece(vpk[u], vcpr);
  }
  // round u of this wave lies inside the chunk (compile-time true for all but the last round)
  const int gw = C::LW > 0 ? wave_u - C::NCW : wave_u;  // gathering wave index (when gwave)
  auto round_in = [&](int u, int npos) -> bool __attribute__((always_inline)) {
    if (u * C::GT + C::GT <= npos) return true;
    return u * C::GT + gw * 64 < npos;
  };
  // Gather of chunk c in NR rounds (K rounds, then V rounds); read_rows fetches the row
  // indices of all rounds first (one batch of LDS reads), issue_round(c, r) issues one load.
  constexpr int NR = C::KLD + (ALIAS ? 0 : C::VLD);
  int jrow[NR];
  auto read_rows = [&](int c) __attribute__((always_inline)) {
    const int* irow = idxl + c * C::CH;
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) jrow[u] = irow[kpk[u] & 255];
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < C::VLD; ++u) jrow[C::KLD + u] = irow[vpk[u] & 255];
    }
  };
  // mask words of chunk c into its slot of the mask ring (wave 0; vmcnt waits stay lower
  // bounds since the other waves issue fewer loads)
  const uint32_t mw_base = smem_lds + C::LDS_FIXED + ((p.split_len * 4 + 15) & ~15);
  auto issue_mask_words = [&](int c) __attribute__((always_inline)) {
    if (p.bm_words && gwave && gw == 0) {
#pragma unroll
      for (int j = 0; j < WS; ++j) {
        const int w = min(bm_w0 + (c * C::CH) / 32 + j, bm_wend - 1);
        for (int i0 = 0; i0 < bm_nrows; i0 += 64) {
          const int i = min(i0 + lane, bm_nrows - 1);
          lds_dma4(p.bm_words + (int64_t)w * p.RS + bm_row0 + i,
                   mw_base + (((c % NBUF) * WS + j) * C::MW + i0) * 4);
        }
      }
    }
  };
  auto issue_round = [&](int c, int r) __attribute__((always_inline)) {
    const uint32_t kb_lds = smem_lds + (c % NBUF) * C::BUF;
    if (r < C::KLD) {
      const int u = r;
      if (round_in(u, C::KPOS))
        lds_dma16_at(kg_ptr, __umul24((uint32_t)clamp_row(jrow[r]), krow_bytes) + ((uint32_t)kpk[u] >> 8) * 16u,
                     kb_lds + (u * C::GT + gw * 64) * 16);
    } else if constexpr (!ALIAS) {
      const int u = r - C::KLD;
      if (round_in(u, C::VPOS))
        lds_dma16_at(vg_ptr, __umul24((uint32_t)clamp_row(jrow[r]), vrow_bytes) + ((uint32_t)vpk[u] >> 8) * 16u,
                     kb_lds + C::KBUF + (u * C::GT + gw * 64) * 16);
    }
  };
  auto issue_gather = [&](int c) __attribute__((always_inline)) {
    if (!gwave) return;
    issue_mask_words(c);
    read_rows(c);
#pragma unroll
    for (int r = 0; r < NR; ++r) issue_round(c, r);
  };

  // Per-lane LDS byte offsets of the MFMA operands; every k-step / tile / dv tile adds a
  // compile-time offset (the XOR of the staged layout only touches lane-dependent bits).
  //  K operand, tile t, k-step ks: row sb + MT*t + col, chunk (KSTEP/8)*ks + kg
  //  V^T operand, PV k-step j, half hh, dv tile dt: rows acc_row(8j + 4hh) + (c16 >> 2),
  //  columns MT*dt + 16*(q16 % (MT/16)) + 4*(c16 & 3)
  const int sb0 = wsl * 32;  // this wave's 32 slots inside a chunk
  // pad-free rows: the XOR covers log2(S) chunk bits, so k-steps (4 chunks each) cycle through
  // S / 4 lane offsets and dv tiles (2 chunks each) through S / 2
  constexpr int PFS = C::PF ? C::PF : 8;
  int lane_k[C::PF ? PFS / 4 : 2], lane_v[C::PF ? PFS / 2 : 2];
  if constexpr (C::PF) {
    const int r = sb0 + col;
#pragma unroll
    for (int q = 0; q < PFS / 4; ++q) lane_k[q] = (r * C::KS + ((4 * q + kg) ^ stage_xor_pf<PFS>(r))) * 16;
    const int rv = sb0 + 4 * q16 + (c16 >> 2);
#pragma unroll
    for (int q = 0; q < PFS / 2; ++q)
      lane_v[q] = (rv * C::KS + ((2 * q + ((c16 & 3) >> 1)) ^ stage_xor_pf<PFS>(rv))) * 16 + 8 * (c16 & 1);
  } else if constexpr (MN == 16) {
    const int r = sb0 + col;
    lane_k[0] = lane_k[1] = (r * C::KS + (kg ^ stage_xor(r))) * 16;
    const int rv = sb0 + 4 * q16 + (c16 >> 2);
#pragma unroll
    for (int par = 0; par < 2; ++par)  // dv-tile parity
      lane_v[par] = (rv * C::VS + ((2 * par + ((c16 & 3) >> 1)) ^ stage_xor(rv))) * 16 + 8 * (c16 & 1);
  } else {
    const int r = sb0 + col;
#pragma unroll
    for (int par = 0; par < 2; ++par)  // k-step parity
      lane_k[par] = (r * C::KS + ((2 * par + kg) ^ stage_xor(r))) * 16;
    const int r0 = sb0 + 4 * (q16 >> 1) + (c16 >> 2);
    const int lo = 2 * (q16 & 1) + ((c16 & 3) >> 1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      lane_v[hh] = ((r0 + 8 * hh) * C::VS + (lo ^ (((r0 >> 1) & 2) | hh))) * 16 + 8 * (c16 & 1);
  }
  auto k_off = [&](int t, int ks) -> int __attribute__((always_inline)) {
    if constexpr (C::PF) return lane_k[ks % (PFS / 4)] + t * 16 * C::KS * 16 + PFS * 16 * (ks / (PFS / 4));
    else if constexpr (MN == 16) return lane_k[0] + t * 16 * C::KS * 16 + 64 * ks;
    else return lane_k[ks & 1] + 64 * (ks >> 1);
  };
  auto v_off = [&](int dt, int j, int hh) -> int __attribute__((always_inline)) {
    if constexpr (C::PF) return lane_v[dt % (PFS / 2)] + hh * 16 * C::KS * 16 + PFS * 16 * (dt / (PFS / 2));
    else if constexpr (MN == 16) return lane_v[dt & 1] + hh * 16 * C::VS * 16 + 64 * (dt >> 1);
    else return lane_v[hh] + j * 16 * C::VS * 16 + 64 * dt;
  };

  // ---- running state (per lane: head column `col`; O^T rows dv = MT*dt + acc_row(E))
  acc_t acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int e = 0; e < NACC; ++e) acc[dt][e] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // wait until every load of the chunk `ahead` chunks before the newest issued one has
  // landed (each wave counts its own loads), then join the workgroup barrier
  auto wait_chunk = [&](int ahead) __attribute__((always_inline)) {
    switch (ahead) {
#define SFA_WAIT_CASE(k) \
  case k:                \
    if constexpr (k <= NBUF - 2) wait_vm_barrier<k * C::CNT>(); \
    break;
      SFA_WAIT_CASE(0)
      SFA_WAIT_CASE(1)
      SFA_WAIT_CASE(2)
      SFA_WAIT_CASE(3)
      SFA_WAIT_CASE(4)
      SFA_WAIT_CASE(5)
      SFA_WAIT_CASE(6)
#undef SFA_WAIT_CASE
      default:
        wait_vm_barrier<0>();
    }
  };

  // S^T = K Q^T of chunk c: NST tiles of MT slots.  Two accumulation chains per tile (even /
  // odd k-steps) keep dependent MFMAs apart; the operands of a group of k-steps are read
  // from LDS together, ahead of their MFMAs.
  auto qk = [&](int c, acc_t (&s)[C::NST]) {
    const char* kb = smem + (c % NBUF) * C::BUF;
    if constexpr (PK) {
      // one tile, 2 x KSTEPS k-steps: step v multiplies the K rows of slot group v / KSTEPS
      // (the rows of unpacked tile v / KSTEPS) by that group's copy of Q^T
      acc_t sp[2];
#pragma unroll
      for (int e = 0; e < NACC; ++e) sp[0][e] = sp[1][e] = 0.f;
      constexpr int NV = 2 * C::KSTEPS, KG = 4;
#pragma unroll
      for (int v0 = 0; v0 < NV; v0 += KG) {
        u32x4 a[KG];
#pragma unroll
        for (int g = 0; g < KG; ++g)
          if (v0 + g < NV) a[g] = *(const u32x4*)(kb + k_off((v0 + g) / C::KSTEPS, (v0 + g) % C::KSTEPS));
#pragma unroll
        for (int g = 0; g < KG; ++g)
          if (v0 + g < NV) sp[g % 2] = TL::mfma(as<vec8>(a[g]), as<vec8>(qreg[v0 + g]), sp[g % 2]);
      }
      s[0] = sp[0] + sp[1];
      return;
    }
    acc_t s2[C::NST][2];
#pragma unroll
    for (int t = 0; t < C::NST; ++t)
#pragma unroll
      for (int e = 0; e < NACC; ++e) s2[t][0][e] = s2[t][1][e] = 0.f;
    constexpr int KG = 4;
#pragma unroll
    for (int k0 = 0; k0 < C::KSTEPS; k0 += KG) {
      u32x4 a[KG][C::NST], bq[KG];
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        const int ks = k0 + g;
        if (ks < C::KSTEPS) {
#pragma unroll
          for (int t = 0; t < C::NST; ++t) a[g][t] = *(const u32x4*)(kb + k_off(t, ks));
          if (ks < C::QREG) bq[g] = qreg[ks < C::QREG ? ks : 0];
          else bq[g] = *(const u32x4*)(qlds + ((wh * (C::KSTEPS - C::QREG) + ks - C::QREG) * 64 + lane) * 16);
        }
      }
#pragma unroll
      for (int g = 0; g < KG; ++g) {
        if (k0 + g < C::KSTEPS) {
#pragma unroll
          for (int t = 0; t < C::NST; ++t) {
            // two waves per SIMD hide the MFMA latency: one chain is enough
            constexpr int NCH = C::NCW >= 8 ? 1 : 2;
            s2[t][g % NCH] = TL::mfma(as<vec8>(a[g][t]), as<vec8>(bq[g]), s2[t][g % NCH]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < C::NST; ++t) {
      if constexpr (C::NCW >= 8) s[t] = s2[t][0];
      else s[t] = s2[t][0] + s2[t][1];
    }
  };

  // Online softmax of chunk c with scores s in three stages, so that the deep pipeline below can
  // put the MFMAs of other chunks in one block with the exponentials:
  //  sm_max  -- mask (in place), chunk max, whether the reference max moves and the max to use;
  //  sm_exp  -- probabilities and their sum, then sm_split -- the P^T operands of the PV product
  //             (neither branches);
  //  sm_fold -- rescale O^T and the running sum when the reference moved, add this chunk's sum.
  constexpr int NE = C::NST * NACC;  // elements per lane: 8 (MT 16), 16 (MT 32) or 4 (packed)
  auto sm_max = [&](int c, acc_t (&s)[C::NST], float& cmax, bool& bump, float& m_use) __attribute__((always_inline)) {
    const int sb = wsl * 32;  // this wave's 32 slots inside the chunk
    // mask and chunk max of the raw scores (scale > 0 is applied inside the exponent).
    // Element E of tile t is slot MN*t + acc_row(E); of a packed tile, 16*grp + acc_row(E).
    const int sg = PK ? 16 * grp : 0;
    // masked elements become -inf in place (the scores are dead after this chunk)
    if (__builtin_amdgcn_readfirstlane(cflag[c])) {
      // 32-wide tiles (16 elements per lane) test the block-sparse mask word only when there is
      // one; 16-wide tiles keep one path (fewer registers)
      if (MN == 16 || p.bm_words) {
        // element mask word of this lane's query row (all ones without a mask)
        uint32_t mword = 0xffffffffu;
        if (p.bm_words) {
          const int lr = min(max(head / p.HR - bm_row0, 0), bm_nrows - 1);
          mword = *(const uint32_t*)(smem + (mw_base - smem_lds) + (((c % NBUF) * WS + wsl) * C::MW + lr) * 4);
        }
#pragma unroll
        for (int t = 0; t < C::NST; ++t) {
#pragma unroll
          for (int e4 = 0; e4 < NACC / 4; ++e4) {
            const int sl = sg + MN * t + acc_row<MN>(4 * e4, kg);  // slot of element 4 e4 in the wave's 32
            const u32x4 jj = *(const u32x4*)(idxl + c * C::CH + sb + sl);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[t][4 * e4 + e] =
                  (selects((int)jj[e]) && ((mword >> (sl + e)) & 1u)) ? s[t][4 * e4 + e] : -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < C::NST; ++t) {
#pragma unroll
          for (int e4 = 0; e4 < NACC / 4; ++e4) {
            const int sl = sg + MN * t + acc_row<MN>(4 * e4, kg);
            const u32x4 jj = *(const u32x4*)(idxl + c * C::CH + sb + sl);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[t][4 * e4 + e] = selects((int)jj[e]) ? s[t][4 * e4 + e] : -INFINITY;
          }
        }
      }
    }
    cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NE; ++i) cmax = fmaxf(cmax, s[i / NACC][i % NACC]);
    cmax = wave_max_lanes<MT>(cmax) * sl2;
    // the reference max moves only when this chunk exceeds it by more than kLazyRescale
    bump = cmax > m_run + kLazyRescale;
    const float m_new = bump ? cmax : m_run;
    m_use = m_new == -INFINITY ? 0.f : m_new;
  };
  auto sm_exp = [&](const acc_t (&s)[C::NST], float m_use, float (&pv)[NE]) __attribute__((always_inline)) -> float {
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      pv[i] = fast_exp2(__builtin_fmaf(s[i / NACC][i % NACC], sl2, -m_use));
      psum += pv[i];
    }
    return psum;
  };
  // P^T operands of the probabilities pv: k-step j takes elements 8j..8j+7 (MFMA k index 8*kg + e)
  auto sm_split = [&](const float (&pv)[NE], u32x4 (&phi)[C::PVK], u32x4 (&plo)[C::PVK]) __attribute__((always_inline)) {
    if constexpr (PK) {
      // A lane holds P of its head over 4 slots of its group; MFMA k index 8*kg + e is slot
      // 4*kg + e for e < 4 (group 0) and 16 + 4*kg + e - 4 for e >= 4 (group 1).  Both columns of
      // a head take the P of both groups (the partner column's values by a row_ror:8 DPP move),
      // so columns c and c + 8 of O^T each accumulate head c over all 32 slots.
      uint32_t h01, l01, h23, l23;
      split2<T>(pv[0], pv[1], h01, l01);
      split2<T>(pv[2], pv[3], h23, l23);
      phi[0] = u32x4{ror8_into<0xC>(h01), ror8_into<0xC>(h23), ror8_into<0x3>(h01), ror8_into<0x3>(h23)};
      plo[0] = u32x4{ror8_into<0xC>(l01), ror8_into<0xC>(l23), ror8_into<0x3>(l01), ror8_into<0x3>(l23)};
    } else {
#pragma unroll
      for (int j = 0; j < C::PVK; ++j) split_hi_lo<T>(pv + 8 * j, phi[j], plo[j]);
    }
  };
  auto sm_fold = [&](float cmax, bool bump, float psum) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(bump)) {
      // lanes that do not move keep alpha = 1 (their m_run may still be -inf: the heads of a
      // wave can have different masks); a moving lane with nothing seen yet gets alpha = 0
      const float alpha = bump ? fast_exp2(m_run - cmax) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) scale_acc<NACC>(acc[dt], alpha);
    }
    if (bump) m_run = cmax;
    l_run += psum;
  };
  // The three stages in order: mask and online softmax of chunk c, and its P^T operands.
  auto softmax_p = [&](int c, acc_t (&s)[C::NST], u32x4 (&phi)[C::PVK], u32x4 (&plo)[C::PVK]) __attribute__((always_inline)) {
    float cmax, m_use, pv[NE];
    bool bump;
    sm_max(c, s, cmax, bump, m_use);
    sm_fold(cmax, bump, sm_exp(s, m_use, pv));
    sm_split(pv, phi, plo);
  };

  // O^T += V^T P^T for chunk c.  The V^T operand of k-step j, dv tile dt: lane (dv row, k-group
  // kg) needs the 8 slots of elements 8j..8j+7, read as two transposed 4-slot halves.  The
  // gather of chunk `gc` (-1: none; its row indices already read) is issued round by round
  // between the MFMAs, where the VALU is otherwise idle.
  auto pv_product = [&](int c, const u32x4 (&phi)[C::PVK], const u32x4 (&plo)[C::PVK], int gc) {
    const char* kb = smem + (c % NBUF) * C::BUF;
    const char* vb = ALIAS ? kb : kb + C::KBUF;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      if (gc >= 0) {
#pragma unroll
        for (int r = dt * NR / C::DT; r < (dt + 1) * NR / C::DT; ++r) issue_round(gc, r);
      }
#pragma unroll
      for (int j = 0; j < C::PVK; ++j) {
        u32x2 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) h[hh] = lds_read_tr16(vb + v_off(dt, j, hh));
        const u32x4 a = {h[0][0], h[0][1], h[1][0], h[1][1]};
        acc[dt] = TL::mfma(as<vec8>(a), as<vec8>(phi[j]), acc[dt]);
        acc[dt] = TL::mfma(as<vec8>(a), as<vec8>(plo[j]), acc[dt]);
      }
    }
  };

  // Mask, online softmax and O^T += V^T P^T for chunk c with scores s.  The gather of chunk
  // `gc` (-1: none) goes out during the product; its row indices are read from LDS up front.
  auto softmax_pv = [&](int c, acc_t (&s)[C::NST], int gc) {
    if (gc >= 0) {
      issue_mask_words(gc);
      read_rows(gc);
    }
    u32x4 phi[C::PVK], plo[C::PVK];
    softmax_p(c, s, phi, plo);
    pv_product(c, phi, plo, gc);
  };

  // Block-sparse words of this split with a clear bit flag their chunks too.  Read before the
  // first gathers are issued: a wait the compiler puts on these loads would otherwise also wait
  // for the gathers in flight.
  if (p.bm_words) {
    for (int w = tid; w < (nslots + 31) / 32; w += C::NT)
      if (p.bm_wflag[bm_w0 + w]) cflag[w * 32 / C::CH] = 1;
  }
  // Deep software pipeline for rings of 5+ buffers without loader waves (below), where its
  // second set of P^T operands costs no residency: Dk >= 128 (the 64-wide kernels would drop
  // from three waves per SIMD to two) and Dv <= 128 (wider accumulators leave no room).
  constexpr bool DEEP = NBUF >= 5 && C::LW == 0 && DK >= 128 && DV <= 128;
  // prologue: the first NBUF - 1 chunks in flight (NBUF - 2 with the deep pipeline)
  constexpr int NPRO = DEEP ? NBUF - 2 : NBUF - 1;
#pragma unroll
  for (int i = 0; i < NPRO; ++i)
    if (i < nchunks) issue_gather(i);
  // Flag the chunks where some slot is masked for some query of this workgroup (an index out
  // of range, past the causal limit of the workgroup's first query row, or a pad); the other
  // chunks skip the per-element mask.  Done while the first chunks are in flight; the flags
  // are published by the first ring barrier.
  {
    const int h0 = hb * MT * WH;
    const uint32_t jend_lo =
        (uint32_t)(p.causal ? max(0, min(p.S2, item_row0(p, s1) + h0 / p.HR + (p.S2 - p.QROWS) + 1)) : p.S2);
    for (int i = tid; i < nslots; i += C::NT)
      if (!((uint32_t)idxl[i] < jend_lo)) cflag[i / C::CH] = 1;
    if (tid == 0 && nslots % C::CH != 0) cflag[nslots / C::CH] = 1;
  }

  if constexpr (DEEP) {
    // Deep software pipeline: a wave hides its own VALU work under its own MFMAs (the two waves
    // of a SIMD do not overlap each other's), so step c puts in one block, with no branch, the
    // QK MFMAs of chunk c + 1, the PV MFMAs of chunk c - 1 and the exponentials of chunk c; the
    // mask and chunk max come before it, the rescale after.  The PV product of a chunk runs one
    // step after its softmax, so its V rows are read until the barrier after next: barrier k
    // (k >= 1: chunk k has landed) sends chunk k + NBUF - 3 into the buffer of chunk k - 3,
    // whose last reader (the PV product of chunk k - 3) ran before barrier k - 1... and the
    // step after; one chunk fewer is in flight.  The last step scores a stale buffer (unused).
    auto ring_step = [&](int k) __attribute__((always_inline)) {
      // chunks 0 .. k + NBUF - 4 are issued: chunk k has landed once the newer ones are all
      // that may be outstanding
      wait_chunk(min(NBUF - 4, nchunks - 1 - k));
      if (k + NBUF - 3 < nchunks) issue_gather(k + NBUF - 3);
    };
    acc_t s_a[C::NST], s_b[C::NST];
    u32x4 phi[C::PVK], plo[C::PVK];  // P^T operands of the chunk whose PV product is pending
    auto step = [&](int c, acc_t (&s_cur)[C::NST], acc_t (&s_nxt)[C::NST], bool with_pv) __attribute__((always_inline)) {
      if (c + 1 < nchunks) ring_step(c + 1);
      float cmax, m_use;
      bool bump;
      sm_max(c, s_cur, cmax, bump, m_use);
      u32x4 phn[C::PVK], pln[C::PVK];
      float pv[NE];
      qk(c + 1, s_nxt);
      if (with_pv) pv_product(c - 1, phi, plo, -1);
      const float psum = sm_exp(s_cur, m_use, pv);
      sm_split(pv, phn, pln);
      sm_fold(cmax, bump, psum);
#pragma unroll
      for (int j = 0; j < C::PVK; ++j) {
        phi[j] = phn[j];
        plo[j] = pln[j];
      }
    };
    if (nchunks > 0) {
      wait_chunk(min(NBUF - 3, nchunks - 1));
      qk(0, s_a);
      step(0, s_a, s_b, false);
      int c = 1;
      for (; c + 1 < nchunks; c += 2) {
        step(c, s_b, s_a, true);
        step(c + 1, s_a, s_b, true);
      }
      if (c < nchunks) step(c, s_b, s_a, true);
      pv_product(nchunks - 1, phi, plo, -1);
    }
  } else if constexpr (NBUF >= 4) {
    // Software pipeline: the scores of chunk c + 1 are computed (MFMA) next to the softmax
    // of chunk c (VALU), whose PV follows.  Chunk c + NBUF - 1 is loaded into the buffer of
    // chunk c - 1, free once every wave passed the barrier of step c.  (It keeps one chunk
    // less in flight, so shallow rings -- the memory-bound decode shapes -- do without it.)
    // Two steps per iteration, so that the score registers of chunks c and c + 1 swap roles
    // instead of being copied.
    acc_t s_a[C::NST], s_b[C::NST];
    if (nchunks > 0) {
      wait_chunk(min(NBUF - 2, nchunks - 1));
      if (!loader) qk(0, s_a);
    }
    auto step = [&](int c, acc_t (&s_cur)[C::NST], acc_t (&s_nxt)[C::NST]) {
      if (c + 1 < nchunks) {
        // chunks 0 .. c + NBUF - 2 are issued; chunk c + 1 has landed once the ones after it
        // are all that may be outstanding
        wait_chunk(min(NBUF - 3, nchunks - 2 - c));
        if (c + NBUF - 1 < nchunks) issue_gather(c + NBUF - 1);
        if (!loader) qk(c + 1, s_nxt);
      }
      if (!loader) softmax_pv(c, s_cur, -1);
    };
    for (int c = 0; c < nchunks; c += 2) {
      step(c, s_a, s_b);
      if (c + 1 < nchunks) step(c + 1, s_b, s_a);
    }
  } else {
    acc_t s_cur[C::NST];
    // buffer (c + NBUF - 1) % NBUF held chunk c - 1, which every wave finished before the
    // barrier of step c
    if (C::LW > 0 && loader) {
      // loader waves: the ring waits and the gathers only, in a loop of their own so that the
      // compute waves' loop holds none of the gather tables in registers
      for (int c = 0; c < nchunks; ++c) {
        wait_chunk(min(NBUF - 2, nchunks - 1 - c));
        const int gc = c + NBUF - 1 < nchunks ? c + NBUF - 1 : -1;
        if (gc >= 0) issue_gather(gc);
      }
    } else {
      for (int c = 0; c < nchunks; ++c) {
        wait_chunk(min(NBUF - 2, nchunks - 1 - c));
        // Without loader waves: with two buffers the next chunk is needed right after this one
        // (issue it now); with more, its gather goes out during this chunk's PV.
        const int gc = c + NBUF - 1 < nchunks ? c + NBUF - 1 : -1;
        if (C::LW == 0 && NBUF == 2 && gc >= 0) issue_gather(gc);
        qk(c, s_cur);
        softmax_pv(c, s_cur, (NBUF == 2 || C::LW > 0) ? -1 : gc);
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before the epilogue reuses LDS
  if constexpr (HF) {
    if (p.fv) {
      const float f = p.fv[kvh];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) scale_acc<NACC>(acc[dt], f);
    }
  }

  // ---- epilogue
  const float l_tot = wave_sum_lanes<MT>(l_run);
  const int64_t row = ws_row(p, b, s1, n2, hv);

  if constexpr (WS == 1) {
    if (loader) {
      // loader waves hold no output
    } else if (direct) {
      if (head_ok && grp == 0) {  // packed tiles: columns c and c + 8 hold the same head
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* orow = p.out + qv_offset(p, p.os, b, s1, n2, hv);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
          for (int e4 = 0; e4 < NACC / 4; ++e4) {
            if (dt * MN + acc_row<MN>(4 * e4, kg) >= p.dv) continue;
            u32x2 w;
            w[0] = (uint32_t)T::from_float(acc[dt][4 * e4] * inv) |
                   ((uint32_t)T::from_float(acc[dt][4 * e4 + 1] * inv) << 16);
            w[1] = (uint32_t)T::from_float(acc[dt][4 * e4 + 2] * inv) |
                   ((uint32_t)T::from_float(acc[dt][4 * e4 + 3] * inv) << 16);
            *(u32x2*)(orow + dt * MN + acc_row<MN>(4 * e4, kg)) = w;
          }
        }
        if (p.lse && kg == 0)
          p.lse[qv_offset(p, p.ls, b, s1, n2, hv)] =
              l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
      }
    } else {
      if (head_ok && grp == 0) {  // packed tiles: columns c and c + 8 hold the same head
        float* po = p.ws_o + (row * p.nsplit + split) * DV;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int e4 = 0; e4 < NACC / 4; ++e4)
            *(f32x4*)(po + dt * MN + acc_row<MN>(4 * e4, kg)) =
                f32x4{acc[dt][4 * e4], acc[dt][4 * e4 + 1], acc[dt][4 * e4 + 2], acc[dt][4 * e4 + 3]};
        if (kg == 0) {
          float* pm = p.ws_ml + (row * p.nsplit + split) * 2;
          pm[0] = m_run;
          pm[1] = l_tot;
        }
      }
    }
  } else {
    // merge the WS slot parts of each head tile through LDS
    constexpr int MOS = topk_merge_stride(DV);
    float* mo = (float*)smem;               // [WS][WH][MT][MOS]
    float* mml = mo + WS * WH * MT * MOS;   // [WS][WH][MT][2]
    // every wave finished its last chunk (barrier after the loop)
    if (!loader && grp == 0) {
      float* o = mo + ((wsl * WH + wh) * MT + hcol) * MOS;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < NACC / 4; ++e4)
          *(f32x4*)(o + dt * MN + acc_row<MN>(4 * e4, kg)) =
              f32x4{acc[dt][4 * e4], acc[dt][4 * e4 + 1], acc[dt][4 * e4 + 2], acc[dt][4 * e4 + 3]};
      if (kg == 0) {
        float* ml = mml + ((wsl * WH + wh) * MT + hcol) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    __syncthreads();
    // thread -> (head tile, head, 4 dv values)
    constexpr int PER_ROW = DV / 4;
    for (int w = tid; w < WH * MT * PER_ROW; w += C::NT) {
      const int hrow = w / PER_ROW;  // wh*MT + head column
      const int d4 = w % PER_ROW;
      const int hh = hb * MT * WH + hrow;
      if (!item_has(p, s1, hh)) continue;
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < WS; ++q) M = fmaxf(M, mml[(q * WH * MT + hrow) * 2]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float L = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < WS; ++q) {
        const float wq = fast_exp2(mml[(q * WH * MT + hrow) * 2] - Mu);
        L += mml[(q * WH * MT + hrow) * 2 + 1] * wq;
        o += *(const f32x4*)(mo + (q * WH * MT + hrow) * MOS + 4 * d4) * wq;
      }
      const int64_t rr = ws_row(p, b, s1, n2, hh);
      if (direct) {
        if (4 * d4 >= p.dv) continue;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t* orow = p.out + qv_offset(p, p.os, b, s1, n2, hh);
        u32x2 wv;
        wv[0] = (uint32_t)T::from_float(o[0] * inv) | ((uint32_t)T::from_float(o[1] * inv) << 16);
        wv[1] = (uint32_t)T::from_float(o[2] * inv) | ((uint32_t)T::from_float(o[3] * inv) << 16);
        *(u32x2*)(orow + 4 * d4) = wv;
        if (p.lse && d4 == 0)
          p.lse[qv_offset(p, p.ls, b, s1, n2, hh)] =
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
// lse = -inf.  One thread per 8 output values (one 16-byte store; with 4 the MLA merge needed
// a second, 1/7-full round of workgroups); the loads of U splits are in flight together.
template <typename T, int DV>
__global__ __launch_bounds__(256) void topk_merge(TopkParams p, int64_t nrows) {
  constexpr int PER_ROW = DV / 8;  // threads per row, 8 output values each
  constexpr int U = 4;             // splits whose loads are in flight together
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = w / PER_ROW;
  const int d8 = (int)(w % PER_ROW);
  if (row >= nrows) return;
  // row = ((b * S1 + s1) * N2 + n2) * G + h
  const int h = (int)(row % p.G);
  const int64_t r2 = row / p.G;
  const int n2 = (int)(r2 % p.N2);
  const int s1 = (int)((r2 / p.N2) % p.S1);
  const int b = (int)(r2 / ((int64_t)p.N2 * p.S1));
  if (!item_has(p, s1, h)) return;  // no such query (partial block row)
  int n_all = p.topK;
  if (p.slot_ptr) {
    const int list = item_list(p, s1);
    n_all = p.slot_ptr[list + 1] - p.slot_ptr[list];
  }
  const int nsp = item_split_count(p, item_slots(p, s1, n_all));
  if (nsp == 1) return;  // its single split wrote the output
  const float* ml = p.ws_ml + row * p.nsplit * 2;
  const float* po = p.ws_o + row * p.nsplit * DV + 8 * d8;
  // one pass: the loads of U splits are issued together, then folded into a running
  // (M, L, o) with the log-sum-exp rule
  float M = -INFINITY, L = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nsp; j0 += U) {
    float m[U], l[U];
    f32x4 v0[U], v1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      const bool in = j < nsp;
      m[u] = in ? ml[2 * j] : -INFINITY;
      l[u] = in ? ml[2 * j + 1] : 0.f;
      v0[u] = in ? *(const f32x4*)(po + (int64_t)j * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
      v1[u] = in ? *(const f32x4*)(po + (int64_t)j * DV + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u) Mn = fmaxf(Mn, m[u]);
    if (Mn == -INFINITY) continue;  // nothing seen yet
    const float sc = fast_exp2(M - Mn);  // 0 while M == -inf
    L *= sc;
    o0 *= sc;
    o1 *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wj = fast_exp2(m[u] - Mn);  // 0 for an empty split (m = -inf)
      L += l[u] * wj;
      o0 += v0[u] * wj;
      o1 += v1[u] * wj;
    }
    M = Mn;
  }
  if (p.lse && d8 == 0)
    p.lse[qv_offset(p, p.ls, b, s1, n2, h)] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
  if (8 * d8 >= p.dv) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = p.out + qv_offset(p, p.os, b, s1, n2, h);
  const float y[8] = {o0[0] * inv, o0[1] * inv, o0[2] * inv, o0[3] * inv,
                      o1[0] * inv, o1[1] * inv, o1[2] * inv, o1[3] * inv};
  *(u32x4*)(orow + 8 * d8) = pack8<T>(y);
}

}  // namespace sfa
