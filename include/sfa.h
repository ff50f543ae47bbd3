/*
 * sfa.h -- C ABI of the MI355X (gfx950) sparse flash attention library (libsfa.so).
 *
 * Two operators, both asynchronous on the caller's HIP stream, both reading and
 * writing only caller-owned device memory (the library never allocates device
 * memory on a run call):
 *
 *  1. Top-K sparse attention -- "SparseFlashAttention operator API description",
 *     section 2 (definition) and section 3 (interface, rules, support ranges):
 *         K_sel = gather(K, sparseIndices), V_sel = gather(V, sparseIndices)
 *         y = softmax(Q K_sel^T * scale [+ causal mask]) V_sel
 *     Every query row (b, s1, n1) attends to the topK key/value rows listed in
 *     sparseIndices[b, s1, n2, :] (BSND) or [b, n2, s1, :] (BNSD) with
 *     n2 = n1 / (N1 / N2) (grouped-query attention: the N1/N2 query heads of one
 *     KV head share its index row).  With causal != 0 a slot whose index exceeds
 *     s1 + (S2 - S1) is masked (bottom-right aligned causal mask); a row whose
 *     slots are all masked outputs zeros.
 *
 *  2. Block-sparse (BSR) attention -- "flashinfer.sparse", class
 *     BlockSparseAttentionWrapper (plan / run): attention of q [M, Hq, D] over
 *     k, v [N, Hkv, D] under the boolean mask of a BSR matrix with R x C blocks
 *     (SciPy bsr_matrix: indptr over MB = ceil(M / R) block rows, indices of
 *     column blocks, NB = N / C).  plan() validates and stages the pattern once;
 *     run() may then be called any number of times.
 *
 *  3. Variable block-sparse attention -- "flashinfer.sparse", class
 *     VariableBlockSparseAttentionWrapper (plan / run): every KV head has its own
 *     MB x NB block grid, with block row sizes block_row_sz[h] and column sizes
 *     block_col_sz[h], and its own boolean block_mask_map[h]; the query heads of a
 *     KV head share its pattern.  q [Hq, M, D], k, v [Hkv, N, D] (HND).
 *
 * Conventions
 *  - Element dtypes: query, key, value and output share one dtype, fp16 or bf16;
 *    indices are int32; LSE is fp32.  The block-sparse calls also take FP8 (E4M3 /
 *    E5M2) q, k, v with per-head factors (bsr_run_fp8, vbsr_run_fp8; fp16 output).
 *  - A status code is returned by every call; SFA_OK is 0.  No call aborts.
 *  - Reentrant: no global mutable state besides the per-device kernel attributes
 *    set at first use.  Calls on one stream execute in order.
 */
#ifndef SFA_H_
#define SFA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sfa_status {
  SFA_OK = 0,
  SFA_ERR_NULL = 1,        /* a required pointer is NULL */
  SFA_ERR_DTYPE = 2,       /* dtype not fp16/bf16 */
  SFA_ERR_LAYOUT = 3,      /* layout not BSND/BNSD, or a tensor's last dim is not contiguous */
  SFA_ERR_SHAPE = 4,       /* a negative or inconsistent size (S2 < 1, N1 < 1, N2 < 1 ...) */
  SFA_ERR_GQA = 5,         /* N1 % N2 != 0 (or Hq % Hkv != 0) */
  SFA_ERR_HEAD_DIM = 6,    /* Dk or Dv not a positive multiple of 64, or Dv > Dk */
  SFA_ERR_TOPK = 7,        /* topK outside [1, S2] */
  SFA_ERR_CAUSAL = 8,      /* causal with S1 > S2 (M > N for BSR) */
  SFA_ERR_SCALE = 9,       /* scale not finite or not > 0 */
  SFA_ERR_WORKSPACE = 10,  /* workspace missing or smaller than required */
  SFA_ERR_PLAN = 11,       /* BSR plan missing or malformed pattern */
  SFA_ERR_INDEX = 12,      /* a BSR column block out of range or repeated in a row */
  SFA_ERR_UNSUPPORTED = 13,/* a head dim above 576, or a size beyond the kernels' addressing */
  SFA_ERR_HIP = 14         /* a HIP runtime call failed (no device, launch failure ...) */
} sfa_status;

typedef enum sfa_dtype { SFA_FP16 = 0, SFA_BF16 = 1 } sfa_dtype;

typedef enum sfa_layout { SFA_BSND = 0, SFA_BNSD = 1 } sfa_layout;

/* Layout of k / v in the dense prefill call: NHD [kv_len, heads, D] or HND [heads, kv_len, D]. */
typedef enum sfa_kv_layout { SFA_NHD = 0, SFA_HND = 1 } sfa_kv_layout;

/* 8-bit float encodings of the FP8 inputs of bsr_run_fp8 / vbsr_run_fp8 (OCP 8-bit
 * floating point formats): E4M3 (exponent bias 7, no infinities, S.1111.111 = NaN) and
 * E5M2 (exponent bias 15, exponent field 31 = infinity / NaN). */
typedef enum sfa_fp8 { SFA_FP8_E4M3 = 0, SFA_FP8_E5M2 = 1 } sfa_fp8;

/* Problem sizes of the top-K operator (SparseFlashAttention page, section 3):
 * B batch, S1 query length, S2 key/value length, N1 query heads, N2 KV heads,
 * Dk query/key head dim, Dv value head dim, topK selected slots per row. */
typedef struct sfa_shape {
  int32_t B, S1, S2, N1, N2, Dk, Dv, topK;
} sfa_shape;

/* Element strides of the three outer dims of each tensor, in the layout's own
 * dim order (BSND: batch, seq, head; BNSD: batch, head, seq).  The last dim of
 * every tensor must be contiguous.  Passing NULL for the whole struct means all
 * tensors are contiguous in the layout.  Strides let value be the prefix view
 * key[..., :Dv] (the MLA latent-cache case: value and key then share storage and
 * the library gathers each row once for both). */
typedef struct sfa_strides {
  int64_t q[3];
  int64_t k[3];
  int64_t v[3];
  int64_t idx[3];
  int64_t out[3];
} sfa_strides;

/* Bytes of float workspace sfa_run needs for this problem on the current device
 * (0 when the problem runs without a split of the topK axis).  The workspace
 * holds the per-split partial outputs and (max, sum) pairs of the split-K
 * decode path; the float workspace of the BSR wrapper page serves the same role.
 * Returns 0 as well for an invalid problem (sfa_run then reports the error). */
size_t sfa_workspace_bytes(const sfa_shape* shape, sfa_dtype dtype, int causal);

/* Top-K sparse attention.
 *  q    [B,S1,N1,Dk] (BSND) or [B,N1,S1,Dk] (BNSD), device
 *  k    [B,S2,N2,Dk] or [B,N2,S2,Dk], device
 *  v    [B,S2,N2,Dv] or [B,N2,S2,Dv], device (may be a view of k, see sfa_strides)
 *  sparse_indices [B,S1,N2,topK] or [B,N2,S1,topK] int32, device; values must lie in
 *       [0, S2) (a value outside is treated as a masked slot, never dereferenced)
 *  Dk, Dv: multiples of 64 with Dv <= Dk (operator page, section 3 support ranges) and
 *       Dk <= 576, the widest head dim the page lists; kernels are compiled for the pairs
 *       (64,64) (128,128) (192,128) (192,192) (256,256) (512,512) (576,512) (576,576) and a
 *       call runs on the smallest pair that covers it (q columns past Dk enter the products
 *       as zeros, output columns past Dv are not written), so e.g. (320,256) runs on the
 *       (512,512) kernels.  Dk > 576 is SFA_ERR_UNSUPPORTED.
 *  scale  > 0, multiplies Q K^T before the softmax (typically 1/sqrt(Dk))
 *  causal 0/1: bottom-right causal mask (requires S1 <= S2)
 *  out  [B,S1,N1,Dv] or [B,N1,S1,Dv], device, same dtype as q (written)
 *  lse  NULL, or fp32 [B,S1,N1] (BSND) / [B,N1,S1] (BNSD) contiguous, device (written):
 *       natural-log log-sum-exp of the scaled logits of the unmasked slots, -inf
 *       for a fully masked row
 *  workspace / workspace_bytes: device scratch of at least sfa_workspace_bytes()
 *  stream: HIP stream the kernels are enqueued on (0 = default stream)
 * All buffers stay owned by the caller.  Errors are detected on the host before
 * anything is enqueued, except SFA_ERR_HIP which reports a failed launch.
 * B == 0 or S1 == 0 is a valid empty problem and enqueues nothing. */
sfa_status sfa_run(const sfa_shape* shape, const sfa_strides* strides, sfa_dtype dtype, sfa_layout layout,
                   int causal, float scale, const void* q, const void* k, const void* v,
                   const int32_t* sparse_indices, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* sfa_run for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments minus the workspace.
 * The split-K partials live in a device array inside the library, sfa_run_noalloc_max_workspace()
 * bytes (64 MiB) that every GPU the library runs on holds until the process ends; a problem
 * whose sfa_workspace_bytes() exceeds it returns SFA_ERR_WORKSPACE before anything is enqueued.
 * Nothing is allocated.  All calls on one GPU share that GPU's array: calls that overlap on one
 * GPU (different streams) race on it.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress) with that device current. */
size_t sfa_run_noalloc_max_workspace(void);
sfa_status sfa_run_noalloc(const sfa_shape* shape, const sfa_strides* strides, sfa_dtype dtype, sfa_layout layout,
                           int causal, float scale, const void* q, const void* k, const void* v,
                           const int32_t* sparse_indices, void* out, float* lse, hipStream_t stream);

/* Debug check of sparse_indices (operator page, section 3: every index lies in [0, S2)).
 * Only B, S1, S2, N2 and topK of shape are used; strides NULL means a contiguous index
 * tensor, else strides->idx gives its layout-order element strides (last dim contiguous).
 *  counts: device int32 [2], written (asynchronously, on stream): [0] = slots whose index is
 *      outside [0, S2), [1] = index rows (b, s1, n2) that list some position more than once
 *      (valid for the operator, which takes such slots one by one, but unusual)
 * S2 above 1,048,576 is SFA_ERR_UNSUPPORTED (the check keeps a bitmap of S2 bits on chip). */
sfa_status sfa_validate_indices(const sfa_shape* shape, const sfa_strides* strides, sfa_layout layout,
                                const int32_t* sparse_indices, int32_t* counts, hipStream_t stream);

/* Opaque BSR plan (host memory owned by the library; free with bsr_destroy). */
typedef struct bsr_plan_t bsr_plan_t;

/* Device bytes a bsr_plan() of this pattern needs as its (int) workspace: the expanded
 * key lists and, with a per-block mask, the packed mask words (0 if the arguments are
 * invalid).  Same pattern arguments as bsr_plan(). */
size_t bsr_plan_workspace_bytes(const int32_t* indptr, const int32_t* indices, const uint8_t* mask, int M,
                                int N, int R, int C, int num_qo_heads, int num_kv_heads, int head_dim);

/* Device bytes of float workspace the runs of a bsr_plan() of this pattern need for the
 * partial results of split key lists ("float_workspace_buffer" of the wrapper's
 * constructor on the flashinfer.sparse page: intermediate results of the split-k
 * algorithm).  0 when no key list is split, or if the arguments are invalid.  Depends on
 * the current device (its compute-unit count sets how far long key lists are split). */
size_t bsr_plan_float_workspace_bytes(const int32_t* indptr, const int32_t* indices, int M, int N, int R, int C,
                                      int num_qo_heads, int num_kv_heads, int head_dim);

/* Builds the plan of a block-sparse attention problem
 * (BlockSparseAttentionWrapper.plan: indptr, indices, M, N, R, C, num_qo_heads,
 * num_kv_heads, head_dim, mask, causal, sm_scale, dtype).
 *  indptr  host int32 [MB + 1], MB = ceil(M / R); indptr[0] == 0, non-decreasing
 *  indices host int32 [indptr[MB]]; each in [0, N / C), no repeat within a block row
 *  mask    NULL, or host uint8 [nnz = indptr[MB], R, C]: the page's per-block mask; element
 *          (i, j) of stored block t lets query row br * R + i attend key indices[t] * C + j
 *          iff nonzero.  With a mask, causal is ignored (as the page states); the mask is
 *          packed into the workspace (the host array may be freed on return).  Masked plans
 *          of head_dim 320 to 512 with more than 32 query vectors per block row and KV head
 *          are SFA_ERR_UNSUPPORTED at bsr_run
 *  N % C == 0; Hq % Hkv == 0; D a multiple of 64 up to 576 (run on the smallest compiled
 *  head dim >= D: 64, 128, 192, 256, 512 or 576)
 *  causal  0/1: bottom-right causal mask on top of the block mask (needs M <= N)
 *  sm_scale <= 0 selects 1/sqrt(D)
 *  workspace: device memory of at least bsr_plan_workspace_bytes(...) bytes, owned by
 *       the caller and kept alive and unchanged while the plan is used: it holds the key
 *       lists (and mask words), copied there asynchronously on stream (the host arrays may
 *       be freed on return)
 *  float_workspace: device memory of at least bsr_plan_float_workspace_bytes(...) bytes
 *       (may be NULL when that is 0), owned by the caller: scratch of every bsr_run() of
 *       this plan for the partials of split key lists.  Its contents need not survive
 *       between runs, so plans whose runs do not overlap may share it; runs that overlap
 *       (different streams) race on it.
 * On success *plan receives a new plan. */
sfa_status bsr_plan(bsr_plan_t** plan, const int32_t* indptr, const int32_t* indices, const uint8_t* mask, int M,
                    int N, int R, int C, int num_qo_heads, int num_kv_heads, int head_dim, int causal,
                    float sm_scale, sfa_dtype dtype, void* workspace, size_t workspace_bytes, void* float_workspace,
                    size_t float_workspace_bytes, hipStream_t stream);

/* Runs a planned BSR problem (BlockSparseAttentionWrapper.run).
 *  q [M, Hq, D], k [N, Hkv, D], v [N, Hkv, D], out [M, Hq, D]: contiguous (NHD), device
 *  lse NULL or fp32 [M, Hq] device: natural-log LSE of the scaled logits, -inf for
 *      a row with no allowed key (such a row outputs zeros) */
sfa_status bsr_run(const bsr_plan_t* plan, const void* q, const void* k, const void* v, void* out, float* lse,
                   hipStream_t stream);

/* Device bytes of the workspace bsr_run_fp8() needs for this plan (0 for a NULL plan). */
size_t bsr_fp8_workspace_bytes(const bsr_plan_t* plan);

/* Runs a planned BSR problem on FP8 inputs (BlockSparseAttentionWrapper.run with scale_q,
 * scale_k, scale_v: per-head quantisation factors of FP8 inputs, 1.0 when not given).  The
 * attention is that of q[m, h, :] * scale_q[h], k[n, hk, :] * scale_k[hk] and
 * v[n, hk, :] * scale_v[hk] (hk = h / (Hq / Hkv)).
 *  plan: made with dtype SFA_FP16 (the output dtype, fp16 as the plan page's default
 *      o_data_type; the computation runs on fp16 copies) -- else SFA_ERR_DTYPE
 *  q [M, Hq, D] codes in q_fmt, k and v [N, Hkv, D] codes in kv_fmt: contiguous (NHD),
 *      device, 16-byte aligned
 *  scale_q NULL or device fp32 [Hq]; scale_k, scale_v NULL or device fp32 [Hkv]
 *  out [M, Hq, D] fp16, lse NULL or fp32 [M, Hq], as bsr_run
 *  workspace: device, 16-byte aligned, at least bsr_fp8_workspace_bytes(plan) bytes, owned
 *      by the caller, not shared with a concurrent call.  It receives fp16 copies of q, k
 *      and v, each decoded exactly (every E4M3 / E5M2 value is an fp16 value); v reuses k's
 *      copy when v == k.
 *  scale_q and scale_k must be positive: each logit is multiplied in fp32 by
 *      sm_scale * scale_q[h] * scale_k[hk] before the softmax; the fp32 output row of query
 *      head h (and every split partial of it) is multiplied by scale_v[hk] before it is
 *      rounded to fp16.
 *  The plan's own workspace is used as by bsr_run.  Every check of bsr_run runs before
 *  anything is enqueued. */
sfa_status bsr_run_fp8(const bsr_plan_t* plan, const void* q, const void* k, const void* v, sfa_fp8 q_fmt,
                       sfa_fp8 kv_fmt, const float* scale_q, const float* scale_k, const float* scale_v, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

sfa_status bsr_destroy(bsr_plan_t* plan);

/* Opaque variable block-sparse plan (host memory owned by the library; free with
 * vbsr_destroy). */
typedef struct vbsr_plan_t vbsr_plan_t;

/* Device bytes a vbsr_plan() of this pattern needs as its (int) workspace: key lists and
 * item table (0 if the arguments are invalid).  Same pattern arguments as vbsr_plan(). */
size_t vbsr_plan_workspace_bytes(const uint8_t* block_mask_map, const int32_t* block_row_sz,
                                 const int32_t* block_col_sz, int num_kv_heads, int MB, int NB, int num_qo_heads,
                                 int head_dim);

/* Device bytes of float workspace (split-k partial results, as for bsr_plan) the runs of a
 * vbsr_plan() of this pattern need; 0 when nothing is split.  Depends on the current
 * device. */
size_t vbsr_plan_float_workspace_bytes(const uint8_t* block_mask_map, const int32_t* block_row_sz,
                                       const int32_t* block_col_sz, int num_kv_heads, int MB, int NB,
                                       int num_qo_heads, int head_dim);

/* Builds the plan of a variable block-sparse problem
 * (VariableBlockSparseAttentionWrapper.plan: block_mask_map, block_row_sz, block_col_sz,
 * num_qo_heads, num_kv_heads, head_dim, causal, sm_scale, dtype).
 *  block_mask_map host uint8 [Hkv, MB, NB]: nonzero = block (i, j) of KV head h attended
 *  block_row_sz   host int32 [Hkv, MB], block_col_sz host int32 [Hkv, NB]: sizes >= 0; every
 *                 KV head's row sizes sum to the same M (the query length) and its column
 *                 sizes to the same N >= 1 (the key length).  Block row i of head h holds
 *                 query rows sum(block_row_sz[h][:i]) .. + block_row_sz[h][i] - 1, column
 *                 block j key rows sum(block_col_sz[h][:j]) .. + block_col_sz[h][j] - 1
 *  Hq % Hkv == 0; query head n attends through KV head n / (Hq / Hkv); D a multiple of 64
 *  up to 576, as for bsr_plan
 *  causal  0/1: bottom-right causal mask (key j > row i + N - M masked) on top of the block
 *          mask (needs M <= N)
 *  sm_scale <= 0 selects 1/sqrt(D)
 *  workspace: device memory of at least vbsr_plan_workspace_bytes(...) bytes, owned by the
 *       caller and kept alive and unchanged while the plan is used: it holds the key lists
 *       and item table, copied there asynchronously on stream (the host arrays may be freed
 *       on return)
 *  float_workspace: at least vbsr_plan_float_workspace_bytes(...) bytes (NULL allowed when
 *       that is 0): split-k scratch of every vbsr_run() of this plan, as for bsr_plan
 * On success *plan receives a new plan. */
sfa_status vbsr_plan(vbsr_plan_t** plan, const uint8_t* block_mask_map, const int32_t* block_row_sz,
                     const int32_t* block_col_sz, int num_kv_heads, int MB, int NB, int num_qo_heads, int head_dim,
                     int causal, float sm_scale, sfa_dtype dtype, void* workspace, size_t workspace_bytes,
                     void* float_workspace, size_t float_workspace_bytes, hipStream_t stream);

/* Runs a planned variable block-sparse problem (VariableBlockSparseAttentionWrapper.run).
 *  q [Hq, M, D], k [Hkv, N, D], v [Hkv, N, D], out [Hq, M, D]: contiguous (HND), device; v
 *      may equal k
 *  lse NULL or fp32 [Hq, M] device: natural-log LSE of the scaled logits, -inf for a row
 *      with no allowed key (such a row outputs zeros) */
sfa_status vbsr_run(const vbsr_plan_t* plan, const void* q, const void* k, const void* v, void* out, float* lse,
                    hipStream_t stream);

/* Device bytes of the workspace vbsr_run_fp8() needs for this plan (0 for a NULL plan). */
size_t vbsr_fp8_workspace_bytes(const vbsr_plan_t* plan);

/* Runs a planned variable block-sparse problem on FP8 inputs
 * (VariableBlockSparseAttentionWrapper.run with scale_q [Hq], scale_k [Hkv], scale_v [Hkv]).
 * Same contract as bsr_run_fp8 with the HND shapes of vbsr_run: q [Hq, M, D], k and v
 * [Hkv, N, D] codes, out [Hq, M, D] fp16; the plan must have dtype SFA_FP16. */
sfa_status vbsr_run_fp8(const vbsr_plan_t* plan, const void* q, const void* k, const void* v, sfa_fp8 q_fmt,
                        sfa_fp8 kv_fmt, const float* scale_q, const float* scale_k, const float* scale_v,
                        void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

sfa_status vbsr_destroy(vbsr_plan_t* plan);

/* Static description of a status code. */
const char* sfa_status_str(sfa_status status);

/* Device bytes of workspace sfa_prefill needs for this problem on the current device (the
 * item table, the packed mask when masked != 0, split partials); 0 for invalid sizes. */
size_t sfa_prefill_workspace_bytes(int qo_len, int kv_len, int num_qo_heads, int num_kv_heads, int head_dim_qk,
                                   int head_dim_vo, int masked);

/* Dense attention of one request ("flashinfer.prefill.single_prefill_with_kv_cache": q, k, v,
 * custom_mask, causal, kv_layout, sm_scale, return_lse), the comparison baseline of the
 * sparse forms.
 *  q    [qo_len, Hq, Dqk] contiguous, device
 *  k    [kv_len, Hkv, Dqk] (NHD) or [Hkv, kv_len, Dqk] (HND), device
 *  v    [kv_len, Hkv, Dvo] or [Hkv, kv_len, Dvo], device; may be k itself or its prefix view
 *       k[..., :Dvo] (then each key row is loaded once for both)
 *  kv_strides NULL (k and v contiguous in kv_layout) or element strides {k row, k head, v row,
 *       v head}, multiples of 8; the last dim is contiguous
 *  custom_mask NULL or device uint8 / bool [qo_len, kv_len] contiguous: 0 = masked.  It is
 *       packed into the workspace on stream before the attention runs.  With a mask, causal
 *       is ignored (as the page states); without one, causal != 0 masks key j > row i +
 *       kv_len - qo_len (bottom-right, needs qo_len <= kv_len)
 *  sm_scale 0 selects 1/sqrt(Dqk); negative or non-finite is SFA_ERR_SCALE
 *  out  [qo_len, Hq, Dvo] contiguous, same dtype as q; lse NULL or fp32 [qo_len, Hq]
 *       contiguous: natural-log LSE of the scaled logits; a row with no allowed key outputs
 *       zeros and lse -inf
 *  workspace at least sfa_prefill_workspace_bytes(..., custom_mask != NULL) bytes, owned by
 *       the caller, not shared with a concurrent call
 * Dqk, Dvo multiples of 64 with Dvo <= Dqk <= 576; Hq % Hkv == 0; with a mask and Dvo above
 * 256 at most 32 query heads per KV head (else SFA_ERR_UNSUPPORTED). */
sfa_status sfa_prefill(int qo_len, int kv_len, int num_qo_heads, int num_kv_heads, int head_dim_qk, int head_dim_vo,
                       sfa_dtype dtype, sfa_kv_layout kv_layout, const int64_t* kv_strides, int causal,
                       float sm_scale, const void* q, const void* k, const void* v, const uint8_t* custom_mask,
                       void* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SFA_H_ */
