/*
 * Reference oracle for sparse flash attention, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar CPU statement
 * of what the sparse-attention hot path computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or helper with the GPU library; nothing in the product
 * path may call it.
 *
 * Sources (the pages it is written from):
 *  - "SparseFlashAttention operator API description" (cann-bench operator page):
 *      section 2 "operator definition" (formula y = softmax(Q K_sel^T * scale) V_sel
 *      and its sub-steps: sparse gather, GQA expansion, scaled dot product,
 *      optional bottom-right causal mask, softmax over the topK axis, weighted
 *      sum), the layout table (BSND / BNSD), and section 3 "rules and
 *      constraints" (a query row whose topK slots are all masked outputs 0).
 *  - "flashinfer.prefill.single_prefill_with_kv_cache": dense attention with a
 *      boolean custom_mask (False = masked), causal = tril(diagonal=kv_len-qo_len),
 *      GQA by num_qo_heads / num_kv_heads, LSE shape [qo_len, num_qo_heads].
 *  - "flashinfer.sparse", BlockSparseAttentionWrapper: the BSR mask (SciPy
 *      bsr_matrix definition: indptr over MB = ceil(M/R) block rows, indices of
 *      column blocks, NB = N / C), used as the attention mask of dense attention.
 *
 * Readings where the pages leave a step open (each also listed in the design notes):
 *  - causal rule: slot i of query row s1 is masked iff idx > s1 + (S2 - S1)
 *    (the comparison operators are lost in the page text; "above the bottom-right
 *    diagonal" and the dense tril(diagonal = S2 - S1) mask fix them);
 *  - head n1 uses KV head n1 / G with G = N1 / N2 (the GQA expansion repeats
 *    each KV head G times);
 *  - duplicate indices count once per slot (the gather produces one row per slot);
 *  - LSE is the natural log of the sum of exp of the scaled logits of the
 *    unmasked slots; a fully masked row has y = 0 and LSE = -inf;
 *  - BSR: a query row's allowed keys are the union of its block row's column
 *    blocks; duplicate column blocks are the same set.
 *
 * Parallelism: rows are independent; they are split across pthreads.  Each
 * row is computed by the same scalar loop whatever the thread count, so the
 * result does not depend on it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BSND = 0, ORACLE_BNSD = 1 };

/* ------------------------------------------------------------------------ */
/* Top-K sparse attention                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *q, *k, *v;
  const int32_t *idx;
  /* element strides of the three outer dims, in the layout's own order
     (BSND: b, s, n ; BNSD: b, n, s); the last dim is contiguous */
  int64_t qs[3], ks[3], vs[3], is[3];
  int B, S1, S2, N1, N2, Dk, Dv, topK, layout, causal;
  double scale;
  const int64_t *rows; /* flat row ids r = (b*S1 + s1)*N1 + n1, or NULL */
  int64_t nrows;
  double *y;   /* [nrows, Dv] */
  double *lse; /* [nrows] */
  int nthreads;
} sfa_job;

typedef struct {
  const sfa_job *job;
  int64_t begin, end;
} sfa_span;

/* Offset of element (b, s, n, 0) for a tensor with the given outer strides. */
static int64_t off_bsn(const int64_t st[3], int layout, int64_t b, int64_t s, int64_t n) {
  if (layout == ORACLE_BSND) return b * st[0] + s * st[1] + n * st[2];
  return b * st[0] + n * st[1] + s * st[2];
}

static void sfa_one_row(const sfa_job *J, int64_t out_row, int64_t r, double *scores) {
  const int G = J->N1 / J->N2;
  const int64_t n1 = r % J->N1;
  const int64_t s1 = (r / J->N1) % J->S1;
  const int64_t b = r / ((int64_t)J->N1 * J->S1);
  const int64_t n2 = n1 / G; /* GQA: each KV head serves G consecutive query heads */
  const double *qrow = J->q + off_bsn(J->qs, J->layout, b, s1, n1);
  const int32_t *irow = J->idx + off_bsn(J->is, J->layout, b, s1, n2);
  double *yrow = J->y + out_row * J->Dv;
  const int64_t causal_limit = s1 + ((int64_t)J->S2 - J->S1); /* bottom-right diagonal */

  /* scores_i = (q . K_sel[i]) * scale, or -inf where the causal mask applies */
  for (int i = 0; i < J->topK; ++i) {
    const int64_t j = irow[i];
    if (J->causal && j > causal_limit) {
      scores[i] = -INFINITY;
      continue;
    }
    const double *krow = J->k + off_bsn(J->ks, J->layout, b, j, n2);
    double dot = 0.0;
    for (int d = 0; d < J->Dk; ++d) dot += qrow[d] * krow[d];
    scores[i] = dot * J->scale;
  }

  /* softmax over the topK axis */
  double m = -INFINITY;
  for (int i = 0; i < J->topK; ++i)
    if (scores[i] > m) m = scores[i];
  for (int d = 0; d < J->Dv; ++d) yrow[d] = 0.0;
  if (m == -INFINITY) { /* every slot masked: the row outputs zeros */
    J->lse[out_row] = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int i = 0; i < J->topK; ++i) l += exp(scores[i] - m); /* exp(-inf) = 0 */
  for (int i = 0; i < J->topK; ++i) {
    const double w = exp(scores[i] - m) / l;
    if (w == 0.0) continue;
    const double *vrow = J->v + off_bsn(J->vs, J->layout, b, irow[i], n2);
    for (int d = 0; d < J->Dv; ++d) yrow[d] += w * vrow[d];
  }
  J->lse[out_row] = m + log(l);
}

static void *sfa_worker(void *arg) {
  const sfa_span *sp = (const sfa_span *)arg;
  const sfa_job *J = sp->job;
  double *scores = (double *)malloc(sizeof(double) * (size_t)(J->topK > 0 ? J->topK : 1));
  for (int64_t t = sp->begin; t < sp->end; ++t) {
    const int64_t r = J->rows ? J->rows[t] : t;
    sfa_one_row(J, t, r, scores);
  }
  free(scores);
  return NULL;
}

static void run_spans(void *(*fn)(void *), void *job, size_t span_size, int64_t n, int nthreads,
                      void (*fill)(void *span, void *job, int64_t b, int64_t e)) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
  char *spans = (char *)calloc((size_t)nthreads, span_size);
  for (int t = 0; t < nthreads; ++t) {
    const int64_t b = n * t / nthreads, e = n * (t + 1) / nthreads;
    fill(spans + span_size * t, job, b, e);
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fn, spans + span_size * t);
  fn(spans);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(spans);
  free(th);
}

static void sfa_fill(void *span, void *job, int64_t b, int64_t e) {
  sfa_span *s = (sfa_span *)span;
  s->job = (const sfa_job *)job;
  s->begin = b;
  s->end = e;
}

/* Computes rows of y (and LSE) for the top-K sparse attention operator.
 * q: [B,S1,N1,Dk] (BSND) or [B,N1,S1,Dk] (BNSD), k: [.,S2,N2,Dk], v: [.,S2,N2,Dv],
 * idx: [B,S1,N2,topK] or [B,N2,S1,topK]; each given by its three outer element
 * strides in layout order and a contiguous last dim.  rows: flat (b,s1,n1) ids
 * (r = (b*S1 + s1)*N1 + n1) to compute, or NULL for all B*S1*N1 rows in order.
 * y: [nrows, Dv]; lse: [nrows].  Returns 0, or -1 on an invalid shape. */
int oracle_sfa(const double *q, const int64_t *q_strides, const double *k, const int64_t *k_strides,
               const double *v, const int64_t *v_strides, const int32_t *idx, const int64_t *idx_strides,
               int B, int S1, int S2, int N1, int N2, int Dk, int Dv, int topK, int layout, int causal,
               double scale, const int64_t *rows, int64_t nrows, double *y, double *lse, int nthreads) {
  if (B < 0 || S1 < 0 || S2 < 1 || N1 < 1 || N2 < 1 || N1 % N2 || Dk < 1 || Dv < 1 || topK < 0) return -1;
  if (layout != ORACLE_BSND && layout != ORACLE_BNSD) return -1;
  sfa_job J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.idx = idx;
  memcpy(J.qs, q_strides, sizeof J.qs);
  memcpy(J.ks, k_strides, sizeof J.ks);
  memcpy(J.vs, v_strides, sizeof J.vs);
  memcpy(J.is, idx_strides, sizeof J.is);
  J.B = B; J.S1 = S1; J.S2 = S2; J.N1 = N1; J.N2 = N2; J.Dk = Dk; J.Dv = Dv; J.topK = topK;
  J.layout = layout; J.causal = causal; J.scale = scale;
  J.rows = rows;
  J.nrows = rows ? nrows : (int64_t)B * S1 * N1;
  J.y = y; J.lse = lse;
  run_spans(sfa_worker, &J, sizeof(sfa_span), J.nrows, nthreads, sfa_fill);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dense attention with a boolean mask (NHD layout)                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *q, *k, *v;
  const uint8_t *mask; /* [qo_len, kv_len], nonzero = attend; NULL = none */
  int causal;
  int qo_len, kv_len, Hq, Hkv, Dqk, Dvo;
  double scale;
  const int64_t *rows; /* flat ids r = qo_row*Hq + head, or NULL */
  int64_t nrows;
  double *y, *lse;
} dense_job;

typedef struct {
  const dense_job *job;
  int64_t begin, end;
} dense_span;

static void dense_one_row(const dense_job *J, int64_t out_row, int64_t r, double *scores) {
  const int G = J->Hq / J->Hkv;
  const int64_t h = r % J->Hq, qi = r / J->Hq;
  const int64_t hk = h / G;
  const double *qrow = J->q + (qi * J->Hq + h) * J->Dqk;
  double *yrow = J->y + out_row * J->Dvo;
  double m = -INFINITY;
  for (int64_t j = 0; j < J->kv_len; ++j) {
    int allowed;
    if (J->mask) allowed = J->mask[qi * J->kv_len + j] != 0;
    else if (J->causal) allowed = j <= qi + (J->kv_len - J->qo_len); /* tril(diagonal = kv_len - qo_len) */
    else allowed = 1;
    if (!allowed) {
      scores[j] = -INFINITY;
      continue;
    }
    const double *krow = J->k + (j * J->Hkv + hk) * J->Dqk;
    double dot = 0.0;
    for (int d = 0; d < J->Dqk; ++d) dot += qrow[d] * krow[d];
    scores[j] = dot * J->scale;
    if (scores[j] > m) m = scores[j];
  }
  for (int d = 0; d < J->Dvo; ++d) yrow[d] = 0.0;
  if (m == -INFINITY) {
    J->lse[out_row] = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < J->kv_len; ++j) l += exp(scores[j] - m);
  for (int64_t j = 0; j < J->kv_len; ++j) {
    const double w = exp(scores[j] - m) / l;
    if (w == 0.0) continue;
    const double *vrow = J->v + (j * J->Hkv + hk) * J->Dvo;
    for (int d = 0; d < J->Dvo; ++d) yrow[d] += w * vrow[d];
  }
  J->lse[out_row] = m + log(l);
}

static void *dense_worker(void *arg) {
  const dense_span *sp = (const dense_span *)arg;
  const dense_job *J = sp->job;
  double *scores = (double *)malloc(sizeof(double) * (size_t)(J->kv_len > 0 ? J->kv_len : 1));
  for (int64_t t = sp->begin; t < sp->end; ++t) dense_one_row(J, t, J->rows ? J->rows[t] : t, scores);
  free(scores);
  return NULL;
}

static void dense_fill(void *span, void *job, int64_t b, int64_t e) {
  dense_span *s = (dense_span *)span;
  s->job = (const dense_job *)job;
  s->begin = b;
  s->end = e;
}

/* Dense attention.  q: [qo_len, Hq, Dqk], k: [kv_len, Hkv, Dqk], v: [kv_len, Hkv, Dvo]
 * (contiguous NHD); mask: [qo_len, kv_len] bytes (nonzero = attend) or NULL, in which
 * case causal selects the bottom-right causal mask.  rows: flat ids qo_row*Hq + head,
 * or NULL for all.  y: [nrows, Dvo]; lse: [nrows]. */
int oracle_dense_masked(const double *q, const double *k, const double *v, const uint8_t *mask, int causal,
                        int qo_len, int kv_len, int Hq, int Hkv, int Dqk, int Dvo, double scale,
                        const int64_t *rows, int64_t nrows, double *y, double *lse, int nthreads) {
  if (qo_len < 0 || kv_len < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || Dqk < 1 || Dvo < 1) return -1;
  dense_job J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.mask = mask; J.causal = causal;
  J.qo_len = qo_len; J.kv_len = kv_len; J.Hq = Hq; J.Hkv = Hkv; J.Dqk = Dqk; J.Dvo = Dvo;
  J.scale = scale;
  J.rows = rows;
  J.nrows = rows ? nrows : (int64_t)qo_len * Hq;
  J.y = y; J.lse = lse;
  run_spans(dense_worker, &J, sizeof(dense_span), J.nrows, nthreads, dense_fill);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Block-sparse (BSR) attention                                              */
/* ------------------------------------------------------------------------ */

/* Expands a BSR block pattern into the dense [M, N] boolean mask it denotes:
 * element (r, c) is set iff column block c / C is listed for block row r / R.
 * Returns 0, or -1 if the pattern is malformed. */
int oracle_bsr_mask(const int32_t *indptr, const int32_t *indices, int M, int N, int R, int C, uint8_t *mask) {
  if (M < 0 || N < 0 || R < 1 || C < 1 || N % C) return -1;
  const int MB = (M + R - 1) / R, NB = N / C;
  if (indptr[0] != 0) return -1;
  memset(mask, 0, (size_t)M * (size_t)N);
  for (int br = 0; br < MB; ++br) {
    if (indptr[br + 1] < indptr[br]) return -1;
    for (int t = indptr[br]; t < indptr[br + 1]; ++t) {
      const int bc = indices[t];
      if (bc < 0 || bc >= NB) return -1;
      for (int r = br * R; r < (br + 1) * R && r < M; ++r)
        for (int c = bc * C; c < (bc + 1) * C; ++c) mask[(size_t)r * N + c] = 1;
    }
  }
  return 0;
}

/* BSR attention: dense attention under the BSR mask.  q: [M, Hq, D], k, v: [N, Hkv, D];
 * scale <= 0 means 1/sqrt(D).  bmask (NULL: every stored block is full) is the per-block mask
 * of the plan page, [nnz, R, C] bytes: element (i, j) of stored block t (block row br, column
 * block indices[t]) is attended iff bmask[(t * R + i) * C + j] != 0, for query row br * R + i
 * and key column indices[t] * C + j.  causal applies only without a per-block mask (the page
 * ignores it when a mask is given) and adds the bottom-right causal mask. */
int oracle_bsr(const double *q, const double *k, const double *v, const int32_t *indptr, const int32_t *indices,
               const uint8_t *bmask, int M, int N, int R, int C, int Hq, int Hkv, int D, int causal, double scale,
               const int64_t *rows, int64_t nrows, double *y, double *lse, int nthreads) {
  uint8_t *mask = (uint8_t *)malloc((size_t)M * (size_t)N + 1);
  if (!mask) return -1;
  if (oracle_bsr_mask(indptr, indices, M, N, R, C, mask)) {
    free(mask);
    return -1;
  }
  if (bmask) {
    const int MB = (M + R - 1) / R;
    for (int br = 0; br < MB; ++br)
      for (int t = indptr[br]; t < indptr[br + 1]; ++t)
        for (int i = 0; i < R && br * R + i < M; ++i)
          for (int j = 0; j < C; ++j)
            mask[(size_t)(br * R + i) * N + (size_t)indices[t] * C + j] = bmask[((size_t)t * R + i) * C + j] != 0;
    causal = 0;
  }
  if (causal)
    for (int64_t r = 0; r < M; ++r)
      for (int64_t c = 0; c < N; ++c)
        if (c > r + ((int64_t)N - M)) mask[r * N + c] = 0;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  const int rc = oracle_dense_masked(q, k, v, mask, 0, M, N, Hq, Hkv, D, D, scale, rows, nrows, y, lse, nthreads);
  free(mask);
  return rc;
}
