/*
 * Plain CPU oracle for the matrix-absorbed, NoPE Gated MLA attention layer
 * (and, at the end of the file, for chunk_kda's recurrence).
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header,
 * table or helper with the HIP library; neither side includes the other.
 *
 * Every floating-point quantity is accumulated in float64.  Inputs are the
 * stored values (float32, or bf16 widened exactly to float32 by the caller).
 * No intermediate result is rounded to a narrower type.
 *
 * Sources (the K3 teaching notes):
 *   [MLA]  page "Gated MLA（矩阵吸收版）" (matrix-absorbed Gated MLA):
 *          section 低秩压缩 (low-rank compression: the latent c, W_UK, W_UV),
 *          section 矩阵吸收的核心思路 (absorbing W_UK into q),
 *          section 完整计算流（四步） (the four-step computation, steps 2-4),
 *          section 代码对照 (the GatedMLA.forward listing),
 *          the warning box on reordering (attn·c)·W_UV^T by associativity.
 *   [SYM]  page "符号表" (symbol table): section MLA 变量 (MLA variables and
 *          their shapes) and section Einsum 速查 (einsum cheat-sheet).
 *
 * Definition computed (prefill), for every batch b, head h, query t:
 *   1. qa[j]  = sum_d q[b,t,h,d] * W_UK[h,d,j]                 ([MLA] step 2, absorb)
 *   2. s_u    = scale * sum_j qa[j] * c[b,u,j]   for u <= t     ([MLA] step 2, score;
 *               keys u > t are excluded, the causal mask keeps the diagonal)
 *   3. w_u    = exp(s_u - m) / sum_{u'<=t} exp(s_u' - m),  m = max_u s_u
 *                                                              ([MLA] step 2, softmax)
 *   4. ol[j]  = sum_{u<=t} w_u * c[b,u,j]                       ([MLA] step 3, latent sum)
 *   5. o[v]   = sum_j ol[j] * W_UV[h,v,j]                       ([MLA] step 3, W_UV^T)
 *   6. out[b,t,h*d_v+v] = o[v] / (1 + exp(-gate[b,t,h*d_v+v])) ([MLA] step 4, gate;
 *               heads flattened head-major, the output projection is not applied)
 * The softmax scale is an explicit argument: the pages print none.
 *
 * Chunked prefill (oracle_extend): the T queries of a chunk sit after a
 * cached prefix of S - T positions and attend to it as well.
 *
 * Decode: sequence i with cache rows c_cache[cu[i] .. cu[i+1]) is the same
 * computation for the query at position len_i - 1, which attends to all
 * len_i cached rows (its own latent included).
 *
 * ORACLE_MUTANT (default 0) plants one known mistake; it exists only so that
 * the pin tests can show that each such mistake is caught.  Product builds
 * and every parity comparison use ORACLE_MUTANT == 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

int oracle_mutant(void) { return ORACLE_MUTANT; }

/* Step 1 for one (row, head): qa[j] = sum_d q[d] W_UK[h,d,j]. */
static void absorb_row(const float* qh, const float* wuk_h, int dq, int r, double* qa) {
  for (int j = 0; j < r; ++j) qa[j] = 0.0;
  for (int d = 0; d < dq; ++d) {
    const double qd = (double)qh[d];
    for (int j = 0; j < r; ++j) {
#if ORACLE_MUTANT == 3
      /* planted mistake: W_UK read as [H, r, d_q] */
      qa[j] += qd * (double)wuk_h[(int64_t)j * dq + d];
#else
      qa[j] += qd * (double)wuk_h[(int64_t)d * r + j];
#endif
    }
  }
}

/*
 * One query row, all heads.  keys: nkeys latent rows of length r (row-major),
 * qrow: [H, dq], grow: [H*dv] gate logits, out: [H*dv].
 * scratch: r (qa) + r (ol) + nkeys (scores) doubles.
 */
static void attend_row(const float* qrow, const float* keys, int64_t nkeys, const float* grow,
                       const float* w_uk, const float* w_uv, int H, int dq, int dv, int r,
                       double scale, double* scratch, double* out) {
  double* qa = scratch;
  double* ol = scratch + r;
  double* s = scratch + 2 * (int64_t)r;
  for (int h = 0; h < H; ++h) {
    /* step 1: absorb W_UK into the query */
    absorb_row(qrow + (int64_t)h * dq, w_uk + (int64_t)h * dq * r, dq, r, qa);

    /* step 2: latent scores against every visible key */
    for (int64_t u = 0; u < nkeys; ++u) {
      const float* cu = keys + u * r;
      double acc = 0.0;
#pragma omp simd reduction(+ : acc)
      for (int j = 0; j < r; ++j) acc += qa[j] * (double)cu[j];
#if ORACLE_MUTANT == 7
      s[u] = acc; /* planted mistake: scale ignored */
#else
      s[u] = scale * acc;
#endif
    }

    /* step 3: softmax over the visible keys (max-subtracted) */
    double m = -INFINITY;
    for (int64_t u = 0; u < nkeys; ++u) m = s[u] > m ? s[u] : m;
    double sum = 0.0;
    for (int64_t u = 0; u < nkeys; ++u) {
#if ORACLE_MUTANT == 2
      s[u] = exp(m - s[u]); /* planted mistake: sign of the exponent */
#else
      s[u] = exp(s[u] - m);
#endif
      sum += s[u];
    }
#if ORACLE_MUTANT != 8
    for (int64_t u = 0; u < nkeys; ++u) s[u] /= sum;
#endif
    /* (mutant 8 plants a missing normalisation) */

    /* step 4: weighted sum in the latent space */
    for (int j = 0; j < r; ++j) ol[j] = 0.0;
    for (int64_t u = 0; u < nkeys; ++u) {
#if ORACLE_MUTANT == 9
      const float* cu = keys + (nkeys - 1) * r; /* planted mistake: the query's own row */
#else
      const float* cu = keys + u * r;
#endif
      const double w = s[u];
      for (int j = 0; j < r; ++j) ol[j] += w * (double)cu[j];
    }

    /* step 5: up-project with W_UV[h]^T, step 6: sigmoid gate, head-major flatten */
    const float* wuv_h = w_uv + (int64_t)h * dv * r;
    for (int v = 0; v < dv; ++v) {
      double o = 0.0;
#pragma omp simd reduction(+ : o)
      for (int j = 0; j < r; ++j) {
#if ORACLE_MUTANT == 4
        o += ol[j] * (double)wuv_h[(int64_t)j * dv + v]; /* planted: W_UV read as [H, r, d_v] */
#else
        o += ol[j] * (double)wuv_h[(int64_t)v * r + j];
#endif
      }
#if ORACLE_MUTANT == 5
      const int64_t col = (int64_t)v * H + h; /* planted mistake: value-major flatten */
#else
      const int64_t col = (int64_t)h * dv + v;
#endif
#if ORACLE_MUTANT == 6
      out[col] = o / (1.0 + exp((double)grow[col])); /* planted: sigmoid(-g) */
#else
      out[col] = o / (1.0 + exp(-(double)grow[col]));
#endif
    }
  }
}

/*
 * Chunked prefill against a cached prefix (and, with S == T, plain prefill).
 * Sequence b holds S latent rows c[b, 0..S); its T queries sit at positions
 * P .. P+T-1 with P = S - T, and query t attends to keys 0 .. P+t (the
 * causal mask of the MLA page, section 完整计算流（四步） step 2, measured
 * from the chunk's first position).  q, gate and the output have T rows per
 * sequence; rows[] (flattened b*T + t) selects which of them to compute, or
 * all when rows == NULL.
 */
int oracle_extend(const float* q, const float* c, const float* w_uk, const float* w_uv,
                  const float* gate, int B, int T, int S, int H, int dq, int dv, int r, double scale,
                  const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (!q || !c || !w_uk || !w_uv || !gate || !out) return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || S < T || H <= 0 || dq <= 0 || dv <= 0 || r <= 0 || nrows < 0)
    return ORACLE_EINVAL;
  if (!rows && nrows != (int64_t)B * T) return ORACLE_EINVAL;
  if (rows)
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= (int64_t)B * T) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t P = (int64_t)S - T;
  const int64_t scratch_len = 2 * (int64_t)r + S;
  int err = ORACLE_OK;
#pragma omp parallel num_threads(nthreads)
  {
    double* scratch = (double*)malloc(sizeof(double) * scratch_len);
    if (!scratch) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    }
#pragma omp barrier
    if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t row = rows ? rows[i] : i;
        const int64_t b = row / T, t = row % T;
#if ORACLE_MUTANT == 1
        const int64_t nkeys = P + t; /* planted mistake: diagonal excluded */
#elif ORACLE_MUTANT == 11
        const int64_t nkeys = t + 1; /* planted mistake: cached prefix ignored */
#else
        const int64_t nkeys = P + t + 1;
#endif
        attend_row(q + row * H * dq, c + b * (int64_t)S * r, nkeys, gate + row * H * dv, w_uk,
                   w_uv, H, dq, dv, r, scale, scratch, out + i * (int64_t)H * dv);
      }
    }
    free(scratch);
  }
  return err;
}

/* Prefill: every position of B sequences of length T (no cached prefix). */
int oracle_prefill(const float* q, const float* c, const float* w_uk, const float* w_uv,
                   const float* gate, int B, int T, int H, int dq, int dv, int r, double scale,
                   const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  return oracle_extend(q, c, w_uk, w_uv, gate, B, T, T, H, dq, dv, r, scale, rows, nrows, out, nthreads);
}

/*
 * Decode.  q [B,H,dq] (one query per sequence), c_cache [sum_len, r],
 * cu_seqlens [B+1] exclusive prefix sums with len_i >= 1, gate [B,H*dv].
 * seqs: nseqs sequence indices (NULL: all B in order).  out: [nseqs, H*dv].
 */
int oracle_decode(const float* q, const float* c_cache, const int64_t* cu_seqlens,
                  const float* w_uk, const float* w_uv, const float* gate, int B, int H, int dq,
                  int dv, int r, double scale, const int64_t* seqs, int64_t nseqs, double* out,
                  int nthreads) {
  if (!q || !c_cache || !cu_seqlens || !w_uk || !w_uv || !gate || !out) return ORACLE_EINVAL;
  if (B <= 0 || H <= 0 || dq <= 0 || dv <= 0 || r <= 0 || nseqs < 0) return ORACLE_EINVAL;
  if (!seqs && nseqs != B) return ORACLE_EINVAL;
  if (cu_seqlens[0] != 0) return ORACLE_EINVAL;
  int64_t max_len = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
    if (len < 1) return ORACLE_EINVAL;
    if (len > max_len) max_len = len;
  }
  if (seqs)
    for (int64_t k = 0; k < nseqs; ++k)
      if (seqs[k] < 0 || seqs[k] >= B) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t scratch_len = 2 * (int64_t)r + max_len;
  int err = ORACLE_OK;
#pragma omp parallel num_threads(nthreads)
  {
    double* scratch = (double*)malloc(sizeof(double) * scratch_len);
    if (!scratch) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    }
#pragma omp barrier
    if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
      for (int64_t k = 0; k < nseqs; ++k) {
        const int64_t i = seqs ? seqs[k] : k;
        const int64_t start = cu_seqlens[i];
#if ORACLE_MUTANT == 10
        const int64_t len = cu_seqlens[i + 1] - start - 1; /* planted: newest row dropped */
#else
        const int64_t len = cu_seqlens[i + 1] - start;
#endif
        attend_row(q + i * (int64_t)H * dq, c_cache + start * r, len, gate + i * (int64_t)H * dv,
                   w_uk, w_uv, H, dq, dv, r, scale, scratch, out + k * (int64_t)H * dv);
      }
    }
    free(scratch);
  }
  return err;
}

/*
 * The decompressed ("standard") route, written separately: per head,
 * K_h = c W_UK[h]^T  [T, dq] and V_h = c W_UV[h]^T  [T, dv], then causal
 * softmax(scale * q_h K_h^T) V_h and the same gate.  By associativity this
 * equals the absorbed route ([MLA] section 矩阵吸收的核心思路 and the warning
 * box on reordering the W_UV product).  All rows, out [B,T,H*dv].
 */
int oracle_prefill_decompressed(const float* q, const float* c, const float* w_uk,
                                const float* w_uv, const float* gate, int B, int T, int H, int dq,
                                int dv, int r, double scale, double* out, int nthreads) {
  if (!q || !c || !w_uk || !w_uv || !gate || !out) return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || H <= 0 || dq <= 0 || dv <= 0 || r <= 0) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int err = ORACLE_OK;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      double* K = (double*)malloc(sizeof(double) * (size_t)T * dq);
      double* V = (double*)malloc(sizeof(double) * (size_t)T * dv);
      double* p = (double*)malloc(sizeof(double) * (size_t)T);
      if (!K || !V || !p) {
#pragma omp atomic write
        err = ORACLE_ENOMEM;
      } else {
        const float* cb = c + (int64_t)b * T * r;
        const float* wk = w_uk + (int64_t)h * dq * r;
        const float* wv = w_uv + (int64_t)h * dv * r;
        for (int u = 0; u < T; ++u) {
          for (int d = 0; d < dq; ++d) {
            double a = 0.0;
            for (int j = 0; j < r; ++j) a += (double)cb[(int64_t)u * r + j] * (double)wk[(int64_t)d * r + j];
            K[(int64_t)u * dq + d] = a;
          }
          for (int v = 0; v < dv; ++v) {
            double a = 0.0;
            for (int j = 0; j < r; ++j) a += (double)cb[(int64_t)u * r + j] * (double)wv[(int64_t)v * r + j];
            V[(int64_t)u * dv + v] = a;
          }
        }
        for (int t = 0; t < T; ++t) {
          const float* qv = q + (((int64_t)b * T + t) * H + h) * dq;
          double mx = -INFINITY;
          for (int u = 0; u <= t; ++u) {
            double a = 0.0;
            for (int d = 0; d < dq; ++d) a += (double)qv[d] * K[(int64_t)u * dq + d];
            p[u] = scale * a;
            if (p[u] > mx) mx = p[u];
          }
          double sum = 0.0;
          for (int u = 0; u <= t; ++u) {
            p[u] = exp(p[u] - mx);
            sum += p[u];
          }
          for (int v = 0; v < dv; ++v) {
            double a = 0.0;
            for (int u = 0; u <= t; ++u) a += p[u] * V[(int64_t)u * dv + v];
            const int64_t col = (((int64_t)b * T + t) * H + h) * dv + v;
            out[col] = (a / sum) / (1.0 + exp(-(double)gate[col]));
          }
        }
      }
      free(K);
      free(V);
      free(p);
    }
  }
  return err;
}

/*
 * Step 3 exposed for the structural pins: the attention weights
 * attn[b,h,t,u] (zero for u > t), shape [B,H,T,T].  Same code path as
 * oracle_prefill's steps 1-3.
 */
int oracle_prefill_attn(const float* q, const float* c, const float* w_uk, int B, int T, int H,
                        int dq, int r, double scale, double* attn) {
  if (!q || !c || !w_uk || !attn) return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || H <= 0 || dq <= 0 || r <= 0) return ORACLE_EINVAL;
  double* qa = (double*)malloc(sizeof(double) * (size_t)r);
  double* s = (double*)malloc(sizeof(double) * (size_t)T);
  if (!qa || !s) {
    free(qa);
    free(s);
    return ORACLE_ENOMEM;
  }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < T; ++t) {
        absorb_row(q + (((int64_t)b * T + t) * H + h) * dq, w_uk + (int64_t)h * dq * r, dq, r, qa);
#if ORACLE_MUTANT == 1
        const int nkeys = t;
#else
        const int nkeys = t + 1;
#endif
        double m = -INFINITY;
        for (int u = 0; u < nkeys; ++u) {
          const float* cu = c + ((int64_t)b * T + u) * r;
          double acc = 0.0;
          for (int j = 0; j < r; ++j) acc += qa[j] * (double)cu[j];
          s[u] = scale * acc;
          if (s[u] > m) m = s[u];
        }
        double sum = 0.0;
        for (int u = 0; u < nkeys; ++u) {
#if ORACLE_MUTANT == 2
          s[u] = exp(m - s[u]);
#else
          s[u] = exp(s[u] - m);
#endif
          sum += s[u];
        }
        double* row = attn + (((int64_t)b * H + h) * T + t) * T;
        for (int u = 0; u < T; ++u) row[u] = 0.0;
        for (int u = 0; u < nkeys; ++u) {
#if ORACLE_MUTANT == 8
          row[u] = s[u];
#else
          row[u] = s[u] / sum;
#endif
        }
      }
  free(qa);
  free(s);
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Paged latent cache.  The pages cache only c ([MLA] section 低秩压缩); a
 * paged cache stores each sequence's latent rows in fixed-size pages of a
 * shared pool: row u of sequence b lives in page block_table[b, u / page_size]
 * at slot u % page_size.  The paged entry points compute exactly what their
 * packed counterparts compute on the rows gathered in order; the gather is
 * written out here and the packed functions above do the rest.
 */
static int gather_rows(const float* pages, int64_t num_pages, int page_size, const int64_t* block_table,
                       int max_pages, int64_t b, int64_t len, int r, float* dst) {
  for (int64_t u = 0; u < len; ++u) {
#if ORACLE_MUTANT == 20
    const int64_t pg = block_table[b * page_size + u / page_size]; /* planted: wrong block-table stride */
#else
    const int64_t pg = block_table[b * max_pages + u / page_size];
#endif
    if (pg < 0 || pg >= num_pages) return ORACLE_EINVAL;
#if ORACLE_MUTANT == 21
    const int64_t slot = (u + 1) % page_size; /* planted mistake: slot off by one */
#else
    const int64_t slot = u % page_size;
#endif
    memcpy(dst + u * r, pages + (pg * page_size + slot) * (int64_t)r, sizeof(float) * (size_t)r);
  }
  return ORACLE_OK;
}

/* Decode against a paged cache: sequence i holds seq_lens[i] rows (>= 1).
 * Only the selected sequences (seqs, or all) are gathered. */
int oracle_decode_paged(const float* q, const float* pages, int64_t num_pages, int page_size,
                        const int64_t* block_table, int max_pages, const int64_t* seq_lens, const float* w_uk,
                        const float* w_uv, const float* gate, int B, int H, int dq, int dv, int r, double scale,
                        const int64_t* seqs, int64_t nseqs, double* out, int nthreads) {
  if (!q || !pages || !block_table || !seq_lens || !gate || B <= 0 || H <= 0 || dq <= 0 || dv <= 0 ||
      page_size <= 0 || max_pages <= 0 || r <= 0 || nseqs < 0 || (!seqs && nseqs != B))
    return ORACLE_EINVAL;
  for (int i = 0; i < B; ++i)
    if (seq_lens[i] < 1 || seq_lens[i] > (int64_t)max_pages * page_size) return ORACLE_EINVAL;
  if (seqs)
    for (int64_t k = 0; k < nseqs; ++k)
      if (seqs[k] < 0 || seqs[k] >= B) return ORACLE_EINVAL;
  if (nseqs == 0) return ORACLE_OK;
  int64_t* cu = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseqs + 1));
  float* qs = (float*)malloc(sizeof(float) * (size_t)nseqs * H * dq);
  float* gs = (float*)malloc(sizeof(float) * (size_t)nseqs * H * dv);
  int err = (cu && qs && gs) ? ORACLE_OK : ORACLE_ENOMEM;
  float* packed = NULL;
  if (err == ORACLE_OK) {
    cu[0] = 0;
    for (int64_t k = 0; k < nseqs; ++k) cu[k + 1] = cu[k] + seq_lens[seqs ? seqs[k] : k];
    packed = (float*)malloc(sizeof(float) * (size_t)cu[nseqs] * r);
    if (!packed) err = ORACLE_ENOMEM;
  }
  for (int64_t k = 0; k < nseqs && err == ORACLE_OK; ++k) {
    const int64_t i = seqs ? seqs[k] : k;
    memcpy(qs + k * H * dq, q + i * H * dq, sizeof(float) * (size_t)H * dq);
    memcpy(gs + k * H * dv, gate + i * H * dv, sizeof(float) * (size_t)H * dv);
    err = gather_rows(pages, num_pages, page_size, block_table, max_pages, i, seq_lens[i], r, packed + cu[k] * r);
  }
  if (err == ORACLE_OK)
    err = oracle_decode(qs, packed, cu, w_uk, w_uv, gs, (int)nseqs, H, dq, dv, r, scale, NULL, nseqs, out,
                        nthreads);
  free(packed);
  free(cu);
  free(qs);
  free(gs);
  return err;
}

/* Chunked prefill against a paged cache: every sequence holds S rows, the
 * chunk's T queries are its positions S-T .. S-1 (as oracle_extend). */
int oracle_extend_paged(const float* q, const float* pages, int64_t num_pages, int page_size,
                        const int64_t* block_table, int max_pages, const float* w_uk, const float* w_uv,
                        const float* gate, int B, int T, int S, int H, int dq, int dv, int r, double scale,
                        const int64_t* rows, int64_t nrows, double* out, int nthreads) {
  if (!pages || !block_table || B <= 0 || T <= 0 || S < T || page_size <= 0 || r <= 0 ||
      (int64_t)max_pages * page_size < S)
    return ORACLE_EINVAL;
  float* packed = (float*)malloc(sizeof(float) * (size_t)B * S * r);
  int err = packed ? ORACLE_OK : ORACLE_ENOMEM;
  for (int b = 0; b < B && err == ORACLE_OK; ++b)
    err = gather_rows(pages, num_pages, page_size, block_table, max_pages, b, S, r, packed + (int64_t)b * S * r);
  if (err == ORACLE_OK)
    err = oracle_extend(q, packed, w_uk, w_uv, gate, B, T, S, H, dq, dv, r, scale, rows, nrows, out, nthreads);
  free(packed);
  return err;
}

/* Varlen chunked prefill against a paged cache: sequence b owns the
 * T_b = cu_q[b+1] - cu_q[b] packed query rows cu_q[b] .. (q [Nq, H, dq], gate
 * and out [Nq, H*dv]) and seq_lens[b] = S_b >= T_b cache rows; its chunk is
 * positions S_b - T_b .. S_b - 1.  A batch that mixes prefill chunks
 * (S_b = T_b), chunks after a cached prefix and decode steps (T_b = 1) is one
 * call.  Each sequence is oracle_extend on its gathered rows. */
int oracle_extend_varlen_paged(const float* q, const float* pages, int64_t num_pages, int page_size,
                               const int64_t* block_table, int max_pages, const int64_t* cu_q, const int64_t* seq_lens,
                               const float* w_uk, const float* w_uv, const float* gate, int B, int H, int dq, int dv,
                               int r, double scale, double* out, int nthreads) {
  if (!q || !pages || !block_table || !cu_q || !seq_lens || !gate || !out || B <= 0 || H <= 0 || dq <= 0 ||
      dv <= 0 || r <= 0 || page_size <= 0 || max_pages <= 0 || cu_q[0] != 0)
    return ORACLE_EINVAL;
  int err = ORACLE_OK;
  for (int b = 0; b < B && err == ORACLE_OK; ++b) {
    const int64_t T = cu_q[b + 1] - cu_q[b], S = seq_lens[b];
    if (T < 0 || S < T || S > (int64_t)max_pages * page_size) return ORACLE_EINVAL;
    if (T == 0) continue;
    float* rows = (float*)malloc(sizeof(float) * (size_t)S * r);
    if (!rows) return ORACLE_ENOMEM;
    err = gather_rows(pages, num_pages, page_size, block_table, max_pages, b, S, r, rows);
    if (err == ORACLE_OK)
#if ORACLE_MUTANT == 26
      /* planted mistake: the chunk placed at the start of the sequence */
      err = oracle_extend(q + cu_q[b] * H * dq, rows, w_uk, w_uv, gate + cu_q[b] * H * dv, 1, (int)T, (int)T, H, dq,
                          dv, r, scale, NULL, T, out + cu_q[b] * H * dv, nthreads);
#else
      err = oracle_extend(q + cu_q[b] * H * dq, rows, w_uk, w_uv, gate + cu_q[b] * H * dv, 1, (int)T, (int)S, H, dq,
                          dv, r, scale, NULL, T, out + cu_q[b] * H * dv, nthreads);
#endif
    free(rows);
  }
  return err;
}

/* Cache append: row c_new[i] becomes row positions[i] of sequence i, i.e. it
 * is written to page block_table[i, positions[i] / page_size], slot
 * positions[i] % page_size, in place. */
int oracle_cache_append(const float* c_new, float* pages, int64_t num_pages, int page_size,
                        const int64_t* block_table, int max_pages, const int64_t* positions, int B, int r) {
  if (!c_new || !pages || !block_table || !positions || B <= 0 || page_size <= 0 || r <= 0) return ORACLE_EINVAL;
  for (int i = 0; i < B; ++i) {
    const int64_t u = positions[i];
    if (u < 0 || u >= (int64_t)max_pages * page_size) return ORACLE_EINVAL;
    const int64_t pg = block_table[(int64_t)i * max_pages + u / page_size];
    if (pg < 0 || pg >= num_pages) return ORACLE_EINVAL;
    memcpy(pages + (pg * page_size + u % page_size) * (int64_t)r, c_new + (int64_t)i * r, sizeof(float) * (size_t)r);
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Full Gated MLA forward around the absorbed core ([MLA] section 低秩压缩 for
 * the latent, section 完整计算流（四步） step 1 for the query low-rank path,
 * step 4 for the gate and the output projection, the parameter table of
 * section 形状与参数对比 for the weight layouts):
 *
 *   c    = RMSNorm_kv(x W_kv_down^T)       [N, r]        (N = B*T rows)
 *   ql   = RMSNorm_q(x W_q_down^T)         [N, q_rank]
 *   q    = ql W_q_up^T                     [N, H*dq], viewed [B, T, H, dq]
 *   g    = x W_gate^T                      [N, H*dv]    (gate logits)
 *   o    = steps 1-6 above on (q, c, g)    [N, H*dv]
 *   y    = o W_o^T                         [N, D]
 *
 * Every weight is a linear layer without bias (the pages show none), laid out
 * out_features x in_features.  RMSNorm(v) = v / sqrt(mean_j v_j^2 + eps),
 * times a per-feature gain (the pages name the norm without writing it out;
 * eps is an argument).
 *
 * Storage of the stage results: the core consumes stored values, as every
 * other entry of this file does.  stage_dtype selects the activation type of
 * the layer: ORACLE_STAGE_F32 rounds each stored stage result to float32,
 * ORACLE_STAGE_BF16 to bf16 (round to nearest, ties to even).  Rounded are:
 * the two down-projections (before their norms), the norms' outputs, q, g and
 * o; y is returned unrounded.  Everything between two stores is float64.
 */
#define ORACLE_STAGE_F32 0
#define ORACLE_STAGE_BF16 1

#define BF16_MAX 3.3895313892515355e38 /* (2 - 2^-7) 2^127 */

/* Nearest bf16 value of v, ties to even.  bf16 keeps 8 significant bits and
 * float32's exponent range (quantum 2^-133 below 2^-126). */
static double round_bf16(double v) {
  if (!isfinite(v) || v == 0.0) return v;
  int e;
  const double m = frexp(v, &e); /* v = m 2^e, 0.5 <= |m| < 1 */
  const int shift = (e - 8 < -133) ? e + 133 : 8;
#if ORACLE_MUTANT == 19
  const double n = round(ldexp(m, shift)); /* planted mistake: ties away from zero */
#else
  const double n = nearbyint(ldexp(m, shift)); /* the default mode rounds ties to even */
#endif
  const double r = ldexp(n, e - shift);
  return fabs(r) > BF16_MAX ? copysign(INFINITY, v) : r;
}

static double store(double v, int stage_dtype) {
  return stage_dtype == ORACLE_STAGE_BF16 ? round_bf16(v) : (double)(float)v;
}

int oracle_round_bf16(const double* in, int64_t n, double* out) {
  if ((!in || !out) && n > 0) return ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
  return ORACLE_OK;
}

/* out[i, n] = sum_k in[i, k] W[n, k] for N outputs over K inputs (a linear
 * layer, weight [N, K]); `transposed` is only set by planted mistakes, which
 * read W as [K, N]. */
static void linear(const double* in, int64_t M, int K, const float* W, int N, int transposed,
                   double* out, int nthreads) {
#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t i = 0; i < M; ++i)
    for (int n = 0; n < N; ++n) {
      const double* xi = in + i * K;
      double acc = 0.0;
      if (transposed) {
        for (int k = 0; k < K; ++k) acc += xi[k] * (double)W[(int64_t)k * N + n];
      } else {
        const float* wn = W + (int64_t)n * K;
#pragma omp simd reduction(+ : acc)
        for (int k = 0; k < K; ++k) acc += xi[k] * (double)wn[k];
      }
      out[i * N + n] = acc;
    }
}

/* Row-wise RMSNorm with gain, in place on M rows of n features.  which: 0 for
 * the latent's norm, 1 for the query's (planted mistakes pick one). */
static void rmsnorm_rows(double* v, int64_t M, int n, const float* gain, double eps, int which) {
  for (int64_t i = 0; i < M; ++i) {
    double* row = v + i * n;
#if ORACLE_MUTANT == 13
    if (which == 0)
      for (int j = 0; j < n; ++j) row[j] *= (double)gain[j]; /* planted: gain inside the norm */
#endif
    double ss = 0.0;
    for (int j = 0; j < n; ++j) ss += row[j] * row[j];
#if ORACLE_MUTANT == 18
    const double inv = 1.0 / sqrt(ss + eps); /* planted mistake: sum instead of mean */
#else
    const double inv = 1.0 / sqrt(ss / n + eps);
#endif
#if ORACLE_MUTANT == 12
    if (which == 0) {
      for (int j = 0; j < n; ++j) row[j] *= (double)gain[j]; /* planted: latent not normalised */
      continue;
    }
#elif ORACLE_MUTANT == 14
    if (which == 1) {
      for (int j = 0; j < n; ++j) row[j] *= (double)gain[j]; /* planted: query latent not normalised */
      continue;
    }
#endif
    for (int j = 0; j < n; ++j) {
#if ORACLE_MUTANT == 13
      row[j] = which == 0 ? row[j] * inv : row[j] * inv * (double)gain[j];
#else
      row[j] = row[j] * inv * (double)gain[j];
#endif
    }
    (void)which;
  }
}

static void store_all(double* v, int64_t n, int stage_dtype) {
  for (int64_t i = 0; i < n; ++i) v[i] = store(v[i], stage_dtype);
}

/*
 * x [B,T,D]; weights as listed above; rows[] (flattened b*T + t) selects the
 * output rows (NULL: all B*T).  The latent c is formed for every position
 * (it is every query's key set); q, g, o and y only for the selected rows.
 * y: [nrows, D].  Optional stage outputs (NULL to skip): c_out [B*T, r],
 * q_out [nrows, H*dq], g_out and o_out [nrows, H*dv], all as stored.
 */
int oracle_forward(const float* x, const float* w_kv_down, const float* kv_norm, const float* w_q_down,
                   const float* q_norm, const float* w_q_up, const float* w_uk, const float* w_uv,
                   const float* w_gate, const float* w_o, int B, int T, int D, int q_rank, int H, int dq,
                   int dv, int r, double eps, double scale, int stage_dtype, const int64_t* rows,
                   int64_t nrows, double* y, double* c_out, double* q_out, double* g_out, double* o_out,
                   int nthreads) {
  if (!x || !w_kv_down || !kv_norm || !w_q_down || !q_norm || !w_q_up || !w_uk || !w_uv || !w_gate ||
      !w_o || !y)
    return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || D <= 0 || q_rank <= 0 || H <= 0 || dq <= 0 || dv <= 0 || r <= 0 || nrows < 0 ||
      !(eps >= 0.0))
    return ORACLE_EINVAL;
  if (stage_dtype != ORACLE_STAGE_F32 && stage_dtype != ORACLE_STAGE_BF16) return ORACLE_EINVAL;
  const int64_t N = (int64_t)B * T;
  if (!rows && nrows != N) return ORACLE_EINVAL;
  if (rows)
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= N) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int HQ = H * dq, HV = H * dv;

  double* xd = (double*)malloc(sizeof(double) * (size_t)N * D);
  double* xs = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * D);
  double* c = (double*)malloc(sizeof(double) * (size_t)N * r);
  double* ql = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * q_rank);
  double* q = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * HQ);
  double* g = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * HV);
  double* o = (double*)malloc(sizeof(double) * (size_t)(nrows ? nrows : 1) * HV);
  float* cf = (float*)malloc(sizeof(float) * (size_t)N * r);
  float* qf = (float*)malloc(sizeof(float) * (size_t)B * T * HQ);
  float* gf = (float*)malloc(sizeof(float) * (size_t)B * T * HV);
  int err = ORACLE_OK;
  if (!xd || !xs || !c || !ql || !q || !g || !o || !cf || !qf || !gf) {
    err = ORACLE_ENOMEM;
    goto done;
  }
  for (int64_t i = 0; i < N * D; ++i) xd[i] = (double)x[i];
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t row = rows ? rows[i] : i;
    memcpy(xs + i * D, xd + row * D, sizeof(double) * (size_t)D);
  }

  /* the latent of every position: c = RMSNorm_kv(W_kv_down x) */
  linear(xd, N, D, w_kv_down, r, 0, c, nthreads);
  store_all(c, N * r, stage_dtype);
  rmsnorm_rows(c, N, r, kv_norm, eps, 0);
  store_all(c, N * r, stage_dtype);

  /* the query low-rank path of the selected rows: q = W_q_up RMSNorm_q(W_q_down x) */
  linear(xs, nrows, D, w_q_down, q_rank, 0, ql, nthreads);
  store_all(ql, nrows * q_rank, stage_dtype);
  rmsnorm_rows(ql, nrows, q_rank, q_norm, eps, 1);
  store_all(ql, nrows * q_rank, stage_dtype);
#if ORACLE_MUTANT == 15
  linear(ql, nrows, q_rank, w_q_up, HQ, 1, q, nthreads); /* planted: W_q_up read transposed */
#else
  linear(ql, nrows, q_rank, w_q_up, HQ, 0, q, nthreads);
#endif
  store_all(q, nrows * HQ, stage_dtype);

  /* gate logits of the selected rows */
#if ORACLE_MUTANT == 16
  linear(xs, nrows, D, w_gate, HV, 1, g, nthreads); /* planted: W_gate read transposed */
#else
  linear(xs, nrows, D, w_gate, HV, 0, g, nthreads);
#endif
  store_all(g, nrows * HV, stage_dtype);

  /* the core on the stored values; rows that were not selected stay zero */
  for (int64_t i = 0; i < N * r; ++i) cf[i] = (float)c[i];
  memset(qf, 0, sizeof(float) * (size_t)N * HQ);
  memset(gf, 0, sizeof(float) * (size_t)N * HV);
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t row = rows ? rows[i] : i;
    for (int k = 0; k < HQ; ++k) qf[row * HQ + k] = (float)q[i * HQ + k];
    for (int k = 0; k < HV; ++k) gf[row * HV + k] = (float)g[i * HV + k];
  }
  err = oracle_extend(qf, cf, w_uk, w_uv, gf, B, T, T, H, dq, dv, r, scale, rows, nrows, o, nthreads);
  if (err != ORACLE_OK) goto done;
  store_all(o, nrows * HV, stage_dtype);

  /* output projection */
#if ORACLE_MUTANT == 17
  linear(o, nrows, HV, w_o, D, 1, y, nthreads); /* planted: W_o read transposed */
#else
  linear(o, nrows, HV, w_o, D, 0, y, nthreads);
#endif

  if (c_out) memcpy(c_out, c, sizeof(double) * (size_t)N * r);
  if (q_out) memcpy(q_out, q, sizeof(double) * (size_t)nrows * HQ);
  if (g_out) memcpy(g_out, g, sizeof(double) * (size_t)nrows * HV);
  if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)nrows * HV);
done:
  free(xd);
  free(xs);
  free(c);
  free(ql);
  free(q);
  free(g);
  free(o);
  free(cf);
  free(qf);
  free(gf);
  return err;
}

/* ---------------------------------------------------------------------------
 * Backward of the absorbed core (prefill).  The pages train the model with a
 * cross-entropy loss and backpropagation ([MLA] describes only the forward);
 * the gradients below are the chain rule applied to steps 1-6 above, for
 * every batch b and head h (a_t = q_t W_UK[h] is the absorbed query, S the
 * scaled scores, P the causal softmax, ol_t the latent output, o_t = W_UV[h]
 * ol_t and out_t = sigmoid(g_t) o_t), given dout = dLoss/dout:
 *
 *   dg_t    = dout_t * o_t * s (1 - s),  s = sigmoid(g_t)
 *   do_t    = dout_t * s
 *   dW_UV  += do_t ol_t^T
 *   dol_t   = W_UV^T do_t
 *   dP_ts   = dol_t . c_s                         (s <= t)
 *   dS_ts   = P_ts (dP_ts - sum_u P_tu dP_tu)
 *   da_t    = scale sum_s dS_ts c_s
 *   dc_s   += scale dS_ts a_t + P_ts dol_t        (c is both key and value)
 *   dq_t    = W_UK da_t
 *   dW_UK  += q_t da_t^T
 *
 * Weight gradients and dc sum over batches and heads.  Everything is
 * float64; outputs: dq [B,T,H,dq], dc [B,T,r], dw_uk [H,dq,r], dw_uv [H,dv,r],
 * dgate [B,T,H*dv].
 */
int oracle_prefill_backward(const float* q, const float* c, const float* w_uk, const float* w_uv,
                            const float* gate, const float* dout, int B, int T, int H, int dq, int dv, int r,
                            double scale, double* dq_out, double* dc_out, double* dwuk_out, double* dwuv_out,
                            double* dgate_out, int nthreads) {
  if (!q || !c || !w_uk || !w_uv || !gate || !dout || !dq_out || !dc_out || !dwuk_out || !dwuv_out || !dgate_out)
    return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || H <= 0 || dq <= 0 || dv <= 0 || r <= 0) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t ndc = (int64_t)B * T * r, nwk = (int64_t)H * dq * r, nwv = (int64_t)H * dv * r;
  memset(dc_out, 0, sizeof(double) * (size_t)ndc);
  memset(dwuk_out, 0, sizeof(double) * (size_t)nwk);
  memset(dwuv_out, 0, sizeof(double) * (size_t)nwv);
  int err = ORACLE_OK;
#pragma omp parallel num_threads(nthreads)
  {
    /* private accumulators for the sums over (b, h) */
    double* dc_p = (double*)calloc((size_t)ndc, sizeof(double));
    double* wk_p = (double*)calloc((size_t)nwk, sizeof(double));
    double* wv_p = (double*)calloc((size_t)nwv, sizeof(double));
    double* a = (double*)malloc(sizeof(double) * (size_t)T * r);
    double* P = (double*)malloc(sizeof(double) * (size_t)T);
    double* dS = (double*)malloc(sizeof(double) * (size_t)T);
    double* ol = (double*)malloc(sizeof(double) * (size_t)r);
    double* dol = (double*)malloc(sizeof(double) * (size_t)r);
    double* da = (double*)malloc(sizeof(double) * (size_t)r);
    double* dov = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!dc_p || !wk_p || !wv_p || !a || !P || !dS || !ol || !dol || !da || !dov) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    }
#pragma omp barrier
    if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const float* wk = w_uk + h * (int64_t)dq * r;
        const float* wv = w_uv + h * (int64_t)dv * r;
        const float* cb = c + b * (int64_t)T * r;
        for (int t = 0; t < T; ++t)
          absorb_row(q + ((b * T + t) * H + h) * dq, wk, dq, r, a + (int64_t)t * r);
        for (int t = 0; t < T; ++t) {
          const double* at = a + (int64_t)t * r;
          const int64_t row = b * T + t;
          /* forward quantities of row t */
          double m = -INFINITY;
          for (int s = 0; s <= t; ++s) {
            double acc = 0.0;
            for (int j = 0; j < r; ++j) acc += at[j] * (double)cb[(int64_t)s * r + j];
            P[s] = scale * acc;
            m = P[s] > m ? P[s] : m;
          }
          double z = 0.0;
          for (int s = 0; s <= t; ++s) {
            P[s] = exp(P[s] - m);
            z += P[s];
          }
          for (int s = 0; s <= t; ++s) P[s] /= z;
          for (int j = 0; j < r; ++j) ol[j] = 0.0;
          for (int s = 0; s <= t; ++s)
            for (int j = 0; j < r; ++j) ol[j] += P[s] * (double)cb[(int64_t)s * r + j];
          /* gate, output and W_UV */
          for (int v = 0; v < dv; ++v) {
            double o = 0.0;
            for (int j = 0; j < r; ++j) o += (double)wv[(int64_t)v * r + j] * ol[j];
            const int64_t col = row * H * dv + h * dv + v;
            const double sg = 1.0 / (1.0 + exp(-(double)gate[col]));
            const double g = (double)dout[col];
#if ORACLE_MUTANT == 24
            dgate_out[col] = g * o * sg; /* planted mistake: sigmoid instead of its derivative */
#else
            dgate_out[col] = g * o * sg * (1.0 - sg);
#endif
            dov[v] = g * sg;
            for (int j = 0; j < r; ++j) wv_p[(h * dv + v) * (int64_t)r + j] += dov[v] * ol[j];
          }
          for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int v = 0; v < dv; ++v) acc += (double)wv[(int64_t)v * r + j] * dov[v];
            dol[j] = acc;
          }
          /* softmax backward */
          double D = 0.0;
          for (int s = 0; s <= t; ++s) {
            double acc = 0.0;
            for (int j = 0; j < r; ++j) acc += dol[j] * (double)cb[(int64_t)s * r + j];
            dS[s] = acc; /* dP for now */
            D += P[s] * acc;
          }
          for (int s = 0; s <= t; ++s) {
#if ORACLE_MUTANT == 22
            dS[s] = P[s] * dS[s]; /* planted mistake: the row term of the softmax Jacobian dropped */
#else
            dS[s] = P[s] * (dS[s] - D);
#endif
          }
          /* query side */
          for (int j = 0; j < r; ++j) da[j] = 0.0;
          for (int s = 0; s <= t; ++s)
            for (int j = 0; j < r; ++j) da[j] += dS[s] * (double)cb[(int64_t)s * r + j];
#if ORACLE_MUTANT != 25
          for (int j = 0; j < r; ++j) da[j] *= scale;
#endif
          /* (mutant 25 plants a missing scale on the query-side gradient) */
          for (int d = 0; d < dq; ++d) {
            double acc = 0.0;
            for (int j = 0; j < r; ++j) acc += (double)wk[(int64_t)d * r + j] * da[j];
            dq_out[((b * T + t) * H + h) * dq + d] = acc;
            const double qd = (double)q[((b * T + t) * H + h) * dq + d];
            for (int j = 0; j < r; ++j) wk_p[(h * dq + d) * (int64_t)r + j] += qd * da[j];
          }
          /* key and value side: c enters as both */
          for (int s = 0; s <= t; ++s) {
            double* dcs = dc_p + (b * T + s) * (int64_t)r;
            for (int j = 0; j < r; ++j) {
#if ORACLE_MUTANT == 23
              dcs[j] += scale * dS[s] * at[j]; /* planted mistake: the value path of c dropped */
#else
              dcs[j] += scale * dS[s] * at[j] + P[s] * dol[j];
#endif
            }
          }
        }
      }
#pragma omp critical
      {
        for (int64_t i = 0; i < ndc; ++i) dc_out[i] += dc_p[i];
        for (int64_t i = 0; i < nwk; ++i) dwuk_out[i] += wk_p[i];
        for (int64_t i = 0; i < nwv; ++i) dwuv_out[i] += wv_p[i];
      }
    }
    free(dc_p);
    free(wk_p);
    free(wv_p);
    free(a);
    free(P);
    free(dS);
    free(ol);
    free(dol);
    free(da);
    free(dov);
  }
  return err;
}

/* Log-sum-exp of each causal score row, natural log: lse[b,h,t] =
 * log sum_{s<=t} exp(scale * a_t . c_s) with a_t = q_t W_UK[h], the
 * normaliser of step 3's softmax (what a training forward keeps for its
 * backward).  Max-subtracted, float64. */
int oracle_prefill_lse(const float* q, const float* c, const float* w_uk, int B, int T, int H, int dq, int r,
                       double scale, double* lse, int nthreads) {
  if (!q || !c || !w_uk || !lse || B <= 0 || T <= 0 || H <= 0 || dq <= 0 || r <= 0) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  int err = ORACLE_OK;
#pragma omp parallel num_threads(nthreads)
  {
    double* qa = (double*)malloc(sizeof(double) * (size_t)r);
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    if (!qa || !s) {
#pragma omp atomic write
      err = ORACLE_ENOMEM;
    }
#pragma omp barrier
    if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bht = 0; bht < (int64_t)B * H * T; ++bht) {
        const int64_t b = bht / ((int64_t)H * T), h = (bht / T) % H, t = bht % T;
        absorb_row(q + ((b * T + t) * H + h) * dq, w_uk + h * (int64_t)dq * r, dq, r, qa);
        double m = -INFINITY;
        for (int64_t u = 0; u <= t; ++u) {
          const float* cu = c + (b * T + u) * (int64_t)r;
          double acc = 0.0;
          for (int j = 0; j < r; ++j) acc += qa[j] * (double)cu[j];
          s[u] = scale * acc;
          m = s[u] > m ? s[u] : m;
        }
        double z = 0.0;
        for (int64_t u = 0; u <= t; ++u) z += exp(s[u] - m);
        lse[bht] = m + log(z);
      }
    }
    free(qa);
    free(s);
  }
  return err;
}

/* ---------------------------------------------------------------------------
 * Backward of the full Gated MLA layer (the forward of oracle_forward, stage
 * results stored as float32), given dy = dLoss/dy [B,T,D]: the chain rule
 * through the output projection, the core (oracle_prefill_backward), the gate
 * projection, the query up- and down-projections with the query norm, and the
 * latent down-projection with the latent norm.  For RMSNorm
 * u = g * v / rms(v), rms = sqrt(mean(v^2) + eps):
 *   dg   = sum over rows of du * v / rms
 *   dv_i = (du_i g_i - n_i * mean_j(du_j g_j n_j)) / rms,   n = v / rms
 * Outputs (float64): dx [B,T,D], dw_kv_down [r,D], dkv_norm [r],
 * dw_q_down [q_rank,D], dq_norm [q_rank], dw_q_up [H*dq,q_rank],
 * dw_uk [H,dq,r], dw_uv [H,dv,r], dw_gate [H*dv,D], dw_o [D,H*dv].
 */
static void rmsnorm_backward(const double* pre, int64_t M, int n, const float* gain, double eps,
                             const double* du, double* dpre, double* dgain) {
  for (int j = 0; j < n; ++j) dgain[j] = 0.0;
  for (int64_t i = 0; i < M; ++i) {
    const double* v = pre + i * n;
    const double* g_ = du + i * n;
    double ss = 0.0;
    for (int j = 0; j < n; ++j) ss += v[j] * v[j];
    const double rms = sqrt(ss / n + eps);
    double dot = 0.0;
    for (int j = 0; j < n; ++j) {
      const double nj = v[j] / rms;
      dgain[j] += g_[j] * nj;
      dot += g_[j] * (double)gain[j] * nj;
    }
    dot /= n;
    for (int j = 0; j < n; ++j) {
#if ORACLE_MUTANT == 27
      dpre[i * n + j] = g_[j] * (double)gain[j] / rms; /* planted mistake: the norm's projection term dropped */
#else
      dpre[i * n + j] = (g_[j] * (double)gain[j] - (v[j] / rms) * dot) / rms;
#endif
    }
  }
}

/* out[i, k] += sum_n g[i, n] W[n, k] (input gradient of a linear layer, weight [N, K]) */
static void linear_dx(const double* g, int64_t M, int N, const float* W, int K, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int n = 0; n < N; ++n) {
      const double gi = g[i * N + n];
      if (gi == 0.0) continue;
      const float* wn = W + (int64_t)n * K;
      for (int k = 0; k < K; ++k) out[i * K + k] += gi * (double)wn[k];
    }
}

/* dW[n, k] = sum_i g[i, n] in[i, k] (weight gradient of a linear layer) */
static void linear_dw(const double* g, int64_t M, int N, const double* in, int K, double* dW) {
  memset(dW, 0, sizeof(double) * (size_t)N * K);
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int64_t i = 0; i < M; ++i) {
      const double gi = g[i * N + n];
      if (gi == 0.0) continue;
      for (int k = 0; k < K; ++k) dW[(int64_t)n * K + k] += gi * in[i * K + k];
    }
}

int oracle_forward_backward(const float* x, const float* w_kv_down, const float* kv_norm, const float* w_q_down,
                            const float* q_norm, const float* w_q_up, const float* w_uk, const float* w_uv,
                            const float* w_gate, const float* w_o, const float* dy, int B, int T, int D, int q_rank,
                            int H, int dq, int dv, int r, double eps, double scale, double* dx, double* dw_kv_down,
                            double* dkv_norm, double* dw_q_down, double* dq_norm, double* dw_q_up, double* dw_uk,
                            double* dw_uv, double* dw_gate, double* dw_o, int nthreads) {
  if (!x || !w_kv_down || !kv_norm || !w_q_down || !q_norm || !w_q_up || !w_uk || !w_uv || !w_gate || !w_o || !dy ||
      !dx || !dw_kv_down || !dkv_norm || !dw_q_down || !dq_norm || !dw_q_up || !dw_uk || !dw_uv || !dw_gate || !dw_o)
    return ORACLE_EINVAL;
  if (B <= 0 || T <= 0 || D <= 0 || q_rank <= 0 || H <= 0 || dq <= 0 || dv <= 0 || r <= 0 || !(eps >= 0.0))
    return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t N = (int64_t)B * T;
  const int HQ = H * dq, HV = H * dv;
  double* xd = (double*)malloc(sizeof(double) * (size_t)N * D);
  double* c_pre = (double*)malloc(sizeof(double) * (size_t)N * r);
  double* c = (double*)malloc(sizeof(double) * (size_t)N * r);
  double* ql_pre = (double*)malloc(sizeof(double) * (size_t)N * q_rank);
  double* ql = (double*)malloc(sizeof(double) * (size_t)N * q_rank);
  double* q = (double*)malloc(sizeof(double) * (size_t)N * HQ);
  double* g = (double*)malloc(sizeof(double) * (size_t)N * HV);
  double* o = (double*)malloc(sizeof(double) * (size_t)N * HV);
  double* dyd = (double*)malloc(sizeof(double) * (size_t)N * D);
  double* dout = (double*)malloc(sizeof(double) * (size_t)N * HV);
  float* qf = (float*)malloc(sizeof(float) * (size_t)N * HQ);
  float* cf = (float*)malloc(sizeof(float) * (size_t)N * r);
  float* gf = (float*)malloc(sizeof(float) * (size_t)N * HV);
  float* doutf = (float*)malloc(sizeof(float) * (size_t)N * HV);
  double* dqv = (double*)malloc(sizeof(double) * (size_t)N * HQ);
  double* dcv = (double*)malloc(sizeof(double) * (size_t)N * r);
  double* dgv = (double*)malloc(sizeof(double) * (size_t)N * HV);
  double* dql = (double*)malloc(sizeof(double) * (size_t)N * q_rank);
  double* dql_pre = (double*)malloc(sizeof(double) * (size_t)N * q_rank);
  double* dc_pre = (double*)malloc(sizeof(double) * (size_t)N * r);
  int err = ORACLE_OK;
  if (!xd || !c_pre || !c || !ql_pre || !ql || !q || !g || !o || !dyd || !dout || !qf || !cf || !gf || !doutf || !dqv ||
      !dcv || !dgv || !dql || !dql_pre || !dc_pre) {
    err = ORACLE_ENOMEM;
    goto done;
  }
  for (int64_t i = 0; i < N * D; ++i) {
    xd[i] = (double)x[i];
    dyd[i] = (double)dy[i];
  }
  /* forward stages, stored as float32 as oracle_forward does */
  linear(xd, N, D, w_kv_down, r, 0, c_pre, nthreads);
  store_all(c_pre, N * r, ORACLE_STAGE_F32);
  memcpy(c, c_pre, sizeof(double) * (size_t)N * r);
  rmsnorm_rows(c, N, r, kv_norm, eps, 0);
  store_all(c, N * r, ORACLE_STAGE_F32);
  linear(xd, N, D, w_q_down, q_rank, 0, ql_pre, nthreads);
  store_all(ql_pre, N * q_rank, ORACLE_STAGE_F32);
  memcpy(ql, ql_pre, sizeof(double) * (size_t)N * q_rank);
  rmsnorm_rows(ql, N, q_rank, q_norm, eps, 1);
  store_all(ql, N * q_rank, ORACLE_STAGE_F32);
  linear(ql, N, q_rank, w_q_up, HQ, 0, q, nthreads);
  store_all(q, N * HQ, ORACLE_STAGE_F32);
  linear(xd, N, D, w_gate, HV, 0, g, nthreads);
  store_all(g, N * HV, ORACLE_STAGE_F32);
  for (int64_t i = 0; i < N * HQ; ++i) qf[i] = (float)q[i];
  for (int64_t i = 0; i < N * r; ++i) cf[i] = (float)c[i];
  for (int64_t i = 0; i < N * HV; ++i) gf[i] = (float)g[i];
  err = oracle_extend(qf, cf, w_uk, w_uv, gf, B, T, T, H, dq, dv, r, scale, NULL, N, o, nthreads);
  if (err != ORACLE_OK) goto done;
  store_all(o, N * HV, ORACLE_STAGE_F32);

  /* output projection y = o W_o^T */
  linear_dw(dyd, N, D, o, HV, dw_o);
  memset(dout, 0, sizeof(double) * (size_t)N * HV);
  linear_dx(dyd, N, D, w_o, HV, dout);
  /* the core */
  for (int64_t i = 0; i < N * HV; ++i) doutf[i] = (float)dout[i];
  err = oracle_prefill_backward(qf, cf, w_uk, w_uv, gf, doutf, B, T, H, dq, dv, r, scale, dqv, dcv, dw_uk, dw_uv, dgv,
                                nthreads);
  if (err != ORACLE_OK) goto done;
  /* gate projection */
  memset(dx, 0, sizeof(double) * (size_t)N * D);
  linear_dw(dgv, N, HV, xd, D, dw_gate);
  linear_dx(dgv, N, HV, w_gate, D, dx);
  /* query path */
  linear_dw(dqv, N, HQ, ql, q_rank, dw_q_up);
  memset(dql, 0, sizeof(double) * (size_t)N * q_rank);
  linear_dx(dqv, N, HQ, w_q_up, q_rank, dql);
  rmsnorm_backward(ql_pre, N, q_rank, q_norm, eps, dql, dql_pre, dq_norm);
  linear_dw(dql_pre, N, q_rank, xd, D, dw_q_down);
#if ORACLE_MUTANT != 28
  linear_dx(dql_pre, N, q_rank, w_q_down, D, dx);
#endif
  /* (mutant 28 plants an input gradient without the query path) */
  /* latent path */
  rmsnorm_backward(c_pre, N, r, kv_norm, eps, dcv, dc_pre, dkv_norm);
  linear_dw(dc_pre, N, r, xd, D, dw_kv_down);
  linear_dx(dc_pre, N, r, w_kv_down, D, dx);
done:
  free(xd); free(c_pre); free(c); free(ql_pre); free(ql); free(q); free(g); free(o); free(dyd); free(dout);
  free(qf); free(cf); free(gf); free(doutf); free(dqv); free(dcv); free(dgv); free(dql); free(dql_pre); free(dc_pre);
  return err;
}

/* ---------------------------------------------------------------------------
 * chunk_kda's recurrence (page "符号表": section KDA 变量 for the variables
 * and section Einsum 速查 for the three contractions; the summary list on the
 * same page states that the chunked form equals this step-by-step one).  Per
 * batch b and value head hv (query/key head hv / G, the GVA expansion), with
 * the state S [K, V] starting at S0 (zero when s0 is NULL), for t = 0..T-1:
 *   S_dec = diag(exp(g_t)) S          decay per key channel (log-space g)
 *   p_t   = k_t^T S_dec               the old state's prediction for k_t
 *   r_t   = v_t - p_t                 delta-rule residual
 *   a_t   = beta_t k_t                write vector
 *   S     = S_dec + a_t r_t^T         outer-product write
 *   o_t   = q_t^T S                   read-out after the write
 * Layouts: q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K]; beta [B,T,HV];
 * s0 and s_out [B,HV,K,V]; o [B,T,HV,V]; HV = G H.  float64 throughout.
 */
int oracle_kda(const float* q, const float* k, const float* v, const float* g, const float* beta, const float* s0,
               int B, int T, int H, int G, int K, int V, double* o, double* s_out, int nthreads) {
  if (!q || !k || !v || !g || !beta || !o) return ORACLE_EINVAL;
  if (B <= 0 || T < 0 || H <= 0 || G <= 0 || K <= 0 || V <= 0) return ORACLE_EINVAL;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int HV = G * H;
  int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t bh = 0; bh < (int64_t)B * HV; ++bh) {
    const int64_t b = bh / HV;
    const int hv = (int)(bh % HV);
#if ORACLE_MUTANT == 33
    const int h = hv % H; /* planted mistake: GVA heads interleaved instead of repeated */
#else
    const int h = hv / G;
#endif
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    if (!S || !p) {
      free(S);
      free(p);
#pragma omp atomic write
      err = ORACLE_ENOMEM;
      continue;
    }
    for (int64_t i = 0; i < (int64_t)K * V; ++i) S[i] = s0 ? (double)s0[bh * K * V + i] : 0.0;
    for (int t = 0; t < T; ++t) {
      const float* qt = q + ((b * T + t) * H + h) * (int64_t)K;
      const float* kt = k + ((b * T + t) * H + h) * (int64_t)K;
      const float* vt = v + ((b * T + t) * HV + hv) * (int64_t)V;
      const float* gt = g + ((b * T + t) * HV + hv) * (int64_t)K;
      const double bt = (double)beta[(b * T + t) * HV + hv];
#if ORACLE_MUTANT != 29
      for (int i = 0; i < K; ++i) {
#if ORACLE_MUTANT == 32
        const double dcy = exp(-(double)gt[i]); /* planted mistake: decay sign flipped */
#else
        const double dcy = exp((double)gt[i]);
#endif
        for (int j = 0; j < V; ++j) S[i * V + j] *= dcy;
      }
#endif
      double* ot = o + ((b * T + t) * HV + hv) * (int64_t)V;
#if ORACLE_MUTANT == 30
      for (int j = 0; j < V; ++j) { /* planted mistake: read-out before the write */
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += (double)qt[i] * S[i * V + j];
        ot[j] = acc;
      }
#endif
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += (double)kt[i] * S[i * V + j];
        p[j] = acc;
      }
      for (int i = 0; i < K; ++i) {
#if ORACLE_MUTANT == 31
        const double ai = (double)kt[i]; /* planted mistake: write strength ignored */
#else
        const double ai = bt * (double)kt[i];
#endif
        for (int j = 0; j < V; ++j) S[i * V + j] += ai * ((double)vt[j] - p[j]);
      }
#if ORACLE_MUTANT == 29
      for (int i = 0; i < K; ++i) { /* planted mistake: decay after the write */
        const double dcy = exp((double)gt[i]);
        for (int j = 0; j < V; ++j) S[i * V + j] *= dcy;
      }
#endif
#if ORACLE_MUTANT != 30
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += (double)qt[i] * S[i * V + j];
        ot[j] = acc;
      }
#endif
    }
    if (s_out)
      for (int64_t i = 0; i < (int64_t)K * V; ++i) s_out[bh * K * V + i] = S[i];
    free(S);
    free(p);
  }
  return err;
}
