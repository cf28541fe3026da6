/*
 * sdpa_oracle.c -- plain fp64 CPU reference for scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py load this library.  It shares no code, header,
 * table or helper with the HIP library under flash_attention_head_amd/, and the
 * product path never calls it.
 *
 * What it computes is the plain definition of attention that the fused
 * kernels must reproduce: the "unfused" matmul + softmax + matmul path that
 * ml-explore/mlx PR #3293 ("fix: add head_dim=256 to fused SDPA full attention
 * kernel", Benchmark section) times against the fused kernel, and whose
 * outputs ml-explore/mlx PR #3660 ("Fused SDPA full-attention for
 * head_dim=192/256", Microbenchmarks and Validation) reports the fused kernel
 * reproduces.  For one query row it
 *   1. takes the scores s_j = scale * <q, k_j> over the keys the row may see,
 *   2. subtracts their maximum and exponentiates (base e),
 *   3. normalises by the sum of the exponentials,
 *   4. returns the weighted sum of the value rows.
 * Nothing is blocked, fused or reordered beyond that: each row is three
 * straight passes over its allowed keys, in ascending key order, in double.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes):
 *   - layout: Q and O are [B, Hq, qL, D], K and V are [B, Hkv, kL, D], rows
 *     contiguous, as in the (B, H, L, D) arrays of the M3 Ultra test script
 *     in mlx PR #3293;
 *   - grouped-query heads: query head hq reads KV head hq / (Hq / Hkv), i.e.
 *     contiguous groups (n_q=16 over n_kv=8 in the mlx PR #3660
 *     Microbenchmarks table);
 *   - query row i sits at absolute position p = q_offset + i, so a chunk of
 *     queries can be aligned to the end of a longer key prefix (chunked
 *     prefill over a prefix cache, mlx PR #3660 End-to-end section; a verify
 *     row attends its own trimmed prefix, mlxcel issue #2160 Proposed
 *     Solution step 2);
 *   - causal: key j is visible iff j <= p; window w > 0: also p - j < w, so
 *     the window counts w keys including the row's own (the causal/windowed
 *     mask of mlxcel issue #672 Root cause; window 1024 in mlxcel issue #2160
 *     Current Behavior);
 *   - a masked key is excluded outright (weight exactly zero), never given a
 *     large finite negative score;
 *   - inputs are the exact fp16/bf16 bit patterns, widened exactly; scale is
 *     the fp32 value the caller passes, widened exactly;
 *   - an optional additive mask array ("bias") is added to the scaled score,
 *     s_j = scale * <q, k_j> + bias[b, hq, i, j] (the array mask that
 *     lablup/mlxcel issue #672, Root cause, hands to SDPA and that the cuDNN
 *     path takes as a bias); it has the input dtype, and keys are contiguous
 *     within a bias row, its batch, head and row strides are given (0 for a
 *     broadcast dimension).  A key whose biased score is -inf is excluded
 *     like a masked key; a row with no finite score is a zero row.  The
 *     causal and window rules still apply on top;
 *   - the value rows may be longer than the query/key rows (Dv != D: the
 *     Q=192/K=192/V=256 heads named in the review discussion of mlx PR
 *     #3293): the scores take the D-long dot products, the output row is the
 *     weighted sum of the Dv-long value rows, V is [B, Hkv, kL, Dv] and the
 *     output [B, Hq, qL, Dv];
 *   - K and V may instead be 4-bit quantized (the prefix KV cache kept 4-bit
 *     at rest in the End-to-end section of mlx PR #3660; the pages give no
 *     format, so the affine, group-64 form that mlxcel issue #2160 names for
 *     its checkpoints is read as the plain one): the head dim of each key and
 *     value row splits into groups of 64 consecutive elements, each with a
 *     scale and a bias in the input dtype, and element d of a row is
 *     scale[d / 64] * c_d + bias[d / 64] with its 4-bit code c_d in 0..15.
 *     The codes of a row are packed eight to a 32-bit word, element 8w + n
 *     in bits 4n .. 4n + 3 of word w.  The oracle dequantizes each element in
 *     double and runs the same three passes on those values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_FP16 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one IEEE binary16 bit pattern. */
static double widen_fp16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac + 1024), expo - 25); /* (1.frac) * 2^(e-15) */
  }
  return sign ? -mag : mag;
}

/* Exact widening of one bfloat16 bit pattern: it is the top half of a float. */
static double widen_bf16(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double widen(uint16_t h, int dtype) {
  return dtype == ORACLE_BF16 ? widen_bf16(h) : widen_fp16(h);
}

typedef struct {
  const uint16_t *q, *k, *v;
  /* 4-bit K and V (NULL: k and v hold the fp16/bf16 rows): codes [B, Hkv,
   * kL, D / 8] words, scales and biases [B, Hkv, kL, D / 64] */
  const uint32_t *kq, *vq;
  const uint16_t *ks, *kb, *vs, *vb;
  const uint16_t *bias; /* NULL: none */
  int64_t bias_sb, bias_sh, bias_sq;
  int B, Hq, Hkv, qL, kL, D, Dv; /* D: q and k rows; Dv: v and output rows */
  double scale;
  int causal, window, q_offset, dtype;
} problem_t;

/* Element d of a 4-bit row: its code, times its group's scale, plus the
 * group's bias.  `row` is the row's index among all [B, Hkv, kL] rows. */
static double dequant4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                       long row, long D, long d, int dtype) {
  const uint32_t word = codes[row * (D / 8) + d / 8];
  const unsigned c = (word >> (4 * (d % 8))) & 0xfu;
  const long g = row * (D / 64) + d / 64;
  return widen(scales[g], dtype) * (double)c + widen(biases[g], dtype);
}

/* Element d of key row / value row `row` (an index among all [B, Hkv, kL] rows). */
static double key_elem(const problem_t *pr, long row, long d) {
  if (pr->kq) return dequant4(pr->kq, pr->ks, pr->kb, row, pr->D, d, pr->dtype);
  return widen(pr->k[row * pr->D + d], pr->dtype);
}
static double value_elem(const problem_t *pr, long row, long d) {
  if (pr->vq) return dequant4(pr->vq, pr->vs, pr->vb, row, pr->Dv, d, pr->dtype);
  return widen(pr->v[row * pr->Dv + d], pr->dtype);
}

/* Is key j visible from absolute query position p? */
static int key_visible(const problem_t *pr, long p, long j) {
  if (pr->causal && j > p) return 0;
  if (pr->window > 0 && p - j >= pr->window) return 0;
  return 1;
}

/*
 * One output row.  `row` is the flat index (b * Hq + hq) * qL + i.
 * `s` is caller scratch of kL + D doubles.  Writes Dv doubles to `o`.
 */
static void attend_row(const problem_t *pr, long row, double *s, double *o) {
  const long D = pr->D, Dv = pr->Dv;
  const long i = row % pr->qL;
  const long bh = row / pr->qL;
  const long hq = bh % pr->Hq;
  const long b = bh / pr->Hq;
  const long group = pr->Hq / pr->Hkv;
  const long hk = hq / group;
  const long p = (long)pr->q_offset + i;

  const uint16_t *qrow = pr->q + row * D;
  const long kvrow0 = (b * pr->Hkv + hk) * (long)pr->kL; /* the head's first K/V row */

  double *qd = s + pr->kL; /* the widened query row */
  for (long d = 0; d < D; ++d) qd[d] = widen(qrow[d], pr->dtype);
  const uint16_t *brow = pr->bias ? pr->bias + b * pr->bias_sb + hq * pr->bias_sh + i * pr->bias_sq : NULL;

  /* pass 1: scores of the visible keys (plus the bias), and their maximum;
   * a key whose score is -inf takes no part from here on */
  int any = 0;
  double m = -INFINITY;
  for (long j = 0; j < pr->kL; ++j) {
    if (!key_visible(pr, p, j)) continue;
    double dot = 0.0;
    for (long d = 0; d < D; ++d) dot += qd[d] * key_elem(pr, kvrow0 + j, d);
    s[j] = pr->scale * dot;
    if (brow) s[j] += widen(brow[j], pr->dtype);
    if (s[j] == -INFINITY) continue;
    if (!any || s[j] > m) m = s[j];
    any = 1;
  }
  for (long d = 0; d < Dv; ++d) o[d] = 0.0;
  if (!any) return; /* no visible key with a finite score: defined as a zero row */

  /* pass 2: exponentials relative to the maximum, and their sum */
  double l = 0.0;
  for (long j = 0; j < pr->kL; ++j) {
    if (!key_visible(pr, p, j) || s[j] == -INFINITY) continue;
    s[j] = exp(s[j] - m);
    l += s[j];
  }

  /* pass 3: weighted sum of value rows, then normalise */
  for (long j = 0; j < pr->kL; ++j) {
    if (!key_visible(pr, p, j) || s[j] == -INFINITY) continue;
    for (long d = 0; d < Dv; ++d) o[d] += s[j] * value_elem(pr, kvrow0 + j, d);
  }
  for (long d = 0; d < Dv; ++d) o[d] /= l;
}

typedef struct {
  const problem_t *pr;
  const int64_t *rows; /* NULL: all rows */
  int64_t nrows;
  double *out;
  int64_t first, stride; /* this worker takes rows first, first+stride, ... */
  int failed;
} work_t;

static void *worker(void *arg) {
  work_t *w = (work_t *)arg;
  double *s = (double *)malloc(sizeof(double) * ((size_t)w->pr->kL + (size_t)w->pr->D));
  if (!s) {
    w->failed = 1;
    return NULL;
  }
  for (int64_t n = w->first; n < w->nrows; n += w->stride) {
    long row = w->rows ? (long)w->rows[n] : (long)n;
    attend_row(w->pr, row, s, w->out + n * (int64_t)w->pr->Dv);
  }
  free(s);
  return NULL;
}

static int run(const problem_t *pr, const int64_t *rows, int64_t nrows, double *out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 512) nthreads = 512;
  if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
  pthread_t tid[512];
  work_t w[512];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    w[t].pr = pr;
    w[t].rows = rows;
    w[t].nrows = nrows;
    w[t].out = out;
    w[t].first = t;
    w[t].stride = nthreads;
    w[t].failed = 0;
    if (t == 0) continue;
    if (pthread_create(&tid[t], NULL, worker, &w[t]) != 0) {
      rc = -2;
      break;
    }
    started = t;
  }
  if (rc == 0) worker(&w[0]);
  for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
  for (int t = 0; t < nthreads && rc == 0; ++t)
    if (w[t].failed) rc = -3;
  return rc;
}

static int make_problem(problem_t *pr, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int B, int Hq, int Hkv, int qL, int kL, int D, float scale, int causal,
                        int window, int q_offset, int dtype) {
  if (!q || !k || !v) return -1;
  if (B < 1 || Hq < 1 || Hkv < 1 || qL < 1 || kL < 1 || D < 1) return -1;
  if (Hq % Hkv != 0) return -1;
  if (dtype != ORACLE_FP16 && dtype != ORACLE_BF16) return -1;
  pr->q = q;
  pr->k = k;
  pr->v = v;
  pr->kq = pr->vq = NULL;
  pr->ks = pr->kb = pr->vs = pr->vb = NULL;
  pr->bias = NULL;
  pr->bias_sb = pr->bias_sh = pr->bias_sq = 0;
  pr->B = B;
  pr->Hq = Hq;
  pr->Hkv = Hkv;
  pr->qL = qL;
  pr->kL = kL;
  pr->D = D;
  pr->Dv = D;
  pr->scale = (double)scale;
  pr->causal = causal;
  pr->window = window;
  pr->q_offset = q_offset;
  pr->dtype = dtype;
  return 0;
}

/* Every output row: out is [B, Hq, qL, D] doubles.  Returns 0 on success. */
int oracle_sdpa_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *out, int B,
                    int Hq, int Hkv, int qL, int kL, int D, float scale, int causal, int window,
                    int q_offset, int dtype, int nthreads) {
  problem_t pr;
  if (!out || make_problem(&pr, q, k, v, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset,
                           dtype))
    return -1;
  return run(&pr, NULL, (int64_t)B * Hq * qL, out, nthreads);
}

/*
 * Selected rows only: rows[n] is the flat row index (b * Hq + hq) * qL + i,
 * out is [nrows, D] doubles.  Used where a full-size problem is too large for
 * every row to be computed on the host.
 */
int oracle_sdpa_rows_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *out,
                         int B, int Hq, int Hkv, int qL, int kL, int D, float scale, int causal,
                         int window, int q_offset, int dtype, const int64_t *rows, int64_t nrows,
                         int nthreads) {
  problem_t pr;
  if (!out || !rows || nrows < 0 ||
      make_problem(&pr, q, k, v, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype))
    return -1;
  const int64_t total = (int64_t)B * Hq * qL;
  for (int64_t n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return -1;
  if (nrows == 0) return 0;
  return run(&pr, rows, nrows, out, nthreads);
}

/*
 * The same with an additive mask array: bias row (b, hq, i) starts at element
 * b * bias_sb + hq * bias_sh + i * bias_sq of `bias` and holds kL keys.
 * rows == NULL: every row, out [B, Hq, qL, D]; else out is [nrows, D].
 */
int oracle_sdpa_bias_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq,
                         double *out, int B, int Hq, int Hkv, int qL, int kL, int D, float scale,
                         int causal, int window, int q_offset, int dtype, const int64_t *rows,
                         int64_t nrows, int nthreads) {
  problem_t pr;
  if (!out || !bias || bias_sb < 0 || bias_sh < 0 || bias_sq < 0 ||
      make_problem(&pr, q, k, v, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype))
    return -1;
  pr.bias = bias;
  pr.bias_sb = bias_sb;
  pr.bias_sh = bias_sh;
  pr.bias_sq = bias_sq;
  if (!rows) return run(&pr, NULL, (int64_t)B * Hq * qL, out, nthreads);
  const int64_t total = (int64_t)B * Hq * qL;
  for (int64_t n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return -1;
  if (nrows <= 0) return nrows == 0 ? 0 : -1;
  return run(&pr, rows, nrows, out, nthreads);
}

/*
 * A value head dim Dv that may differ from D: v is [B, Hkv, kL, Dv].
 * rows == NULL: every row, out [B, Hq, qL, Dv]; else out is [nrows, Dv].
 */
int oracle_sdpa_dv_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *out,
                       int B, int Hq, int Hkv, int qL, int kL, int D, int Dv, float scale,
                       int causal, int window, int q_offset, int dtype, const int64_t *rows,
                       int64_t nrows, int nthreads) {
  problem_t pr;
  if (!out || Dv < 1 ||
      make_problem(&pr, q, k, v, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype))
    return -1;
  pr.Dv = Dv;
  if (!rows) return run(&pr, NULL, (int64_t)B * Hq * qL, out, nthreads);
  const int64_t total = (int64_t)B * Hq * qL;
  for (int64_t n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return -1;
  if (nrows <= 0) return nrows == 0 ? 0 : -1;
  return run(&pr, rows, nrows, out, nthreads);
}

/*
 * 4-bit K and V: kq/vq hold the codes [B, Hkv, kL, D / 8] (32-bit words),
 * ks/kb and vs/vb the scales and biases [B, Hkv, kL, D / 64] in the input
 * dtype; D must be a multiple of 64.
 * rows == NULL: every row, out [B, Hq, qL, D]; else out is [nrows, D].
 */
int oracle_sdpa_q4kv_f64(const uint16_t *q, const uint32_t *kq, const uint16_t *ks,
                         const uint16_t *kb, const uint32_t *vq, const uint16_t *vs,
                         const uint16_t *vb, double *out, int B, int Hq, int Hkv, int qL, int kL,
                         int D, float scale, int causal, int window, int q_offset, int dtype,
                         const int64_t *rows, int64_t nrows, int nthreads) {
  problem_t pr;
  /* k and v are not read: the quantized rows stand for them */
  if (!out || !kq || !ks || !kb || !vq || !vs || !vb || D % 64 != 0 ||
      make_problem(&pr, q, ks, vs, B, Hq, Hkv, qL, kL, D, scale, causal, window, q_offset, dtype))
    return -1;
  pr.kq = kq;
  pr.ks = ks;
  pr.kb = kb;
  pr.vq = vq;
  pr.vs = vs;
  pr.vb = vb;
  if (!rows) return run(&pr, NULL, (int64_t)B * Hq * qL, out, nthreads);
  const int64_t total = (int64_t)B * Hq * qL;
  for (int64_t n = 0; n < nrows; ++n)
    if (rows[n] < 0 || rows[n] >= total) return -1;
  if (nrows <= 0) return nrows == 0 ? 0 : -1;
  return run(&pr, rows, nrows, out, nthreads);
}

/* The dequantized values of n 4-bit rows of D elements (out [n, D]), for the
 * tests of the format itself. */
void oracle_dequant4(const uint32_t *codes, const uint16_t *scales, const uint16_t *biases,
                     double *out, int64_t n, int D, int dtype) {
  for (int64_t r = 0; r < n; ++r)
    for (long d = 0; d < D; ++d) out[r * D + d] = dequant4(codes, scales, biases, (long)r, D, d, dtype);
}

/* Exact widening exposed for the tests of the input decoding itself. */
void oracle_widen(const uint16_t *h, double *out, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen(h[i], dtype);
}
