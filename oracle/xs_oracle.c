/*
 * xs_oracle.c -- CPU fp64 oracle for the attention forward pass of one GPU's
 * share of Ulysses sequence-parallel attention, with the output relaid into a
 * P-way destination-ordered buffer.
 *
 * THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the HIP library: it is written
 * from the definition of attention and of the all-to-all chunk layout alone.
 *
 * What it follows (the X-Stage paper, "X-Stage: An Overlooked Pipeline Stage
 * for Communication-Computation Overlap in DiT Inference"):
 *  - catalyzex.com abstract, and the gist.science explainer, section
 *    "Zentrale Beitraege", item "FlashAttention-A2A (Piggybacking)": Ulysses
 *    sequence-parallel attention whose post-attention All-to-All is fused into
 *    FlashAttention at tile granularity; the owner of an output tile stores it
 *    to its destination.  FlashAttention computes softmax(scale * Q K^T) V
 *    exactly (up to rounding), so the oracle is that definition written out:
 *    for every batch b, head h and query row i
 *        s_j  = scale * sum_d q[b,i,h,d] * k[b,j,h,d]
 *        m    = max_j s_j                      (exact row max, first pass)
 *        w_j  = exp(s_j - m),  l = sum_j w_j   (second pass)
 *        O[b,i,h,:] = (sum_j w_j * v[b,j,h,:]) / l
 *    There is no online rescaling and no blocking: one query row at a time
 *    (the score pass walks eight keys side by side, each dot product still
 *    summed over d in index order, so every value is the one the plain loop
 *    gives).
 *  - The destination-ordered buffer is the layout an All-to-All over P ranks
 *    delivers when the sequence is cut into P contiguous slices of T = S/P
 *    rows: out_packed[p][b][s'][h][d] = O[b][p*T + s'][h][d].
 *
 *  - The log-sum-exp of a row, lse = log(sum_j exp(s_j)) = m + log(l) in
 *    natural-log units, the by-product of the same two passes.
 *  - Inputs may also arrive in the chunk layout the pre-attention All-to-All
 *    delivers, [P][B][S/P][H][D] (chunk p = rows p*T .. p*T+T-1 of every batch,
 *    the same relayout as the output): element (b, s, h, d) then sits at
 *    (((p*B + b)*T + s')*H + h)*D + d with p = floor(s/T), s' = s - p*T.
 *
 * Inputs are stored as fp64, bf16 (bit patterns) or OCP fp8 e4m3fn codes with
 * a per-tensor fp64 descale; every element is decoded exactly to fp64 once per
 * call, into [B][S][H][D] arrays, before any arithmetic.  All arithmetic is
 * fp64 with libm exp(); each dot product and sum runs in index order.  Build
 * without -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define XSO_F64 0
#define XSO_BF16 1
#define XSO_E4M3 2

/* bf16 is the top half of an IEEE binary32: widen the 16 bits into the high
 * half of a float, which is exact, then widen to double. */
double xs_oracle_decode_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit float E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; there are no
 * infinities and the codes S.1111.111 are NaN; the largest finite is 448. */
double xs_oracle_decode_e4m3(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* The problem after decoding: q, k, v as fp64 [B][H][S][D] arrays, each
 * element the exact value of the input element (x8 * descale for e4m3). */
typedef struct {
  const double *q, *k, *v;
  int64_t B, S, H, D;
  double scale;
} xso_problem;

/* Decodes one input tensor, stored as fp64, bf16 bit patterns or e4m3 codes
 * (times descale) in [B][S][H][D] (in_P = 0) or in the chunk layout
 * [in_P][B][S/in_P][H][D], into a new fp64 array ordered [B][H][S][D], so that
 * the rows of one (batch, head) are contiguous (NULL when the allocation
 * fails).  Every element is decoded exactly, once per call. */
static double *decode_input(int dtype, const void *base, double descale, int64_t in_P, int64_t B,
                            int64_t S, int64_t H, int64_t D) {
  double *x = (double *)malloc((size_t)(B * S * H * D) * sizeof(double));
  if (!x) return NULL;
  double e4m3[256];
  for (int c = 0; c < 256; ++c) e4m3[c] = xs_oracle_decode_e4m3((uint8_t)c) * descale;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t s = 0; s < S; ++s)
      for (int64_t h = 0; h < H; ++h)
        for (int64_t d = 0; d < D; ++d) {
          int64_t idx; /* position of element (b, s, h, d) in the input's layout */
          if (in_P > 0) {
            const int64_t T = S / in_P, p = s / T, sp = s - p * T;
            idx = (((p * B + b) * T + sp) * H + h) * D + d;
          } else {
            idx = ((b * S + s) * H + h) * D + d;
          }
          double val;
          switch (dtype) {
            case XSO_BF16:
              val = xs_oracle_decode_bf16(((const uint16_t *)base)[idx]);
              break;
            case XSO_E4M3:
              val = e4m3[((const uint8_t *)base)[idx]];
              break;
            default:
              val = ((const double *)base)[idx];
          }
          x[((b * H + h) * S + s) * D + d] = val;
        }
  return x;
}

/* One output row O[b,i,h,:] by the two-pass definition above, and the row's
 * log-sum-exp.  `s` is a scratch row of S doubles and `acc` one of D doubles. */
static double attention_row(const xso_problem *pr, int64_t b, int64_t i, int64_t h, double *s,
                            double *acc, double *out_row) {
  const int64_t S = pr->S, H = pr->H, D = pr->D;
  const size_t head = (size_t)((b * H + h) * S) * D; /* row 0 of (b, h) */
  const double *qi = pr->q + head + i * D, *K = pr->k + head, *V = pr->v + head;
  /* pass 1: the scores.  Keys are taken eight at a time only so that the
   * eight dot products -- each summed over d in index order -- proceed side
   * by side; the remaining keys one at a time. */
  int64_t j = 0;
  for (; j + 8 <= S; j += 8) {
    const double *k0 = K + j * D;
    double dot[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int64_t d = 0; d < D; ++d)
      for (int u = 0; u < 8; ++u) dot[u] += qi[d] * k0[u * D + d];
    for (int u = 0; u < 8; ++u) s[j + u] = pr->scale * dot[u];
  }
  for (; j < S; ++j) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qi[d] * K[j * D + d];
    s[j] = pr->scale * dot;
  }
  double m = -INFINITY;
  for (j = 0; j < S; ++j)
    if (s[j] > m) m = s[j];
  /* pass 2 */
  double l = 0.0;
  for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
  for (j = 0; j < S; ++j) {
    const double *vj = V + j * D;
    double w = exp(s[j] - m);
    l += w;
    for (int64_t d = 0; d < D; ++d) acc[d] += w * vj[d];
  }
  for (int64_t d = 0; d < D; ++d) out_row[d] = acc[d] / l;
  return m + log(l);
}

/* Flat offset of element (b, s, h, d) of O inside the destination-ordered
 * buffer [P][B][T][H][D], T = S/P, slice p = floor(s/T) holding rows
 * p*T .. p*T+T-1 of every batch. */
int64_t xs_oracle_packed_offset(int64_t B, int64_t S, int64_t H, int64_t D, int64_t P, int64_t b,
                                int64_t s, int64_t h, int64_t d) {
  int64_t T = S / P;
  int64_t p = s / T;
  int64_t sp = s - p * T;
  return (((p * B + b) * T + sp) * H + h) * D + d;
}

/* Relayout of a [B][S][H][D] fp64 tensor into [P][B][S/P][H][D].
 * Returns 0, or -2 when a size is < 1 or S is not a multiple of P. */
int xs_oracle_pack(const double *o, int64_t B, int64_t S, int64_t H, int64_t D, int64_t P,
                   double *out_packed) {
  if (B < 1 || S < 1 || H < 1 || D < 1 || P < 1 || S % P != 0) return -2;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t s = 0; s < S; ++s)
      for (int64_t h = 0; h < H; ++h)
        for (int64_t d = 0; d < D; ++d)
          out_packed[xs_oracle_packed_offset(B, S, H, D, P, b, s, h, d)] =
              o[((b * S + s) * H + h) * D + d];
  return 0;
}

typedef struct {
  const xso_problem *pr;
  const int64_t *rows; /* nrows triples (b, s, h) */
  int64_t nrows;
  double *out;         /* row r -> out + r*D, unless packed */
  int64_t P;           /* > 0: write into the packed buffer instead */
  double *lse;         /* NULL, or row r -> lse[r] (rows) / lse[(b*H + h)*S + s] (packed) */
  int tid, nthreads;
  int status;
} xso_job;

static void *worker(void *arg) {
  xso_job *job = (xso_job *)arg;
  const xso_problem *pr = job->pr;
  double *s = (double *)malloc((size_t)pr->S * sizeof(double));
  double *acc = (double *)malloc((size_t)pr->D * sizeof(double));
  double *row = (double *)malloc((size_t)pr->D * sizeof(double));
  if (!s || !acc || !row) {
    job->status = -1;
    free(s), free(acc), free(row);
    return NULL;
  }
  for (int64_t r = job->tid; r < job->nrows; r += job->nthreads) {
    int64_t b = job->rows[3 * r], i = job->rows[3 * r + 1], h = job->rows[3 * r + 2];
    const double lse = attention_row(pr, b, i, h, s, acc, row);
    if (job->lse) job->lse[job->P > 0 ? (b * pr->H + h) * pr->S + i : r] = lse;
    for (int64_t d = 0; d < pr->D; ++d) {
      if (job->P > 0)
        job->out[xs_oracle_packed_offset(pr->B, pr->S, pr->H, pr->D, job->P, b, i, h, d)] = row[d];
      else
        job->out[r * pr->D + d] = row[d];
    }
  }
  free(s), free(acc), free(row);
  job->status = 0;
  return NULL;
}

static int run_rows(const xso_problem *pr, const int64_t *rows, int64_t nrows, double *out,
                    int64_t P, double *lse, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int created[256];
  xso_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (xso_job){pr, rows, nrows, out, P, lse, t, nthreads, -1};
    created[t] = pthread_create(&th[t], NULL, worker, &jobs[t]) == 0;
    if (!created[t]) worker(&jobs[t]); /* run this share on the calling thread */
  }
  int status = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (created[t]) pthread_join(th[t], NULL);
    if (jobs[t].status != 0) status = -1;
  }
  return status;
}

/* Decodes q, k, v (see decode_input) and computes the given rows; the decoded
 * copies are freed before returning.  Returns 0 or -1 (allocation). */
static int solve(int dtype, const void *q, const void *k, const void *v, double q_descale,
                 double k_descale, double v_descale, int64_t in_P, int64_t B, int64_t S,
                 int64_t H, int64_t D, double scale, const int64_t *rows, int64_t nrows,
                 double *out, int64_t P, double *lse, int nthreads) {
  double *qd = decode_input(dtype, q, q_descale, in_P, B, S, H, D);
  double *kd = decode_input(dtype, k, k_descale, in_P, B, S, H, D);
  double *vd = decode_input(dtype, v, v_descale, in_P, B, S, H, D);
  int rc = -1;
  if (qd && kd && vd) {
    xso_problem pr = {qd, kd, vd, B, S, H, D, scale};
    rc = run_rows(&pr, rows, nrows, out, P, lse, nthreads);
  }
  free(qd), free(kd), free(vd);
  return rc;
}

static int check(int dtype, const void *q, const void *k, const void *v, int64_t B, int64_t S,
                 int64_t H, int64_t D) {
  if (!q || !k || !v) return -1;
  if (B < 1 || S < 1 || H < 1 || D < 1) return -2;
  if (dtype < XSO_F64 || dtype > XSO_E4M3) return -3;
  return 0;
}

/* Attention rows O[b,s,h,:] for nrows (b, s, h) triples; out is nrows x D;
 * lse (may be NULL) receives the rows' log-sum-exp.  in_P = 0 for
 * [B][S][H][D] inputs, >= 1 for inputs in the [in_P][B][S/in_P][H][D] chunk
 * layout.  Returns 0, -1 (null pointer / allocation), -2 (shape), -3 (dtype). */
int xs_oracle_attention_rows_ex(int dtype, const void *q, const void *k, const void *v,
                                double q_descale, double k_descale, double v_descale, int64_t in_P,
                                int64_t B, int64_t S, int64_t H, int64_t D, double scale,
                                const int64_t *rows, int64_t nrows, double *out, double *lse,
                                int nthreads) {
  int rc = check(dtype, q, k, v, B, S, H, D);
  if (rc) return rc;
  if (!rows || !out) return -1;
  if (in_P < 0 || (in_P > 0 && S % in_P != 0)) return -2;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 || rows[3 * r + 1] >= S ||
        rows[3 * r + 2] < 0 || rows[3 * r + 2] >= H)
      return -2;
  return solve(dtype, q, k, v, q_descale, k_descale, v_descale, in_P, B, S, H, D, scale, rows,
               nrows, out, 0, lse, nthreads);
}

int xs_oracle_attention_rows(int dtype, const void *q, const void *k, const void *v,
                             double q_descale, double k_descale, double v_descale, int64_t B,
                             int64_t S, int64_t H, int64_t D, double scale, const int64_t *rows,
                             int64_t nrows, double *out, int nthreads) {
  return xs_oracle_attention_rows_ex(dtype, q, k, v, q_descale, k_descale, v_descale, 0, B, S, H,
                                     D, scale, rows, nrows, out, NULL, nthreads);
}

/* The whole hot path: attention over every (b, s, h) row, written straight
 * into the destination-ordered buffer [P][B][S/P][H][D] (fp64); lse (may be
 * NULL) receives the log-sum-exp of every row as [B][H][S].  in_P as above.
 * Returns 0, -1, -2 (also S % P != 0), -3. */
int xs_oracle_attention_packed_ex(int dtype, const void *q, const void *k, const void *v,
                                  double q_descale, double k_descale, double v_descale,
                                  int64_t in_P, int64_t B, int64_t S, int64_t H, int64_t D,
                                  int64_t P, double scale, double *out_packed, double *lse,
                                  int nthreads) {
  int rc = check(dtype, q, k, v, B, S, H, D);
  if (rc) return rc;
  if (!out_packed) return -1;
  if (P < 1 || S % P != 0) return -2;
  if (in_P < 0 || (in_P > 0 && S % in_P != 0)) return -2;
  int64_t nrows = B * S * H;
  int64_t *rows = (int64_t *)malloc((size_t)nrows * 3 * sizeof(int64_t));
  if (!rows) return -1;
  int64_t r = 0; /* ordered by (b, h, s): threads work on the rows of one head together */
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t s = 0; s < S; ++s) {
        rows[3 * r] = b, rows[3 * r + 1] = s, rows[3 * r + 2] = h;
        ++r;
      }
  rc = solve(dtype, q, k, v, q_descale, k_descale, v_descale, in_P, B, S, H, D, scale, rows, nrows,
             out_packed, P, lse, nthreads);
  free(rows);
  return rc;
}

int xs_oracle_attention_packed(int dtype, const void *q, const void *k, const void *v,
                               double q_descale, double k_descale, double v_descale, int64_t B,
                               int64_t S, int64_t H, int64_t D, int64_t P, double scale,
                               double *out_packed, int nthreads) {
  return xs_oracle_attention_packed_ex(dtype, q, k, v, q_descale, k_descale, v_descale, 0, B, S,
                                       H, D, P, scale, out_packed, NULL, nthreads);
}
