/*
 * fp64 CPU oracle for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the CPU
 * baseline of the benchmark call this file; the GPU library never does, and
 * the two share no code, header or table.
 *
 * What it computes is the plain definition of attention, not the tiled
 * algorithm:
 *   - "Android Transformer Optimization: Attention and Mobile GPU
 *     Bottlenecks", section "The Self-Attention Bottleneck Is Memory Traffic,
 *     Not Compute": S = Q K^T, P = softmax(S) taken along each row, O = P V.
 *   - "Flash Attention on Android: tiled SGEMM with RenderScript", section
 *     "Architecture: tiled attention with RenderScript BLAS": the scores are
 *     multiplied by a softmax scale (1/sqrt(headDim) there; a caller-supplied
 *     factor here).
 *   - The first page's section "The Essence of FlashAttention: Reordering the
 *     Computation" says that the tiled pass with an online softmax reaches the
 *     same result and only changes the order of the arithmetic; so this
 *     definition is what the tiled GPU kernel is checked against.
 *   - Causal mask (not on the pages): key j is excluded from query i when
 *     j > i; the diagonal is kept.
 *
 * Every score row S[i, :] and probability row P[i, :] is materialised in
 * fp64.  The softmax subtracts the row maximum before exp (the stabilisation
 * that the first page's "Essence" section explains); this changes nothing
 * mathematically.  Inputs are decoded from their storage bits by decoders
 * written here from the IEEE 754 binary16 / binary32 definitions, so the
 * oracle sees exactly the values the GPU sees.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage types, numbered like the library's public enum but defined here on
 * their own. */
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits. */
double fa_oracle_decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double val;
  if (e == 0) {
    val = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  } else if (e == 31) {
    val = f ? NAN : INFINITY;
  } else {
    val = ldexp((double)(f | 0x400), e - 25); /* (1024+f) * 2^(e-15-10) */
  }
  return sign ? -val : val;
}

/* bfloat16: the upper half of an IEEE 754 binary32, i.e. 1 sign bit, 8
 * exponent bits (bias 127) and 7 fraction bits. */
double fa_oracle_decode_bf16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int f = h & 0x7f;
  double val;
  if (e == 0) {
    val = ldexp((double)f, -133); /* subnormal: f * 2^-126 * 2^-7 */
  } else if (e == 255) {
    val = f ? NAN : INFINITY;
  } else {
    val = ldexp((double)(f | 0x80), e - 134); /* (128+f) * 2^(e-127-7) */
  }
  return sign ? -val : val;
}

/* IEEE 754 binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction
 * bits. */
double fa_oracle_decode_f32(uint32_t u) {
  int sign = (u >> 31) & 1;
  int e = (u >> 23) & 0xff;
  int32_t f = (int32_t)(u & 0x7fffff);
  double val;
  if (e == 0) {
    val = ldexp((double)f, -149);
  } else if (e == 255) {
    val = f ? NAN : INFINITY;
  } else {
    val = ldexp((double)(f | 0x800000), e - 150);
  }
  return sign ? -val : val;
}

static double decode_one(const void* buf, int dtype, int64_t idx) {
  if (dtype == ORACLE_F32) {
    uint32_t u;
    memcpy(&u, (const char*)buf + 4 * idx, 4);
    return fa_oracle_decode_f32(u);
  }
  uint16_t h;
  memcpy(&h, (const char*)buf + 2 * idx, 2);
  return dtype == ORACLE_F16 ? fa_oracle_decode_f16(h) : fa_oracle_decode_bf16(h);
}

/* Decode count consecutive elements starting at element offset. */
static void decode_span(const void* buf, int dtype, int64_t offset, int64_t count, double* dst) {
  for (int64_t t = 0; t < count; ++t) dst[t] = decode_one(buf, dtype, offset + t);
}

/*
 * One output row of one head, straight from the definition.
 *   qrow: D values; Kh, Vh: N x D row-major for this head.
 *   s, p: scratch rows of N doubles (the materialised S[i,:] and P[i,:]).
 *   orow: D outputs.  *psum receives sum_j P[i,j] after normalisation.
 *   *plse receives the log-sum-exp of the row's scores, ln sum_j exp(S[i,j])
 *   = m + ln sum_j exp(S[i,j] - m): the running maximum and denominator of
 *   the first page's section "The Essence of FlashAttention: Reordering the
 *   Computation" folded into one number (m + ln l).
 */
static void attend_row(const double* qrow, const double* Kh, const double* Vh, int64_t i, int64_t N,
                       int64_t D, double scale, int causal, double* s, double* p, double* orow,
                       double* psum, double* plse) {
  /* S[i, j] = scale * <Q[i,:], K[j,:]>; masked keys get -inf. */
  for (int64_t j = 0; j < N; ++j) {
    if (causal && j > i) {
      s[j] = -INFINITY;
      continue;
    }
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += qrow[d] * Kh[j * D + d];
    s[j] = scale * acc;
  }
  /* P[i, :] = softmax(S[i, :]) = exp(S - max) / sum(exp(S - max)). */
  double m = -INFINITY;
  for (int64_t j = 0; j < N; ++j)
    if (s[j] > m) m = s[j];
  double denom = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    p[j] = exp(s[j] - m);
    denom += p[j];
  }
  double total = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    p[j] /= denom;
    total += p[j];
  }
  if (psum) *psum = total;
  if (plse) *plse = m + log(denom);
  /* O[i, :] = sum_j P[i, j] * V[j, :]. */
  for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    const double pj = p[j];
    for (int64_t d = 0; d < D; ++d) orow[d] += pj * Vh[j * D + d];
  }
}

static int valid_args(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                      int64_t N, int64_t D) {
  if (!q || !k || !v) return 0;
  if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16) return 0;
  if (B < 0 || H < 0 || N < 0 || D <= 0) return 0;
  return 1;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/*
 * Full forward pass.  q, k, v: [B, H, N, D] in storage type dtype.
 * o: [B, H, N, D] fp64 output.  rowsum (optional): [B, H, N], sum of each P
 * row.  lse (optional): [B, H, N], log-sum-exp of each score row.  Heads are
 * processed one after another, the rows of a head in parallel.  Returns the
 * number of threads used, or -1 on bad arguments.
 */
int fa_oracle_forward(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                      int64_t N, int64_t D, double scale, int causal, double* o, double* rowsum,
                      double* lse, int nthreads) {
  if (!valid_args(q, k, v, dtype, B, H, N, D) || !o) return -1;
  int used = set_threads(nthreads);
  if (N == 0) return used;
  double* Qh = (double*)malloc(sizeof(double) * N * D);
  double* Kh = (double*)malloc(sizeof(double) * N * D);
  double* Vh = (double*)malloc(sizeof(double) * N * D);
  if (!Qh || !Kh || !Vh) {
    free(Qh);
    free(Kh);
    free(Vh);
    return -1;
  }
  for (int64_t bh = 0; bh < B * H; ++bh) {
    const int64_t base = bh * N * D;
    decode_span(q, dtype, base, N * D, Qh);
    decode_span(k, dtype, base, N * D, Kh);
    decode_span(v, dtype, base, N * D, Vh);
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * N);
      double* p = (double*)malloc(sizeof(double) * N);
#pragma omp for schedule(dynamic, 16)
      for (int64_t i = 0; i < N; ++i) {
        attend_row(Qh + i * D, Kh, Vh, i, N, D, scale, causal, s, p, o + base + i * D,
                   rowsum ? rowsum + bh * N + i : NULL, lse ? lse + bh * N + i : NULL);
      }
      free(s);
      free(p);
    }
  }
  free(Qh);
  free(Kh);
  free(Vh);
  return used;
}

/*
 * Selected output rows only, for checks at sizes where the full pass is too
 * slow.  Row r is query row_idx[r] of flattened head bh_idx[r] (= b*H + h).
 * o_rows: [nrows, D] fp64.  lse_rows (optional): [nrows], each row's
 * log-sum-exp.  Returns threads used, or -1 on bad arguments.
 */
int fa_oracle_rows(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                   int64_t N, int64_t D, double scale, int causal, const int64_t* bh_idx,
                   const int64_t* row_idx, int64_t nrows, double* o_rows, double* lse_rows,
                   int nthreads) {
  if (!valid_args(q, k, v, dtype, B, H, N, D) || !o_rows || (nrows > 0 && (!bh_idx || !row_idx)))
    return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (bh_idx[r] < 0 || bh_idx[r] >= B * H || row_idx[r] < 0 || row_idx[r] >= N) return -1;
  int used = set_threads(nthreads);
  int bad = 0;
#pragma omp parallel
  {
    double* Kh = (double*)malloc(sizeof(double) * N * D);
    double* Vh = (double*)malloc(sizeof(double) * N * D);
    double* qrow = (double*)malloc(sizeof(double) * D);
    double* s = (double*)malloc(sizeof(double) * N);
    double* p = (double*)malloc(sizeof(double) * N);
    int64_t cached = -1;
    if (!Kh || !Vh || !qrow || !s || !p) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      int stop;
#pragma omp atomic read
      stop = bad;
      if (stop) continue;
      const int64_t bh = bh_idx[r];
      const int64_t base = bh * N * D;
      if (bh != cached) {
        decode_span(k, dtype, base, N * D, Kh);
        decode_span(v, dtype, base, N * D, Vh);
        cached = bh;
      }
      decode_span(q, dtype, base + row_idx[r] * D, D, qrow);
      attend_row(qrow, Kh, Vh, row_idx[r], N, D, scale, causal, s, p, o_rows + r * D, NULL,
                 lse_rows ? lse_rows + r : NULL);
    }
    free(Kh);
    free(Vh);
    free(qrow);
    free(s);
    free(p);
  }
  return bad ? -1 : used;
}
