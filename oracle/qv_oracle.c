/*
 * qv_oracle.c -- slow, plain CPU oracle for the quantized speculative-verify path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * file; only the test-suite, the smoke check and the CPU-baseline leg of the benchmark do.
 * It shares no code, header, table or constant with the GPU kernels.
 *
 * Every function is the plain definition of what the method computes, written out with
 * no blocking, fusion or reordering beyond what the definition states:
 *
 *   oracle_quant_act    per-token symmetric int8 quantisation of activations, with the
 *                       optional online smoothing prescale X*diag(s)^-1
 *                       (Quasar, Sec. 3.2 "W8A8 Verification via Enhanced SmoothQuant" and
 *                        Sec. 3.3 "Online Activation Smoothing and Quantization")
 *   oracle_linear_w8a8  int8 x int8 -> int32 dot products, then dequantisation by the
 *                       per-token and per-channel scales
 *                       (Quasar, Sec. 3.3 "INT8 Gemm and Dequantization")
 *   oracle_linear_w4a16 explicit group-wise dequantisation of 4-bit weights, then a
 *                       triple-loop product with 16-bit activations, summed in double
 *                       (Speculative Decoding Meets Quantization review: the W4A16 target
 *                        that verifies the draft in one forward pass)
 *   oracle_argmax       row-wise argmax of fp16 logits, lowest index on ties
 *                       (Quasar, Sec. 4.5: the verifier's top-1 decides acceptance)
 *   oracle_accept       greedy (T=0) accept length: longest draft prefix equal to the
 *                       verifier's argmax (Quasar, Sec. 4.2 / Table 1 mean acceptance length)
 *
 * Readings taken where the pages are silent (the formulas of Sec. 3.2-3.3 are not legible):
 *   - activation scale s_m = absmax_m / 127 (fp32 division), q = clamp(rne(x'/s_m),-127,127),
 *     an all-zero row gives s_m = 0 and q = 0;
 *   - W8A8 output y = fp16( fp32( fp32(acc) * s_x[m] ) * s_w[n] ), two fp32 products in
 *     this order, each rounded to nearest-even, no fused multiply-add;
 *   - W4A16 weight w = (q - z) * s with group g = k / 128, nibble j of a 32-bit word holds
 *     k = 8*word + j (low nibble first); y = fp16(sum over k of x*w) summed in double.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (x86-64 SSE arithmetic, so every
 * float operation is a single IEEE binary32 operation, rounded to nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------ */
/* IEEE binary16 conversions, written from the format's definition.                      */
/* ------------------------------------------------------------------------------------ */

/* binary16 bit pattern -> value (exact in float): sign, 5-bit biased exponent, 10-bit
 * fraction; exponent 0 encodes subnormals (fraction * 2^-24). */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

float oracle_half_to_float(uint16_t h) { return (float)oracle_half_to_double(h); }

/* value -> nearest binary16, ties to even.  The spacing of binary16 values near |d| is
 * 2^(e-10) for 2^e <= |d| < 2^(e+1), e >= -14, and 2^-24 below 2^-14.  Dividing by a
 * power of two is exact, so nearbyint (round-half-even in the default mode) of the scaled
 * value is the correctly rounded result.  Magnitudes that round to 2^16 or beyond are inf. */
uint16_t oracle_double_to_half(double d) {
  uint16_t sign = (d < 0 || (d == 0 && signbit(d))) ? 0x8000 : 0;
  double a = fabs(d);
  if (isnan(d)) return 0x7e00;
  if (a == 0) return sign;
  int e;
  frexp(a, &e);          /* a = m * 2^e with 0.5 <= m < 1, so 2^(e-1) <= a < 2^e */
  e -= 1;                /* now 2^e <= a < 2^(e+1) */
  if (e < -14) e = -14;  /* subnormal range shares the spacing of the smallest normals */
  double quantum = ldexp(1.0, e - 10);
  double r = nearbyint(a / quantum) * quantum;
  if (r >= 65536.0) return sign | 0x7c00;
  /* encode r, which is now exactly representable */
  if (r < ldexp(1.0, -14)) {
    return sign | (uint16_t)(r / ldexp(1.0, -24));
  }
  int re;
  frexp(r, &re);
  re -= 1; /* 2^re <= r < 2^(re+1); rounding may have carried into the next binade */
  uint16_t frac = (uint16_t)(r / ldexp(1.0, re - 10) - 1024.0);
  return sign | (uint16_t)((re + 15) << 10) | frac;
}

uint16_t oracle_float_to_half(float f) { return oracle_double_to_half((double)f); }

/* ------------------------------------------------------------------------------------ */
/* a1: per-token activation quantisation                                                 */
/* ------------------------------------------------------------------------------------ */

/* x: fp16 bits [M][K]; inv_smooth: fp32 [K] or NULL (the smoothing factors' reciprocals);
 * outputs x_q int8 [M][K] and x_scale fp32 [M]. */
void oracle_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                      int8_t* x_q, float* x_scale) {
  for (int m = 0; m < M; ++m) {
    float amax = 0.0f;
    for (int k = 0; k < K; ++k) {
      float v = oracle_half_to_float(x[(size_t)m * K + k]);
      if (inv_smooth) v = v * inv_smooth[k];
      float av = fabsf(v);
      if (av > amax) amax = av;
    }
    float s = amax / 127.0f;
    x_scale[m] = s;
    for (int k = 0; k < K; ++k) {
      int8_t q = 0;
      if (amax != 0.0f) {
        float v = oracle_half_to_float(x[(size_t)m * K + k]);
        if (inv_smooth) v = v * inv_smooth[k];
        float t = v / s;
        float r = nearbyintf(t);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q = (int8_t)r;
      }
      x_q[(size_t)m * K + k] = q;
    }
  }
}

/* ------------------------------------------------------------------------------------ */
/* a2/a3: W8A8 linear                                                                    */
/* ------------------------------------------------------------------------------------ */

/* x_q int8 [M][K], x_scale fp32 [M], w int8 [N][K] (output-channel rows), w_scale fp32 [N].
 * Writes acc int32 [M][N] (may be NULL) and y fp16 bits [M][N] (may be NULL).
 * Returns 0, or 1 if some dot product does not fit in int32. */
int oracle_linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K,
                       const int8_t* w, const float* w_scale, int N,
                       uint16_t* y, int32_t* acc_out) {
  int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
  for (int m = 0; m < M; ++m) {
    for (int n = 0; n < N; ++n) {
      int64_t acc = 0;
      const int8_t* xr = x_q + (size_t)m * K;
      const int8_t* wr = w + (size_t)n * K;
      for (int k = 0; k < K; ++k) acc += (int64_t)xr[k] * (int64_t)wr[k];
      if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;
      int32_t a32 = (int32_t)acc;
      if (acc_out) acc_out[(size_t)m * N + n] = a32;
      if (y) {
        float t = (float)a32;
        t = t * x_scale[m];
        t = t * w_scale[n];
        y[(size_t)m * N + n] = oracle_float_to_half(t);
      }
    }
  }
  return overflow;
}

/* ------------------------------------------------------------------------------------ */
/* a4: W4A16 linear                                                                      */
/* ------------------------------------------------------------------------------------ */

/* Weight code of (n, k): nibble (k % 8) of 32-bit word k / 8 in row n, low nibble first. */
static int w4_code(const uint32_t* qweight, int K, int n, int k) {
  uint32_t word = qweight[(size_t)n * (K / 8) + k / 8];
  return (int)((word >> (4 * (k % 8))) & 0xF);
}

/* x fp16 bits [M][K]; qweight uint32 [N][K/8]; scales fp16 bits [N][K/G]; zeros uint8
 * [N][K/G] (values 0..15); writes y fp16 bits [M][N].  Each weight row is dequantised
 * explicitly, w = (q - z) * s (exact in fp32), then dotted with every activation row in
 * double (products exact, one rounding per addition), and the sum is rounded once to fp16. */
void oracle_linear_w4a16(const uint16_t* x, int M, int K, const uint32_t* qweight,
                         const uint16_t* scales, const uint8_t* zeros, int N, int group_size,
                         uint16_t* y) {
  int ng = K / group_size;
#pragma omp parallel
  {
    float* wrow = (float*)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      for (int k = 0; k < K; ++k) {
        int g = k / group_size;
        int q = w4_code(qweight, K, n, k);
        int z = zeros[(size_t)n * ng + g];
        float s = oracle_half_to_float(scales[(size_t)n * ng + g]);
        wrow[k] = (float)(q - z) * s;
      }
      for (int m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k)
          acc += oracle_half_to_double(x[(size_t)m * K + k]) * (double)wrow[k];
        y[(size_t)m * N + n] = oracle_double_to_half(acc);
      }
    }
    free(wrow);
  }
}

/* ------------------------------------------------------------------------------------ */
/* W4A8 linear: 4-bit weights (the W4A16 format) with per-token int8 activations          */
/* ------------------------------------------------------------------------------------ */

/* x_q int8 [M][K] and x_scale fp32 [M] (as quant_act makes them); qweight, scales, zeros as
 * for W4A16; writes y fp16 bits [M][N].  Per group g the integer dot product
 * acc_g = sum_{k in g} x_q[k] * (q[k] - z_g) is exact; each s_g * acc_g is exact in double
 * (11 + 18 significant bits), their sum over g is added in double, multiplied by x_scale,
 * and rounded once to fp16. */
void oracle_linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        int N, int group_size, uint16_t* y) {
  int ng = K / group_size;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int m = 0; m < M; ++m) {
      double r = 0.0;
      for (int g = 0; g < ng; ++g) {
        int z = zeros[(size_t)n * ng + g];
        long long acc = 0;
        for (int k = g * group_size; k < (g + 1) * group_size; ++k)
          acc += (long long)x_q[(size_t)m * K + k] * (w4_code(qweight, K, n, k) - z);
        r += oracle_half_to_double(scales[(size_t)n * ng + g]) * (double)acc;
      }
      y[(size_t)m * N + n] = oracle_double_to_half(r * (double)x_scale[m]);
    }
  }
}

/* ------------------------------------------------------------------------------------ */
/* a6/a7: greedy verify                                                                  */
/* ------------------------------------------------------------------------------------ */

/* logits fp16 bits [M][V] -> argmax int32 [M]; values compared as real numbers, the lowest
 * index wins a tie, -0 equals +0. */
void oracle_argmax(const uint16_t* logits, int M, int V, int32_t* argmax_out) {
  for (int m = 0; m < M; ++m) {
    int best = 0;
    double bv = oracle_half_to_double(logits[(size_t)m * V]);
    for (int v = 1; v < V; ++v) {
      double cv = oracle_half_to_double(logits[(size_t)m * V + v]);
      if (cv > bv) { bv = cv; best = v; }
    }
    argmax_out[m] = best;
  }
}

/* Row 0 of the verify batch is the last accepted token, rows 1..M-1 the drafts; the
 * verifier's prediction after row i is argmax[i], so draft token i is kept while
 * draft[i] == argmax[i] for every earlier i.  Returns n_accept in [0, M-1]; the step
 * then emits draft[0..n_accept-1] followed by argmax[n_accept]. */
int oracle_accept(const int32_t* draft, const int32_t* argmax_in, int M) {
  int j = 0;
  while (j < M - 1 && draft[j] == argmax_in[j]) ++j;
  return j;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Host threads the OpenMP loops use from now on (n >= 1); only timing changes. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
