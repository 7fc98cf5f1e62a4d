/*
 * q8_oracle.c -- plain, slow, fp64 CPU oracle for the Q8_0 decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library; the two meet only on the seeded
 * inputs.  Every function is the textbook definition written out, evaluated
 * in double precision with ascending-index loops and no blocking or fusion.
 *
 * Sources (web pages, cited by title and section):
 *   [LUMEN]  "Lumen v0.3.0 -- profile, parallelize, 4x faster than v0.2.0",
 *            sections "Phase 7.E.0" (decode profile: qkv, wo, gate_up,
 *            silu_mul, down, lm_head matmuls) and "Phase 7.J" (row split of
 *            Q8 matmuls across threads); "v0.3 -> v0.4 candidate moves"
 *            (dequant -> fp32 FMA path).
 *   [MOE]    "Add Qwen1.5-MoE Q8_0 CPU and single-token TornadoVM GPU
 *            inference - #144", opening description (router + top-k experts
 *            + shared-expert FFN block) and "Key implementation notes"
 *            (Q8_0 scales times 8-bit quants).
 *   [AUGUR]  "augur" README, "Features" (RMSNorm, grouped-query attention,
 *            SwiGLU MLP, decoder block order, greedy generation).
 *   [FUSED]  "fusedtok 1.3.0" PKG-INFO, "API stability" (selection ties
 *            resolve to the earliest index).
 *   [COGNI]  "skuznetsov/cogni-ml" README, "Qwen 3.5 Native Metal" /
 *            cuda_q8_gemv_probe (raw GGUF Q8_0 block layout).
 *
 * Q8_0 block (GGUF): 34 bytes = binary16 scale d (little-endian) followed by
 * 32 signed 8-bit quants q; weight = d * q.  Blocks of a row are
 * consecutive; rows are consecutive.
 *
 * Readings where the pages are silent are listed in the repository's design
 * notes; the ones that change arithmetic here: activations stay fp32 (no
 * requantisation), rmsnorm has unit weight, the shared-expert gate is
 * sigmoid of one logit, top-k weights are renormalised over the selected
 * experts, and the attention stand-in at position 0 copies each query head's
 * value head.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32
#define BLOCK_BYTES 34

/* IEEE 754 binary16 -> double, by the definition of the format:
 *   e == 0       : (-1)^s * m * 2^-24            (zero and subnormals)
 *   0 < e < 31   : (-1)^s * (1024 + m) * 2^(e-25)
 *   e == 31      : infinity (m == 0) or NaN       */
double oracle_f16_to_f64(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

void oracle_f16_decode(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

/* Dequantised weight w[r][k] of an M x K Q8_0 matrix in GGUF block order
 * [COGNI]; w = d * q [MOE "Key implementation notes"]. */
static double q8_weight(const uint8_t* aos, int64_t K, int64_t r, int64_t k) {
  const int64_t nb = K / QK;
  const uint8_t* blk = aos + (r * nb + k / QK) * BLOCK_BYTES;
  uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
  int8_t q = (int8_t)blk[2 + k % QK];
  return oracle_f16_to_f64(dbits) * (double)q;
}

void oracle_dequant_row(const uint8_t* aos, int64_t K, int64_t r, double* out) {
  for (int64_t k = 0; k < K; ++k) out[k] = q8_weight(aos, K, r, k);
}

/* ---------------------------------------------------------------------------
 * Matrix-vector product  y[n][r] = sum_k w[r][k] * x[n][k]   (ascending k)
 * and the magnitude sum  S[n][r] = sum_k |w[r][k] * x[n][k]|  used by the
 * error tolerance.  [LUMEN "Phase 7.E.0": every projection of the decode step
 * is this product; "Phase 7.J": output rows split across threads.]
 * x is [N][K] double, y and S are [N][M] double.
 * ------------------------------------------------------------------------- */
typedef struct {
  const uint8_t* aos;
  int64_t M, K, N;
  const double* x;
  double* y;
  double* S;
  int64_t r0, r1;
} gemv_job;

static void* gemv_rows(void* arg) {
  gemv_job* j = (gemv_job*)arg;
  for (int64_t n = 0; n < j->N; ++n) {
    const double* xn = j->x + n * j->K;
    for (int64_t r = j->r0; r < j->r1; ++r) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < j->K; ++k) {
        double p = q8_weight(j->aos, j->K, r, k) * xn[k];
        acc += p;
        mag += fabs(p);
      }
      j->y[n * j->M + r] = acc;
      if (j->S) j->S[n * j->M + r] = mag;
    }
  }
  return NULL;
}

int oracle_q8_0_gemv_f64(const uint8_t* aos, int64_t M, int64_t K, const double* x,
                         int64_t N, double* y, double* S, int threads) {
  if (M < 0 || K <= 0 || K % QK || N < 1) return -1;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > M) threads = M > 0 ? (int)M : 1;
  gemv_job jobs[256];
  pthread_t tid[256];
  for (int t = 0; t < threads; ++t) {
    jobs[t] = (gemv_job){aos, M, K, N, x, y, S, M * t / threads, M * (t + 1) / threads};
  }
  if (threads == 1) {
    gemv_rows(&jobs[0]);
    return 0;
  }
  for (int t = 0; t < threads; ++t) pthread_create(&tid[t], NULL, gemv_rows, &jobs[t]);
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
  return 0;
}

/* fp32 activations, widened exactly to double. */
int oracle_q8_0_gemv(const uint8_t* aos, int64_t M, int64_t K, const float* x, int64_t N,
                     double* y, double* S, int threads) {
  if (K <= 0 || N < 1) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(N * K));
  if (!xd) return -2;
  for (int64_t i = 0; i < N * K; ++i) xd[i] = (double)x[i];
  int rc = oracle_q8_0_gemv_f64(aos, M, K, xd, N, y, S, threads);
  free(xd);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Integer-activation variant (opt-in; never the graded fp32 path).  [MOE "Key
 * implementation notes": each fp32 activation block is quantized to int8
 * before the dot product, then int8 x int8 products are accumulated and
 * scaled with the Q8_0 scales.]  The pages leave the quantizer open; the
 * reading taken makes each block of 32 activations a Q8_0 block like the
 * weights:
 *   amax = max_j |x_j|,  d = amax / 127  (fp32 division, round to nearest)
 *   q_j  = x_j / d (fp32 division) rounded to the nearest integer, ties to
 *          even; every q_j = 0 when amax == 0
 *   the block's stored scale is binary16(d), rounded to nearest even, and
 *   the dot product uses the stored scale:
 *   y[n][r] = sum_b dw[r][b] * dx[n][b] * sum_j qw[r][b][j] * qx[n][b][j].
 * ------------------------------------------------------------------------- */

/* double (holding a finite fp32 value) -> binary16 bits, round to nearest
 * even, by the definition of the format (subnormals below 2^-14, infinity
 * from 65520 up). */
static uint16_t f64_to_f16_bits(double v) {
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && signbit(v))) {
    sign = 0x8000;
    v = -v;
  }
  if (v == 0) return sign;
  if (v >= 65520.0) return (uint16_t)(sign | 0x7c00);
  int ex;
  const double m = frexp(v, &ex);  /* v = m * 2^ex, m in [0.5, 1) */
  const int E = ex - 1;            /* v = (2m) * 2^E, 2m in [1, 2) */
  if (E < -14) {                   /* subnormal: v = units * 2^-24 */
    const double units = nearbyint(ldexp(v, 24));
    return (uint16_t)(sign | (uint16_t)units);  /* 1024 becomes 2^-14 */
  }
  double frac = nearbyint((2.0 * m - 1.0) * 1024.0);
  int e = E;
  if (frac == 1024.0) {
    frac = 0.0;
    ++e;
  }
  if (e + 15 >= 31) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)frac);
}

uint16_t oracle_f32_to_f16(float f) { return f64_to_f16_bits((double)f); }

/* x [N][K] fp32 -> qx [N][K] int8, dx [N][K/32] binary16 bits. */
int oracle_quantize_act(const float* x, int64_t N, int64_t K, int8_t* qx, uint16_t* dx) {
  if (N < 1 || K <= 0 || K % QK) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t b = 0; b < K / QK; ++b) {
      const float* xb = x + n * K + b * QK;
      float amax = 0.0f;
      for (int j = 0; j < QK; ++j) {
        const float a = fabsf(xb[j]);
        if (a > amax) amax = a;
      }
      const float d = amax / 127.0f;
      for (int j = 0; j < QK; ++j) {
        float q = 0.0f;
        if (amax > 0.0f) q = nearbyintf(xb[j] / d);
        qx[n * K + b * QK + j] = (int8_t)q;
      }
      dx[n * (K / QK) + b] = f64_to_f16_bits((double)d);
    }
  }
  return 0;
}

/* y[n][r] and the magnitude sum S[n][r] = sum_b |dw dx isum_b| (the
 * tolerance's scale): exact integer block sums, scales applied in double
 * (each term is exact: 11 + 11 + 20 bits). */
int oracle_q8_0_gemv_q8act(const uint8_t* aos, int64_t M, int64_t K, const int8_t* qx,
                           const uint16_t* dx, int64_t N, double* y, double* S) {
  if (M < 0 || K <= 0 || K % QK || N < 1) return -1;
  const int64_t nb = K / QK;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t r = 0; r < M; ++r) {
      double acc = 0.0, mag = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = aos + (r * nb + b) * BLOCK_BYTES;
        const uint16_t dbits = (uint16_t)((blk[1] << 8) | blk[0]);  /* little-endian */
        int64_t isum = 0;
        for (int j = 0; j < QK; ++j)
          isum += (int64_t)(int8_t)blk[2 + j] * (int64_t)qx[n * K + b * QK + j];
        const double t =
            oracle_f16_to_f64(dbits) * oracle_f16_to_f64(dx[n * nb + b]) * (double)isum;
        acc += t;
        mag += fabs(t);
      }
      y[n * M + r] = acc;
      if (S) S[n * M + r] = mag;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Q4_K weights (NEXT-2).  [COGNI "Qwen 3.5 Native Metal": cuda_q4k_gemv_probe
 * reads the raw GGUF Q4_K block: d, dmin, 12 bytes of packed scales/mins and
 * 128 bytes of packed nibbles.]  The page lists the fields only; the reading
 * of their packing is the GGUF one.  A 144-byte block holds 256 consecutive
 * weights of one row as 8 sub-blocks of 32:
 *   bytes 0-1    d     binary16, little-endian
 *   bytes 2-3    dmin  binary16, little-endian
 *   bytes 4-15   sc[12]: the 6-bit scale s_j and 6-bit min m_j of sub-block j
 *                  j < 4 : s_j = low 6 bits of sc[j],   m_j = low 6 bits of sc[j+4]
 *                  j >= 4: s_j = low nibble of sc[j+4]  + 16 * (top 2 bits of sc[j-4])
 *                          m_j = high nibble of sc[j+4] + 16 * (top 2 bits of sc[j])
 *   bytes 16-143 qs[128]: the 4-bit quant of weight k lives in byte
 *                  32 * (k / 64) + k % 32, in its low nibble when k % 64 < 32
 *                  (sub-block 2 (k / 64)) and its high nibble otherwise
 *   weight k = d * s_j * q_k - dmin * m_j,  j = k / 32.
 * Blocks of a row are consecutive; rows are consecutive.
 * ------------------------------------------------------------------------- */
#define QKK 256
#define Q4K_BYTES 144

/* The 16-byte header that Q4_K and Q5_K blocks share: d, dmin, and the
 * 6-bit scale and min of sub-block j out of the 12 packed bytes. */
static void kq_header(const uint8_t* b, int j, double* d, double* dmin, int* sj, int* mj) {
  *d = oracle_f16_to_f64((uint16_t)(b[0] | (b[1] << 8)));
  *dmin = oracle_f16_to_f64((uint16_t)(b[2] | (b[3] << 8)));
  const uint8_t* sc = b + 4;
  if (j < 4) {
    *sj = sc[j] & 63;
    *mj = sc[j + 4] & 63;
  } else {
    *sj = (sc[j + 4] & 15) + 16 * (sc[j - 4] >> 6);
    *mj = (sc[j + 4] >> 4) + 16 * (sc[j] >> 6);
  }
}

static double q4k_weight(const uint8_t* blocks, int64_t K, int64_t r, int64_t k) {
  const uint8_t* b = blocks + (r * (K / QKK) + k / QKK) * Q4K_BYTES;
  const int kk = (int)(k % QKK), j = kk / 32;
  double d, dmin;
  int sj, mj;
  kq_header(b, j, &d, &dmin, &sj, &mj);
  const uint8_t byte = b[16 + 32 * (kk / 64) + kk % 32];
  const int q = (kk % 64 < 32) ? (byte & 15) : (byte >> 4);
  return d * (double)sj * (double)q - dmin * (double)mj;
}

void oracle_q4k_dequant_row(const uint8_t* blocks, int64_t K, int64_t r, double* out) {
  for (int64_t k = 0; k < K; ++k) out[k] = q4k_weight(blocks, K, r, k);
}

/* y[n][r] = sum_k w[r][k] * x[n][k] over Q4_K rows (ascending k), with the
 * magnitude sums S; x is fp32 [N][K], widened exactly. */
int oracle_q4k_gemv(const uint8_t* blocks, int64_t M, int64_t K, const float* x, int64_t N,
                    double* y, double* S) {
  if (M < 0 || K <= 0 || K % QKK || N < 1) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t r = 0; r < M; ++r) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double p = q4k_weight(blocks, K, r, k) * (double)x[n * K + k];
        acc = acc + p;
        mag = mag + fabs(p);
      }
      y[n * M + r] = acc;
      if (S) S[n * M + r] = mag;
    }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Q5_K weights (NEXT-2).  [COGNI "Qwen 3.5 Native Metal": cuda_q5k_gemv_probe
 * covers the GGUF Q5_K block of the recurrent layers' attn_qkv.]  Reading of
 * the packing (the page names the format only; the arrangement is GGUF's):
 * a 176-byte block holds 256 weights of one row as 8 sub-blocks of 32, laid
 * out like Q4_K with 32 more bytes for a fifth bit:
 *   bytes 0-15    d, dmin, the 12 scale/min bytes, decoded as for Q4_K
 *   bytes 16-47   qh[32]: the fifth bit of weight k is bit k / 32 of
 *                 qh[k % 32]
 *   bytes 48-175  qs[128]: the low 4 bits of weight k, placed as in Q4_K
 *   weight k = d * s_j * (q_k + 16 * bit_k) - dmin * m_j,  j = k / 32.
 * ------------------------------------------------------------------------- */
#define Q5K_BYTES 176

static double q5k_weight(const uint8_t* blocks, int64_t K, int64_t r, int64_t k) {
  const uint8_t* b = blocks + (r * (K / QKK) + k / QKK) * Q5K_BYTES;
  const int kk = (int)(k % QKK);
  const int j = kk / 32; /* sub-block */
  double d, dmin;
  int s5, m5;
  kq_header(b, j, &d, &dmin, &s5, &m5);
  const uint8_t byte5 = b[48 + 32 * (kk / 64) + kk % 32];
  const int low = (kk % 64 < 32) ? (byte5 & 15) : (byte5 >> 4);
  const int fifth = (b[16 + kk % 32] >> j) & 1;
  return d * (double)s5 * (double)(low + 16 * fifth) - dmin * (double)m5;
}

void oracle_q5k_dequant_row(const uint8_t* blocks, int64_t K, int64_t r, double* out) {
  for (int64_t k = 0; k < K; ++k) out[k] = q5k_weight(blocks, K, r, k);
}

/* y[n][r] = sum_k w[r][k] * x[n][k] over Q5_K rows, with magnitude sums. */
int oracle_q5k_gemv(const uint8_t* blocks, int64_t M, int64_t K, const float* x, int64_t N,
                    double* y, double* S) {
  if (M < 0 || K <= 0 || K % QKK || N < 1) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t r = 0; r < M; ++r) {
      double total = 0.0, absum = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double v = q5k_weight(blocks, K, r, k) * (double)x[n * K + k];
        total = total + v;
        absum = absum + fabs(v);
      }
      y[n * M + r] = total;
      if (S) S[n * M + r] = absum;
    }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Q6_K weights (NEXT-2).  [COGNI "Qwen 3.5 Native Metal": cuda_q6k_gemv_probe
 * covers the GGUF Q6_K block: ql, qh, signed scales, d.]  Reading of the
 * packing (the page lists the fields; the arrangement is GGUF's): a 210-byte
 * block holds 256 weights of one row;
 *   bytes 0-127    ql: low 4 bits of the 6-bit quants
 *   bytes 128-191  qh: high 2 bits
 *   bytes 192-207  16 signed 8-bit scales, one per 16 weights
 *   bytes 208-209  d   binary16, little-endian
 * Weight k (0..255) = 128 h + 32 a + l (h < 2, a < 4, l < 32):
 *   low 4 bits:  byte ql[64 h + 32 (a % 2) + l], low nibble for a < 2, else high
 *   high 2 bits: bits 2a, 2a+1 of qh[32 h + l]
 *   q = low + 16 * high - 32 (so -32..31), weight = d * scale[k / 16] * q.
 * ------------------------------------------------------------------------- */
#define Q6K_BYTES 210

static double q6k_weight(const uint8_t* blocks, int64_t K, int64_t r, int64_t k) {
  const uint8_t* b = blocks + (r * (K / QKK) + k / QKK) * Q6K_BYTES;
  const int kk = (int)(k % QKK);
  const int h = kk / 128, a = (kk % 128) / 32, l = kk % 32;
  const uint8_t lb = b[64 * h + 32 * (a % 2) + l];
  const int low = (a < 2) ? (lb & 15) : (lb >> 4);
  const int high = (b[128 + 32 * h + l] >> (2 * a)) & 3;
  const int q = low + 16 * high - 32;
  const int sc = (int8_t)b[192 + kk / 16];
  const double d = oracle_f16_to_f64((uint16_t)(b[208] | (b[209] << 8)));
  return d * (double)sc * (double)q;
}

void oracle_q6k_dequant_row(const uint8_t* blocks, int64_t K, int64_t r, double* out) {
  for (int64_t k = 0; k < K; ++k) out[k] = q6k_weight(blocks, K, r, k);
}

/* y[n][r] = sum_k w[r][k] * x[n][k] over Q6_K rows, with magnitude sums. */
int oracle_q6k_gemv(const uint8_t* blocks, int64_t M, int64_t K, const float* x, int64_t N,
                    double* y, double* S) {
  if (M < 0 || K <= 0 || K % QKK || N < 1) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t r = 0; r < M; ++r) {
      double sum = 0.0, sabs = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double t = q6k_weight(blocks, K, r, k) * (double)x[n * K + k];
        sum = sum + t;
        sabs = sabs + fabs(t);
      }
      y[n * M + r] = sum;
      if (S) S[n * M + r] = sabs;
    }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Greedy pick: the lowest index among the maxima [AUGUR "Greedy generation";
 * FUSED "API stability": ties resolve to the earliest index].
 * ------------------------------------------------------------------------- */
int64_t oracle_argmax_f32(const float* v, int64_t n) {
  if (n <= 0) return -1;
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

int64_t oracle_argmax_f64(const double* v, int64_t n) {
  if (n <= 0) return -1;
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* ---------------------------------------------------------------------------
 * Router [MOE opening description: router + top-k experts]: the k experts
 * with the largest logits, in descending order, ties to the lower expert
 * index; weights are the softmax over all experts restricted to the chosen
 * ones and renormalised, i.e. exp(l_s - l_max) / sum_{t chosen} exp(l_t -
 * l_max) (the full-softmax denominator cancels in the renormalisation).
 * ------------------------------------------------------------------------- */
int oracle_route_topk(const float* logits, int32_t E, int32_t k, int32_t* ids, double* w) {
  if (E <= 0 || k <= 0 || k > E || E > 4096) return -1;
  char used[4096];
  memset(used, 0, sizeof(used));
  for (int32_t s = 0; s < k; ++s) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (used[e]) continue;
      if (best < 0 || logits[e] > logits[best]) best = e;
    }
    ids[s] = best;
    used[best] = 1;
  }
  double lmax = (double)logits[ids[0]];
  double den = 0.0;
  for (int32_t s = 0; s < k; ++s) den += exp((double)logits[ids[s]] - lmax);
  for (int32_t s = 0; s < k; ++s) w[s] = exp((double)logits[ids[s]] - lmax) / den;
  return 0;
}

/* ---------------------------------------------------------------------------
 * Elementwise glue [AUGUR "Features": RMSNorm, SwiGLU MLP; LUMEN "Phase
 * 7.E.0": silu_mul].
 * ------------------------------------------------------------------------- */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

double oracle_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* h[i] = silu(g[i]) * u[i] */
void oracle_swiglu(const double* g, const double* u, int64_t n, double* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = oracle_silu(g[i]) * u[i];
}

/* Root-mean-square normalisation with unit weight:
 * out[i] = x[i] / sqrt(mean(x^2) + eps). */
void oracle_rmsnorm(const double* x, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double c = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * c;
}

/* Grouped-query attention at position 0 [AUGUR "Grouped-query attention":
 * many query heads share fewer key/value heads].  With a single key the
 * softmax weight is 1, so query head i outputs the value vector of kv head
 * i / (n_heads / n_kv_heads). v is [n_kv_heads][head_dim], out is
 * [n_heads][head_dim]. */
int oracle_gqa_position0(const double* v, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, double* out) {
  if (n_kv_heads <= 0 || n_heads % n_kv_heads) return -1;
  int32_t group = n_heads / n_kv_heads;
  for (int32_t h = 0; h < n_heads; ++h)
    for (int32_t j = 0; j < head_dim; ++j)
      out[(int64_t)h * head_dim + j] = v[(int64_t)(h / group) * head_dim + j];
  return 0;
}

/* ---------------------------------------------------------------------------
 * Mixture-of-experts FFN [MOE opening description and routed-expert fusion
 * comments].  Experts are stacked: expert e's gate_up matrix is the
 * (2I) x H matrix at gu_stack + e * (2I) * (H/32) * 34 bytes, rows 0..I-1
 * gate and I..2I-1 up; its down matrix is H x I at dn_stack + e * H *
 * (I/32) * 34.  The shared expert has the same structure with intermediate
 * Ish.  For each output row the slots are folded in slot order, then the
 * shared expert:  y = sum_s w[s] * down_s(h_s) + sigmoid(lambda) * down_sh(h_sh).
 * ------------------------------------------------------------------------- */

/* Combine stage on given intermediate activations h_routed [S][I] and h_sh
 * [Ish] (double).  Sabs[r] = sum_s |w_s| S_s[r] + |gamma| S_sh[r]. */
int oracle_moe_combine(const uint8_t* dn_stack, int32_t E, int64_t H, int64_t I,
                       const int32_t* ids, const double* w, int32_t S,
                       const double* h_routed, const uint8_t* sh_dn, int64_t Ish,
                       const double* h_sh, double gamma, double* y, double* Sabs,
                       int threads) {
  const int64_t dn_bytes = H * (I / QK) * BLOCK_BYTES;
  double* t = (double*)malloc(sizeof(double) * (size_t)H);
  double* tS = (double*)malloc(sizeof(double) * (size_t)H);
  if (!t || !tS) { free(t); free(tS); return -2; }
  for (int64_t r = 0; r < H; ++r) { y[r] = 0.0; if (Sabs) Sabs[r] = 0.0; }
  for (int32_t s = 0; s < S; ++s) {
    if (ids[s] < 0 || ids[s] >= E) { free(t); free(tS); return -1; }
    oracle_q8_0_gemv_f64(dn_stack + (int64_t)ids[s] * dn_bytes, H, I, h_routed + s * I, 1,
                         t, tS, threads);
    for (int64_t r = 0; r < H; ++r) {
      y[r] += w[s] * t[r];
      if (Sabs) Sabs[r] += fabs(w[s]) * tS[r];
    }
  }
  if (sh_dn) {
    oracle_q8_0_gemv_f64(sh_dn, H, Ish, h_sh, 1, t, tS, threads);
    for (int64_t r = 0; r < H; ++r) {
      y[r] += gamma * t[r];
      if (Sabs) Sabs[r] += fabs(gamma) * tS[r];
    }
  }
  free(t);
  free(tS);
  return 0;
}

/* Whole FFN from x: router weights and ids given (from oracle_route_topk or
 * elsewhere), gamma = sigmoid(lambda) given. */
int oracle_moe_ffn(const uint8_t* gu_stack, const uint8_t* dn_stack, int32_t E, int64_t H,
                   int64_t I, const int32_t* ids, const double* w, int32_t S,
                   const uint8_t* sh_gu, const uint8_t* sh_dn, int64_t Ish, double gamma,
                   const float* x, double* y, int threads) {
  const int64_t gu_bytes = 2 * I * (H / QK) * BLOCK_BYTES;
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  double* gu = (double*)malloc(sizeof(double) * (size_t)(2 * (I > Ish ? I : Ish)));
  double* hr = (double*)malloc(sizeof(double) * (size_t)(S * I + 1));
  double* hs = (double*)malloc(sizeof(double) * (size_t)(Ish + 1));
  if (!xd || !gu || !hr || !hs) { free(xd); free(gu); free(hr); free(hs); return -2; }
  for (int64_t k = 0; k < H; ++k) xd[k] = (double)x[k];
  for (int32_t s = 0; s < S; ++s) {
    if (ids[s] < 0 || ids[s] >= E) { free(xd); free(gu); free(hr); free(hs); return -1; }
    oracle_q8_0_gemv_f64(gu_stack + (int64_t)ids[s] * gu_bytes, 2 * I, H, xd, 1, gu, NULL,
                         threads);
    oracle_swiglu(gu, gu + I, I, hr + s * I);
  }
  if (sh_gu) {
    oracle_q8_0_gemv_f64(sh_gu, 2 * Ish, H, xd, 1, gu, NULL, threads);
    oracle_swiglu(gu, gu + Ish, Ish, hs);
  }
  int rc = oracle_moe_combine(dn_stack, E, H, I, ids, w, S, hr, sh_gu ? sh_dn : NULL, Ish, hs,
                              gamma, y, NULL, threads);
  free(xd);
  free(gu);
  free(hr);
  free(hs);
  return rc;
}

/* ---------------------------------------------------------------------------
 * One decoder layer of the Qwen2-style chain at position 0 [AUGUR "Decoder
 * blocks": norm, attention, residual, norm, MLP, residual; LUMEN "Phase
 * 7.E.0": the qkv, wo, gate_up, silu_mul, down steps].  Unit norm weights, no
 * biases.  h is updated in place (double, length hidden).
 *   a  = rmsnorm(h);  qkv = Wqkv a  (q rows first, then k, then v)
 *   h += Wo * gqa(v);  m = rmsnorm(h);  gu = Wgu m  (gate rows, then up)
 *   h += Wdown * (silu(gate) * up)
 * ------------------------------------------------------------------------- */
int oracle_qwen_layer(const uint8_t* qkv_aos, const uint8_t* wo_aos, const uint8_t* gu_aos,
                      const uint8_t* down_aos, int64_t hidden, int32_t n_heads,
                      int32_t n_kv_heads, int32_t head_dim, int64_t inter, double eps,
                      double* h, int threads) {
  const int64_t qdim = (int64_t)n_heads * head_dim, kvdim = (int64_t)n_kv_heads * head_dim;
  const int64_t nqkv = qdim + 2 * kvdim;
  if (qdim != hidden) return -1;
  double* a = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* qkv = (double*)malloc(sizeof(double) * (size_t)nqkv);
  double* att = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* t = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* gu = (double*)malloc(sizeof(double) * (size_t)(2 * inter));
  double* s = (double*)malloc(sizeof(double) * (size_t)inter);
  int rc = -2;
  if (!a || !qkv || !att || !t || !gu || !s) goto done;
  oracle_rmsnorm(h, hidden, eps, a);
  oracle_q8_0_gemv_f64(qkv_aos, nqkv, hidden, a, 1, qkv, NULL, threads);
  oracle_gqa_position0(qkv + qdim + kvdim, n_heads, n_kv_heads, head_dim, att);
  oracle_q8_0_gemv_f64(wo_aos, hidden, hidden, att, 1, t, NULL, threads);
  for (int64_t i = 0; i < hidden; ++i) h[i] += t[i];
  oracle_rmsnorm(h, hidden, eps, a);
  oracle_q8_0_gemv_f64(gu_aos, 2 * inter, hidden, a, 1, gu, NULL, threads);
  oracle_swiglu(gu, gu + inter, inter, s);
  oracle_q8_0_gemv_f64(down_aos, hidden, inter, s, 1, t, NULL, threads);
  for (int64_t i = 0; i < hidden; ++i) h[i] += t[i];
  rc = 0;
done:
  free(a);
  free(qkv);
  free(att);
  free(t);
  free(gu);
  free(s);
  return rc;
}
