/*
 * CPU oracle for the W1.58A8 BitLinear forward.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path (the HIP library and
 * its Python binding) never calls it and shares no source with it.
 *
 * Sources (the web pages this method is described on):
 *   [TR]  "BitNet b1.58 2B4T Technical Report" paper card, ai-papers.xuzou.cn,
 *         sections "Method Adaptation" and "Compute Setup".
 *   [FA]  fishai news digest on BitNet b1.58 2B4T, news.fishai.com.cn/news/3455510,
 *         the list of what a BitLinear layer contains (weight quantization,
 *         activation quantization).
 *   [DN]  dignews.cc article on the open BitNet b1.58 2B4T model, section 2
 *         (core architectural innovations).
 *   [WP]  wikiprompt.org entry "1.58-bit large language model", introduction.
 *
 * The pages state what is computed in words only: weights are mapped to
 * {-1, 0, +1} with an absmean scheme, activations are mapped per token to
 * 8-bit integers with an absmax scheme, four ternary weights share one byte,
 * and the product runs as an int8 matmul.  They give no formula, epsilon,
 * rounding rule or bit layout.  The readings taken here are:
 *
 *   R1 gamma   = mean |W| over the whole matrix, the sum taken in double:
 *                each row sequentially from 0.0, then the row sums in row order;
 *                one rounding of the double mean to float.
 *                gamma_c = max(gamma, 1e-5f) guards an all-zero matrix.
 *   R2 q_w     = clamp(rint(W / gamma_c), -1, +1); float division, ties to even.
 *   R3 code    = q_w + 1 in {0, 1, 2}; code 3 never occurs.  Layout: see
 *                oracle_pack below (16-row x 256-column tiles of 1 KiB).
 *   R4 a_m     = max_k |x[m,k]|, a_c = max(a_m, 1e-5f), qs = 127 / a_c (float),
 *                q_x = clamp(rint(x * qs), -127, 127), s_x = a_c / 127 (float).
 *                bf16 input is widened to float exactly before anything else.
 *   R5 acc     = sum_k q_x * q_w, exact in int32.
 *   R6 y       = (float)((float)((float)acc * s_x) * gamma_c), left to right,
 *                no fused multiply-add.
 *   R7 ReLU^2  = h = r * r with r = max(y, 0) (a -0 input gives +0).
 *   R8 subln   = the normalization a BitLinear layer contains, read as RMSNorm
 *                of each token's K inputs with a per-feature gain g:
 *                x_hat = x * r * g, r = 1 / sqrt(mean_k x^2 + eps_n), then R4
 *                on x_hat.  Absmax quantization does not see a positive
 *                factor shared by the row, so the codes are R4's codes of
 *                u = x * g (one float product per element) and r enters the
 *                scale only: s_x = (float)(s_x(u) * r).  The sum of squares is
 *                taken in double in index order; r = (float)(1 / sqrt(S / K +
 *                eps_n)) in double.  The 1e-5 guard of R4 applies to u.
 *   R13 base-3 = the denser layout: five codes per byte as a base-3 number,
 *                in tiles of 16 rows by 320 columns (see oracle_pack_b3).
 *   R12 gated FFN = the workload's fused gate+up matrix [N][K] holds the gate
 *                rows 0..F-1 and the up rows F..2F-1 (F = N/2), with one gamma;
 *                h = (r * r) * y_up, r = max(y_gate, 0), left to right, float,
 *                no fused multiply-add; h is [M][F].  The pages give ReLU^2 as
 *                the FFN activation and no formula for the gating.  The packed
 *                layout of such a matrix interleaves the halves: 16-row tile t
 *                holds gate rows 8t..8t+7, then up rows F+8t..F+8t+7.
 *
 * All float arithmetic here is IEEE binary32/binary64 with round-to-nearest-
 * even; the file must be compiled without fast-math and with
 * -ffp-contract=off so that no operation is fused or reassociated.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_EPS 1e-5f

int oracle_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------------- */
/* R1: absmean weight scale ([TR] Method Adaptation; [FA] weight quantization;
 * [DN] section 2).  Writes the unguarded mean and the guarded scale.        */
void oracle_absmean(const float* W, int64_t N, int64_t K, float* gamma_raw,
                    float* gamma_c) {
  double* row_sum = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  int64_t n;
#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    double r = 0.0;
    for (int64_t k = 0; k < K; ++k) r += fabs((double)W[n * K + k]);
    row_sum[n] = r;
  }
  double total = 0.0;
  for (n = 0; n < N; ++n) total += row_sum[n];
  free(row_sum);
  double count = (double)N * (double)K;
  float g = (float)(total / count);
  *gamma_raw = g;
  *gamma_c = g > ORACLE_EPS ? g : ORACLE_EPS;
}

/* R2: ternary value of every weight, given the guarded scale.              */
void oracle_ternarize(const float* W, int64_t count, float gamma_c, int8_t* q) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < count; ++i) {
    float v = rintf(W[i] / gamma_c);
    if (v > 1.0f) v = 1.0f;
    if (v < -1.0f) v = -1.0f;
    q[i] = (int8_t)v;
  }
}

/* ---------------------------------------------------------------------- */
/* R3: packed layout.  The pages say only that four ternary weights are
 * stored in one byte ([TR] Method Adaptation; [DN] section 2).  The layout
 * is this library's own: the matrix is cut into tiles of 16 rows by 256
 * columns; a tile is 1024 bytes, tiles are ordered row-tile major, then by
 * column block.  Inside a tile, 16-byte chunk c holds row (c mod 16) and
 * the 64 columns 64*(c div 16) .. +63 of the block; inside a chunk, column
 * offset t (0..63) sits in 32-bit word t div 16, byte (t mod 4), bits
 * 2*((t mod 16) div 4) and the one above.                                  */
static int64_t packed_byte_index(int64_t n, int64_t k, int64_t K, int* shift) {
  int64_t tile_row = n / 16, row_in_tile = n % 16;
  int64_t kblock = k / 256, kb = k % 256;
  int64_t sub = kb / 64, t = kb % 64;
  int64_t word = t / 16, field = (t % 16) / 4, byte_in_word = t % 4;
  int64_t chunk = sub * 16 + row_in_tile;
  int64_t tile = tile_row * (K / 256) + kblock;
  *shift = (int)(2 * field);
  return tile * 1024 + chunk * 16 + word * 4 + byte_in_word;
}

int64_t oracle_packed_bytes(int64_t N, int64_t K) { return N * K / 4; }

/* Returns 0 on success, -1 if the shape is outside the layout's domain or a
 * value is not ternary.                                                    */
int oracle_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
  if (N % 16 != 0 || K % 256 != 0) return -1;
  memset(packed, 0, (size_t)(N * K / 4));
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      int8_t v = q[n * K + k];
      if (v < -1 || v > 1) return -1;
      int shift;
      int64_t at = packed_byte_index(n, k, K, &shift);
      packed[at] |= (uint8_t)((v + 1) << shift);
    }
  }
  return 0;
}

/* Returns 0 on success, -1 on a bad shape or if a code 3 is met.           */
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q) {
  if (N % 16 != 0 || K % 256 != 0) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      int shift;
      int64_t at = packed_byte_index(n, k, K, &shift);
      int code = (packed[at] >> shift) & 3;
      if (code == 3) return -1;
      q[n * K + k] = (int8_t)(code - 1);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* R13: the denser packed layout, five ternary codes per byte.  A ternary
 * weight carries log2(3), about 1.58 bits ([WP] introduction); the 2B
 * model's weights take 0.4 GB at that density ([TR] Evidence).  Five codes
 * c = q + 1 in {0, 1, 2} fit one byte as the base-3 number
 * c_0 + 3 c_1 + 9 c_2 + 27 c_3 + 81 c_4 (0..242), 1.6 bits per weight.  The
 * layout is this library's own: K is padded up to Kp, a multiple of 320,
 * and the matrix is cut into tiles of 16 rows by 320 columns (1024 bytes),
 * ordered row-tile major, then by column block.  Inside a tile, 16-byte
 * chunk c holds row (c mod 16) and the 80 columns 80*(c div 16) .. +79 of
 * the block; inside a chunk, byte b (0..3) of 32-bit word j (0..3) holds
 * the codes of columns 20j + 4i + b, i = 0..4, digit i being column
 * 20j + 4i + b.  Padding columns (K <= k < Kp) hold code 0.                */
static int64_t b3_padded_k(int64_t K) { return (K + 319) / 320 * 320; }

int64_t oracle_packed_bytes_b3(int64_t N, int64_t K) { return N * b3_padded_k(K) / 5; }

/* Byte index and digit of weight (n, k) in the base-3 layout (k < Kp).     */
static int64_t b3_byte_index(int64_t n, int64_t k, int64_t Kp, int* digit) {
  int64_t tile_row = n / 16, row_in_tile = n % 16;
  int64_t kblock = k / 320, kb = k % 320;
  int64_t quarter = kb / 80, t = kb % 80;      /* chunk column offset 0..79 */
  int64_t word = t / 20, u = t % 20;           /* u = 4i + b                */
  int64_t byte_in_word = u % 4;
  int64_t chunk = quarter * 16 + row_in_tile;
  int64_t tile = tile_row * (Kp / 320) + kblock;
  *digit = (int)(u / 4);
  return tile * 1024 + chunk * 16 + word * 4 + byte_in_word;
}

/* Returns 0 on success, -1 if N % 16 != 0, K % 16 != 0 or a value is not
 * ternary.                                                                 */
int oracle_pack_b3(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
  if (N % 16 != 0 || K % 16 != 0 || N < 0 || K < 0) return -1;
  const int64_t Kp = b3_padded_k(K);
  const int pow3[5] = {1, 3, 9, 27, 81};
  memset(packed, 0, (size_t)(N * Kp / 5));
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      int8_t v = q[n * K + k];
      if (v < -1 || v > 1) return -1;
      int digit;
      int64_t at = b3_byte_index(n, k, Kp, &digit);
      packed[at] = (uint8_t)(packed[at] + (v + 1) * pow3[digit]);
    }
  }
  return 0;
}

/* Returns 0 on success, -1 on a bad shape, a byte above 242 or a padding
 * column whose code is not 0.                                              */
int oracle_unpack_b3(const uint8_t* packed, int64_t N, int64_t K, int8_t* q) {
  if (N % 16 != 0 || K % 16 != 0 || N < 0 || K < 0) return -1;
  const int64_t Kp = b3_padded_k(K);
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t k = 0; k < Kp; ++k) {
      int digit;
      int64_t at = b3_byte_index(n, k, Kp, &digit);
      int v = packed[at];
      if (v > 242) return -1;
      for (int i = 0; i < digit; ++i) v /= 3;
      int code = v % 3;
      if (k >= K) {
        if (code != 0) return -1;
        continue;
      }
      q[n * K + k] = (int8_t)(code - 1);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* R4: per-token absmax activation quantization ([TR] Method Adaptation;
 * [FA] activation quantization).  One row of floats.                      */
static void quant_row(const float* x, int64_t K, int8_t* q, float* s_x,
                      int32_t* rowsum) {
  float a = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float m = fabsf(x[k]);
    if (m > a) a = m;
  }
  float a_c = a > ORACLE_EPS ? a : ORACLE_EPS;
  float qs = 127.0f / a_c;
  int32_t sum = 0;
  for (int64_t k = 0; k < K; ++k) {
    float v = rintf(x[k] * qs);
    if (v > 127.0f) v = 127.0f;
    if (v < -127.0f) v = -127.0f;
    q[k] = (int8_t)v;
    sum += q[k];
  }
  *s_x = a_c / 127.0f;
  if (rowsum) *rowsum = sum;
}

void oracle_quant_acts_f32(const float* X, int64_t M, int64_t K, int8_t* q,
                           float* s_x, int32_t* rowsum) {
  int64_t m;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m)
    quant_row(X + m * K, K, q + m * K, s_x + m, rowsum ? rowsum + m : NULL);
}

/* bf16 bits widen to float by placing them in the top half of the word.   */
static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

void oracle_quant_acts_bf16(const uint16_t* X, int64_t M, int64_t K, int8_t* q,
                            float* s_x, int32_t* rowsum) {
  int64_t m;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m) {
    float* row = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    for (int64_t k = 0; k < K; ++k) row[k] = bf16_to_float(X[m * K + k]);
    quant_row(row, K, q + m * K, s_x + m, rowsum ? rowsum + m : NULL);
    free(row);
  }
}

/* ---------------------------------------------------------------------- */
/* R8: subln before the activation quantization ([FA] the list of what a
 * BitLinear layer contains: normalization; [TR] Method Adaptation).  One row
 * of floats x, gains g.                                                    */
static void quant_row_rmsnorm(const float* x, const float* g, int64_t K, float eps_n,
                              int8_t* q, float* s_x, int32_t* rowsum) {
  float* u = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
  double S = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double d = (double)x[k];
    S += d * d;
    u[k] = x[k] * g[k];
  }
  float r = (float)(1.0 / sqrt(S / (double)K + (double)eps_n));
  quant_row(u, K, q, s_x, rowsum);
  *s_x = *s_x * r;
  free(u);
}

void oracle_quant_acts_rmsnorm_f32(const float* X, const float* g, float eps_n, int64_t M,
                                   int64_t K, int8_t* q, float* s_x, int32_t* rowsum) {
  int64_t m;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m)
    quant_row_rmsnorm(X + m * K, g, K, eps_n, q + m * K, s_x + m, rowsum ? rowsum + m : NULL);
}

void oracle_quant_acts_rmsnorm_bf16(const uint16_t* X, const float* g, float eps_n,
                                    int64_t M, int64_t K, int8_t* q, float* s_x,
                                    int32_t* rowsum) {
  int64_t m;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m) {
    float* row = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    for (int64_t k = 0; k < K; ++k) row[k] = bf16_to_float(X[m * K + k]);
    quant_row_rmsnorm(row, g, K, eps_n, q + m * K, s_x + m, rowsum ? rowsum + m : NULL);
    free(row);
  }
}

/* ---------------------------------------------------------------------- */
/* R5: exact integer contraction of int8 activations with unpacked ternary
 * weights ([TR] Compute Setup, Method Adaptation: an int8 matmul).
 * qw is [N][K] with values in {-1, 0, 1}; acc is [M][N].                  */
void oracle_int_matmul(const int8_t* qx, const int8_t* qw, int64_t M, int64_t N,
                       int64_t K, int32_t* acc) {
  int64_t mn;
#pragma omp parallel for schedule(static)
  for (mn = 0; mn < M * N; ++mn) {
    int64_t m = mn / N, n = mn % N;
    int32_t s = 0;
    for (int64_t k = 0; k < K; ++k)
      s += (int32_t)qx[m * K + k] * (int32_t)qw[n * K + k];
    acc[mn] = s;
  }
}

/* The same sum for a list of (m, n) pairs only, for spot checks at sizes
 * where the full product is too slow for a test.                          */
void oracle_int_dot_samples(const int8_t* qx, const int8_t* qw, int64_t K,
                            const int64_t* m_idx, const int64_t* n_idx,
                            int64_t count, int32_t* out) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < count; ++i) {
    const int8_t* a = qx + m_idx[i] * K;
    const int8_t* b = qw + n_idx[i] * K;
    int32_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += (int32_t)a[k] * (int32_t)b[k];
    out[i] = s;
  }
}

/* R6: float rescale by the activation scale, then the weight scale.       */
void oracle_rescale(const int32_t* acc, const float* s_x, float gamma_c,
                    int64_t M, int64_t N, float* y) {
  int64_t mn;
#pragma omp parallel for schedule(static)
  for (mn = 0; mn < M * N; ++mn) {
    float t = (float)acc[mn] * s_x[mn / N];
    y[mn] = t * gamma_c;
  }
}

/* R7: squared ReLU ([TR] Method Adaptation; [FA] FFN activation).         */
void oracle_relu2(const float* y, int64_t count, float* h) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < count; ++i) {
    float r = y[i] > 0.0f ? y[i] : 0.0f;
    h[i] = r * r;
  }
}

/* R12: the gated squared ReLU of a fused gate+up output, and the packing of
 * such a matrix ([TR] Method Adaptation; [FA] FFN activation: ReLU^2).     */
static int64_t glu_source_row(int64_t p, int64_t N) {
  int64_t t = p / 16, i = p % 16;
  return i < 8 ? 8 * t + i : N / 2 + 8 * t + (i - 8);
}

/* Packs q [N][K] (gate rows first) in the interleaved row order; 0, or -1
 * as oracle_pack.                                                          */
int oracle_pack_glu(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
  if (N % 16 != 0 || K % 256 != 0) return -1;
  int8_t* perm = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
  for (int64_t p = 0; p < N; ++p)
    memcpy(perm + p * K, q + glu_source_row(p, N) * K, (size_t)K);
  int r = oracle_pack(perm, N, K, packed);
  free(perm);
  return r;
}

void oracle_glu_relu2(const float* y, int64_t M, int64_t N, float* h) {
  int64_t F = N / 2, m;
#pragma omp parallel for schedule(static)
  for (m = 0; m < M; ++m) {
    for (int64_t f = 0; f < F; ++f) {
      float g = y[m * N + f];
      float r = g > 0.0f ? g : 0.0f;
      float t = r * r;
      h[m * F + f] = t * y[m * N + F + f];
    }
  }
}

/* ---------------------------------------------------------------------- */
/* The whole per-token forward for one layer: quantize X (dtype 0 = float,
 * 1 = bf16 bits), contract with the ternary weights, rescale.  Any of
 * xq, s_x, acc may be NULL when the caller does not want them.            */
int oracle_forward(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                   const int8_t* qw, float gamma_c, float* y, int8_t* xq_out,
                   float* sx_out, int32_t* acc_out) {
  if (dtype != 0 && dtype != 1) return -1;
  int8_t* xq = xq_out ? xq_out : (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
  float* sx = sx_out ? sx_out : (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
  int32_t* acc = acc_out ? acc_out
                         : (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * N > 0 ? M * N : 1));
  if (dtype == 0)
    oracle_quant_acts_f32((const float*)X, M, K, xq, sx, NULL);
  else
    oracle_quant_acts_bf16((const uint16_t*)X, M, K, xq, sx, NULL);
  oracle_int_matmul(xq, qw, M, N, K, acc);
  oracle_rescale(acc, sx, gamma_c, M, N, y);
  if (!xq_out) free(xq);
  if (!sx_out) free(sx);
  if (!acc_out) free(acc);
  return 0;
}
