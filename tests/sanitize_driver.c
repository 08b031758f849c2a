/*
 * Drives every function of the CPU oracle (oracle/bitlinear_oracle.c) on
 * small and edge-case shapes, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles the two
 * files together with gcc and runs the result).  The checks here are
 * consistency checks only (pack/unpack round trip, forward = its parts); the
 * oracle's values are pinned elsewhere.  Exit status 0 means every call
 * behaved and every check held.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_absmean(const float* W, int64_t N, int64_t K, float* gamma_raw, float* gamma_c);
void oracle_ternarize(const float* W, int64_t count, float gamma_c, int8_t* q);
int64_t oracle_packed_bytes(int64_t N, int64_t K);
int oracle_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed);
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q);
void oracle_quant_acts_f32(const float* X, int64_t M, int64_t K, int8_t* q, float* s_x,
                           int32_t* rowsum);
void oracle_quant_acts_bf16(const uint16_t* X, int64_t M, int64_t K, int8_t* q, float* s_x,
                            int32_t* rowsum);
void oracle_quant_acts_rmsnorm_f32(const float* X, const float* g, float eps_n, int64_t M,
                                   int64_t K, int8_t* q, float* s_x, int32_t* rowsum);
void oracle_quant_acts_rmsnorm_bf16(const uint16_t* X, const float* g, float eps_n, int64_t M,
                                    int64_t K, int8_t* q, float* s_x, int32_t* rowsum);
void oracle_int_matmul(const int8_t* qx, const int8_t* qw, int64_t M, int64_t N, int64_t K,
                       int32_t* acc);
void oracle_int_dot_samples(const int8_t* qx, const int8_t* qw, int64_t K, const int64_t* m_idx,
                            const int64_t* n_idx, int64_t count, int32_t* out);
void oracle_rescale(const int32_t* acc, const float* s_x, float gamma_c, int64_t M, int64_t N,
                    float* y);
void oracle_relu2(const float* y, int64_t count, float* h);
int oracle_pack_glu(const int8_t* q, int64_t N, int64_t K, uint8_t* packed);
int64_t oracle_packed_bytes_b3(int64_t N, int64_t K);
int oracle_pack_b3(const int8_t* q, int64_t N, int64_t K, uint8_t* packed);
int oracle_unpack_b3(const uint8_t* packed, int64_t N, int64_t K, int8_t* q);
void oracle_glu_relu2(const float* y, int64_t M, int64_t N, float* h);
int oracle_forward(const void* X, int dtype, int64_t M, int64_t K, int64_t N, const int8_t* qw,
                   float gamma_c, float* y, int8_t* xq_out, float* sx_out, int32_t* acc_out);

static int failures = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {  /* xorshift64*, a test-only stream */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}
static float next_f(float scale) {
  return scale * ((float)(next_u32() & 0xffffff) / 8388608.0f - 1.0f);
}

static void one_shape(int64_t M, int64_t N, int64_t K) {
  const int64_t nk = N * K, mk = M * K, mn = M * N;
  float* W = malloc(sizeof(float) * (size_t)(nk > 0 ? nk : 1));
  int8_t* q = malloc((size_t)(nk > 0 ? nk : 1));
  int8_t* q2 = malloc((size_t)(nk > 0 ? nk : 1));
  uint8_t* p = malloc((size_t)(nk / 4 > 0 ? nk / 4 : 1));
  float* X = malloc(sizeof(float) * (size_t)(mk > 0 ? mk : 1));
  uint16_t* Xb = malloc(sizeof(uint16_t) * (size_t)(mk > 0 ? mk : 1));
  float* g = malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
  int8_t* xq = malloc((size_t)(mk > 0 ? mk : 1));
  float* sx = malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
  int32_t* rs = malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
  int32_t* acc = malloc(sizeof(int32_t) * (size_t)(mn > 0 ? mn : 1));
  int32_t* acc2 = malloc(sizeof(int32_t) * (size_t)(mn > 0 ? mn : 1));
  float* y = malloc(sizeof(float) * (size_t)(mn > 0 ? mn : 1));
  float* y2 = malloc(sizeof(float) * (size_t)(mn > 0 ? mn : 1));
  float* h = malloc(sizeof(float) * (size_t)(mn > 0 ? mn : 1));
  for (int64_t i = 0; i < nk; ++i) W[i] = next_f(0.05f);
  if (N > 1) memset(W + K, 0, sizeof(float) * (size_t)K); /* an all-zero row */
  for (int64_t i = 0; i < mk; ++i) {
    X[i] = next_f(3.0f);
    Xb[i] = (uint16_t)(next_u32() & 0x3fff) | (uint16_t)((next_u32() & 1) << 15);
  }
  if (M > 1) memset(X + K, 0, sizeof(float) * (size_t)K); /* an all-zero token */
  for (int64_t k = 0; k < K; ++k) g[k] = 0.5f + next_f(0.5f) * 0.5f + 0.5f;

  float gr, gc;
  oracle_absmean(W, N, K, &gr, &gc);
  oracle_ternarize(W, nk, gc, q);
  CHECK(oracle_packed_bytes(N, K) == nk / 4);
  if (N % 16 == 0 && K % 256 == 0) { /* the layout's domain (empty shapes included) */
    CHECK(oracle_pack(q, N, K, p) == 0);
    CHECK(oracle_unpack(p, N, K, q2) == 0);
    CHECK(memcmp(q, q2, (size_t)nk) == 0);
    CHECK(oracle_pack_glu(q, N, K, p) == 0);
  } else {
    CHECK(oracle_pack(q, N, K, p) == -1);
    CHECK(oracle_unpack(p, N, K, q2) == -1);
    CHECK(oracle_pack_glu(q, N, K, p) == -1);
  }
  {
    const int64_t nb = oracle_packed_bytes_b3(N, K);
    uint8_t* p3 = malloc((size_t)(nb > 0 ? nb : 1));
    if (N % 16 == 0 && K % 16 == 0) {
      CHECK(oracle_pack_b3(q, N, K, p3) == 0);
      CHECK(oracle_unpack_b3(p3, N, K, q2) == 0);
      CHECK(memcmp(q, q2, (size_t)nk) == 0);
    } else {
      CHECK(oracle_pack_b3(q, N, K, p3) == -1);
      CHECK(oracle_unpack_b3(p3, N, K, q2) == -1);
    }
    free(p3);
  }
  oracle_quant_acts_f32(X, M, K, xq, sx, rs);
  oracle_quant_acts_f32(X, M, K, xq, sx, NULL);
  oracle_quant_acts_bf16(Xb, M, K, xq, sx, rs);
  oracle_quant_acts_rmsnorm_f32(X, g, 1e-5f, M, K, xq, sx, rs);
  oracle_quant_acts_rmsnorm_bf16(Xb, g, 1e-5f, M, K, xq, sx, NULL);
  oracle_quant_acts_f32(X, M, K, xq, sx, rs);
  oracle_int_matmul(xq, q, M, N, K, acc);
  oracle_rescale(acc, sx, gc, M, N, y);
  oracle_relu2(y, mn, h);
  if (N % 2 == 0) oracle_glu_relu2(y, M, N, h);
  CHECK(oracle_forward(X, 0, M, K, N, q, gc, y2, NULL, NULL, acc2) == 0);
  CHECK(memcmp(acc, acc2, sizeof(int32_t) * (size_t)mn) == 0);
  CHECK(memcmp(y, y2, sizeof(float) * (size_t)mn) == 0);
  CHECK(oracle_forward(Xb, 1, M, K, N, q, gc, y2, xq, sx, acc2) == 0);
  CHECK(oracle_forward(X, 2, M, K, N, q, gc, y2, NULL, NULL, NULL) == -1);
  if (M > 0 && N > 0) {
    int64_t mi[3] = {0, M - 1, M / 2}, ni[3] = {N - 1, 0, N / 2};
    int32_t out[3];
    oracle_int_dot_samples(xq, q, K, mi, ni, 3, out);
    for (int i = 0; i < 3; ++i) CHECK(out[i] == acc2[mi[i] * N + ni[i]]);
  }
  free(W); free(q); free(q2); free(p); free(X); free(Xb); free(g); free(xq);
  free(sx); free(rs); free(acc); free(acc2); free(y); free(y2); free(h);
}

int main(void) {
  const int64_t shapes[][3] = {{4, 256, 256}, {1, 16, 256}, {3, 48, 768}, {0, 16, 256},
                               {2, 16, 0},    {5, 15, 256}, {2, 16, 100}, {7, 32, 512},
                               {1, 0, 256},   {2, 16, 336}, {3, 32, 6912}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
    one_shape(shapes[i][0], shapes[i][1], shapes[i][2]);
  /* invalid codes: a byte with code 3 must be rejected */
  uint8_t bad[1024];
  int8_t out[16 * 256];
  memset(bad, 0xff, sizeof bad);
  CHECK(oracle_unpack(bad, 16, 256, out) == -1);
  /* a non-ternary value must be rejected by the packer */
  int8_t two[16 * 256];
  memset(two, 2, sizeof two);
  CHECK(oracle_pack(two, 16, 256, bad) == -1);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("sanitize driver ok\n");
  return 0;
}
