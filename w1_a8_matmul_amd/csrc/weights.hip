// Offline weight path: absmean scale, ternary quantization and packing into
// the 16x256-tile layout, plus plain pack / unpack of int8 ternary values.
//
// Absmean to {-1, 0, +1} and four ternary weights per byte follow the
// "BitNet b1.58 2B4T Technical Report" card, section "Method Adaptation".
#include "common.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

// One thread per row: sum_k |W[n,k]| in double, strictly in column order,
// so that the result does not depend on the launch shape.
__global__ __launch_bounds__(256) void absmean_rows_kernel(const float* __restrict__ W,
                                                           int64_t N, int64_t K,
                                                           double* __restrict__ row_sum) {
  int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const float4* p = reinterpret_cast<const float4*>(W + n * K);
  double r = 0.0;
  for (int64_t i = 0; i < K / 4; ++i) {
    float4 v = p[i];
    r += fabs((double)v.x);
    r += fabs((double)v.y);
    r += fabs((double)v.z);
    r += fabs((double)v.w);
  }
  row_sum[n] = r;
}

// A single thread adds the row sums in row order and rounds the mean once.
__global__ void absmean_final_kernel(const double* __restrict__ row_sum, int64_t N, int64_t K,
                                     float* __restrict__ gamma) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  double total = 0.0;
  for (int64_t n = 0; n < N; ++n) total += row_sum[n];
  double count = (double)N * (double)K;
  float g = (float)(total / count);
  *gamma = g > kEps ? g : kEps;
}

// Position of packed word w (4 bytes, 16 weights) in the matrix: the tile is
// w / 256; inside it chunk (w % 256) / 4 and word w % 4.  Returns the row and
// the first of the 16 consecutive columns the word holds.
__device__ __forceinline__ void word_origin(int64_t w, int64_t K, int64_t& n, int64_t& k0) {
  const int64_t kblocks = K / kTileCols;
  const int64_t tile = w >> 8;
  const int within = (int)(w & 255);
  const int chunk = within >> 2, word = within & 3;
  const int64_t tile_row = tile / kblocks, kblock = tile - tile_row * kblocks;
  n = tile_row * kTileRows + (chunk & 15);
  k0 = kblock * kTileCols + (chunk >> 4) * 64 + word * 16;
}

// Column offset 4f + e of a word lives in byte e, bits 2f..2f+1.
// Row of W stored at packed row n: itself, or for a fused gate+up matrix
// (glu) the interleaved order, 16-row tile t = gate rows 8t..8t+7, then up
// rows N/2+8t..N/2+8t+7.
__device__ __forceinline__ int64_t source_row(int64_t n, int64_t N, int glu) {
  if (!glu) return n;
  const int64_t t = n / 16, i = n % 16;
  return i < 8 ? 8 * t + i : N / 2 + 8 * t + (i - 8);
}

__global__ __launch_bounds__(256) void quant_pack_kernel(const float* __restrict__ W,
                                                         int64_t N, int64_t K,
                                                         const float* __restrict__ gamma_p,
                                                         uint32_t* __restrict__ out, int glu) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= N * K / 16) return;
  const float gamma = *gamma_p;
  int64_t n, k0;
  word_origin(w, K, n, k0);
  const float4* src = reinterpret_cast<const float4*>(W + source_row(n, N, glu) * K + k0);
  uint32_t word = 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const float4 v = src[f];
    const float vals[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float q = __builtin_rintf(vals[e] / gamma);
      q = fminf(fmaxf(q, -1.0f), 1.0f);
      word |= (uint32_t)((int)q + 1) << (8 * e + 2 * f);
    }
  }
  out[w] = word;
}

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ Wq, int64_t N,
                                                   int64_t K, uint32_t* __restrict__ out) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= N * K / 16) return;
  int64_t n, k0;
  word_origin(w, K, n, k0);
  const uint4 v = *reinterpret_cast<const uint4*>(Wq + n * K + k0);
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  uint32_t word = 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int q = (int)(int8_t)(d[f] >> (8 * e));
      q = q < -1 ? -1 : (q > 1 ? 1 : q);
      word |= (uint32_t)(q + 1) << (8 * e + 2 * f);
    }
  }
  out[w] = word;
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ in, int64_t N,
                                                     int64_t K, int8_t* __restrict__ Wq) {
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= N * K / 16) return;
  int64_t n, k0;
  word_origin(w, K, n, k0);
  const uint32_t word = in[w];
  uint32_t d[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t code = (word >> (8 * e + 2 * f)) & 3u;
      const int q = code == 3u ? 0 : (int)code - 1;
      out |= ((uint32_t)q & 0xffu) << (8 * e);
    }
    d[f] = out;
  }
  *reinterpret_cast<uint4*>(Wq + n * K + k0) = make_uint4(d[0], d[1], d[2], d[3]);
}

// ---- The base-3 layout: five codes per byte (1.6 bits per weight) ----
// A ternary weight carries log2(3) bits ("1.58-bit large language model",
// wikiprompt.org, introduction).  K is padded to Kp, a multiple of 320;
// tiles of 16 rows x 320 columns (1 KiB); 16-byte chunk c of a tile holds
// row c % 16 and columns 80 (c / 16) .. +79 of its block; byte b of 32-bit
// word j of a chunk holds the codes of columns 20j + 4i + b as the base-3
// number sum_i code_i 3^i (i = 0..4).  Padding columns hold code 0.

// Position of packed word d (20 columns): row n and first column k0.
__device__ __forceinline__ void b3_word_origin(int64_t d, int64_t Kp, int64_t& n, int64_t& k0) {
  const int64_t kblocks = Kp / kB3TileCols;
  const int64_t tile = d >> 8;
  const int within = (int)(d & 255);
  const int chunk = within >> 2, word = within & 3;
  const int64_t tile_row = tile / kblocks, kblock = tile - tile_row * kblocks;
  n = tile_row * kTileRows + (chunk & 15);
  k0 = kblock * kB3TileCols + (chunk >> 4) * 80 + word * 20;
}

// The word from the codes (0, 1, 2) of its 20 columns, c[u] for column
// k0 + u: byte b = sum_i c[4i + b] 3^i.
__device__ __forceinline__ uint32_t b3_word_from_codes(const int (&c)[20]) {
  uint32_t word = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int v = 0;
#pragma unroll
    for (int i = 4; i >= 0; --i) v = v * 3 + c[4 * i + b];
    word |= (uint32_t)v << (8 * b);
  }
  return word;
}

__global__ __launch_bounds__(256) void quant_pack_b3_kernel(const float* __restrict__ W,
                                                            int64_t N, int64_t K, int64_t Kp,
                                                            const float* __restrict__ gamma_p,
                                                            uint32_t* __restrict__ out,
                                                            int glu) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= N * Kp / 20) return;
  const float gamma = *gamma_p;
  int64_t n, k0;
  b3_word_origin(d, Kp, n, k0);
  const float* row = W + source_row(n, N, glu) * K;
  int c[20];
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    // K is a multiple of 16 and k0 of 20: each group of 4 lies wholly
    // inside or wholly past the row.
    const bool in = k0 + 4 * t < K;
    const float4 v = in ? *reinterpret_cast<const float4*>(row + k0 + 4 * t)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    const float vals[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float q = __builtin_rintf(vals[e] / gamma);
      q = fminf(fmaxf(q, -1.0f), 1.0f);
      c[4 * t + e] = in ? (int)q + 1 : 0;
    }
  }
  out[d] = b3_word_from_codes(c);
}

__global__ __launch_bounds__(256) void pack_b3_kernel(const int8_t* __restrict__ Wq, int64_t N,
                                                      int64_t K, int64_t Kp,
                                                      uint32_t* __restrict__ out) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= N * Kp / 20) return;
  int64_t n, k0;
  b3_word_origin(d, Kp, n, k0);
  int c[20];
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const bool in = k0 + 4 * t < K;
    const uint32_t v = in ? *reinterpret_cast<const uint32_t*>(Wq + n * K + k0 + 4 * t) : 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int q = (int)(int8_t)(v >> (8 * e));
      q = q < -1 ? -1 : (q > 1 ? 1 : q);
      c[4 * t + e] = in ? q + 1 : 0;
    }
  }
  out[d] = b3_word_from_codes(c);
}

__global__ __launch_bounds__(256) void unpack_b3_kernel(const uint32_t* __restrict__ in,
                                                        int64_t N, int64_t K, int64_t Kp,
                                                        int8_t* __restrict__ Wq) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= N * Kp / 20) return;
  int64_t n, k0;
  b3_word_origin(d, Kp, n, k0);
  const uint32_t word = in[d];
  int c[20];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int v = (int)((word >> (8 * b)) & 0xffu);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      c[4 * i + b] = v % 3;
      v /= 3;
    }
  }
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    if (k0 + 4 * t >= K) break;
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) v |= ((uint32_t)(c[4 * t + e] - 1) & 0xffu) << (8 * e);
    *reinterpret_cast<uint32_t*>(Wq + n * K + k0 + 4 * t) = v;
  }
}

inline unsigned grid_for(int64_t items, int block) {
  return (unsigned)((items + block - 1) / block);
}

}  // namespace

hipError_t bl_launch_absmean_rows(const float* W, int64_t N, int64_t K, double* row_sum,
                                  hipStream_t s) {
  hipLaunchKernelGGL(absmean_rows_kernel, dim3(grid_for(N, 256)), dim3(256), 0, s, W, N, K,
                     row_sum);
  return hipGetLastError();
}

hipError_t bl_launch_absmean_final(const double* row_sum, int64_t N, int64_t K, float* gamma,
                                   hipStream_t s) {
  hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(64), 0, s, row_sum, N, K, gamma);
  return hipGetLastError();
}

hipError_t bl_launch_quant_pack(const float* W, int64_t N, int64_t K, const float* gamma,
                                uint8_t* packed, hipStream_t s, bool glu) {
  const int64_t words = N * K / 16;
  hipLaunchKernelGGL(quant_pack_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, W, N, K,
                     gamma, reinterpret_cast<uint32_t*>(packed), glu ? 1 : 0);
  return hipGetLastError();
}

hipError_t bl_launch_pack(const int8_t* Wq, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t s) {
  const int64_t words = N * K / 16;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, Wq, N, K,
                     reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t bl_launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wq,
                            hipStream_t s) {
  const int64_t words = N * K / 16;
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(packed), N, K, Wq);
  return hipGetLastError();
}

hipError_t bl_launch_quant_pack_b3(const float* W, int64_t N, int64_t K, const float* gamma,
                                   uint8_t* packed, hipStream_t s, bool glu) {
  const int64_t Kp = bl_b3_padded_k(K);
  const int64_t words = N * Kp / 20;
  hipLaunchKernelGGL(quant_pack_b3_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, W, N, K,
                     Kp, gamma, reinterpret_cast<uint32_t*>(packed), glu ? 1 : 0);
  return hipGetLastError();
}

hipError_t bl_launch_pack_b3(const int8_t* Wq, int64_t N, int64_t K, uint8_t* packed,
                             hipStream_t s) {
  const int64_t Kp = bl_b3_padded_k(K);
  const int64_t words = N * Kp / 20;
  hipLaunchKernelGGL(pack_b3_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s, Wq, N, K, Kp,
                     reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t bl_launch_unpack_b3(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wq,
                               hipStream_t s) {
  const int64_t Kp = bl_b3_padded_k(K);
  const int64_t words = N * Kp / 20;
  hipLaunchKernelGGL(unpack_b3_kernel, dim3(grid_for(words, 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(packed), N, K, Kp, Wq);
  return hipGetLastError();
}
