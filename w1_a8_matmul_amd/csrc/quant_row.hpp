// Workgroup-wide quantization of one activation row: absmax, scale, int8
// codes and their sum.  Used by the stand-alone quantizer and by the fused
// prologue of the small-M forward kernels.
#pragma once

#include "common.hpp"

namespace bl {

struct RowQuant {
  float a_c;  // max(max_k |u|, eps), u = x (or x * g with subln)
  float qs;   // 127 / a_c
  float r;    // subln's RMS factor of the row (1 without subln)
};

// Eight consecutive activations as floats (bf16 is widened exactly).
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ X, int64_t idx, float v[8]) {
  if constexpr (DT == 1) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(X) + idx);
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_float(d[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_float(d[i] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(X) + idx);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// max |u| over row m with NT threads; red has NT/64 floats of LDS.  With
// NORM (subln, an RMSNorm with gain g and epsilon eps): u = x * g, and the
// row's RMS factor from the double sum of x^2 (red_d: NT/64 doubles of LDS).
// Absmax quantization cannot see the factor, so it only scales s_x.
template <int DT, int NT, bool NORM = false>
__device__ __forceinline__ RowQuant row_absmax_scale(const void* __restrict__ X, int64_t m,
                                                     int64_t K, float* red,
                                                     const float* __restrict__ g = nullptr,
                                                     float eps = 0.0f,
                                                     double* red_d = nullptr) {
  float amax = 0.0f;
  double ss = 0.0;
  for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += NT * 8) {
    float v[8];
    load8<DT>(X, m * K + k, v);
    if constexpr (NORM) {
      float gv[8];
      load8<0>(g, k, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss = __builtin_fma((double)v[i], (double)v[i], ss);  // exact square: one rounding
        v[i] = v[i] * gv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if constexpr (NORM) ss = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = amax;
    if constexpr (NORM) red_d[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) a = fmaxf(a, red[w]);
  RowQuant r;
  r.r = 1.0f;
  if constexpr (NORM) {
    double S = red_d[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) S += red_d[w];
    r.r = rms_factor(S, K, eps);
  }
  __syncthreads();
  r.a_c = a > kEps ? a : kEps;
  r.qs = kQmax / r.a_c;
  return r;
}

// Writes the int8 codes of row m (of u = x, or x * g with NORM) to dst[0..K)
// and returns their sum (in every thread).  red has NT/64 ints of LDS.
template <int DT, int NT, bool NORM = false>
__device__ __forceinline__ int row_quantize_to(const void* __restrict__ X, int64_t m, int64_t K,
                                               float qs, int8_t* dst, int* red,
                                               const float* __restrict__ g = nullptr) {
  int sum = 0;
  for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += NT * 8) {
    float v[8];
    load8<DT>(X, m * K + k, v);
    if constexpr (NORM) {
      float gv[8];
      load8<0>(g, k, gv);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * gv[i];
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = quant_i8(v[i] * qs);
      sum += q;
      if (i < 4)
        lo |= ((uint32_t)q & 0xffu) << (8 * i);
      else
        hi |= ((uint32_t)q & 0xffu) << (8 * (i - 4));
    }
    *reinterpret_cast<uint2*>(dst + k) = make_uint2(lo, hi);
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += red[w];
  __syncthreads();
  return total;
}

}  // namespace bl
