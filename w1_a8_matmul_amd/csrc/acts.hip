// Per-token absmax int8 quantization of activations (fishai news digest on
// BitNet b1.58 2B4T, activation-quantization item; "BitNet b1.58 2B4T
// Technical Report" card, Method Adaptation), optionally after subln read as
// an RMSNorm with a per-feature gain (fishai digest, list of BitLinear parts:
// normalization).  One workgroup per token.
#include "common.hpp"
#include "gemv_tile.hpp"
#include "quant_row.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

template <int DT, bool NORM>
__global__ __launch_bounds__(256) void quant_acts_kernel(const void* __restrict__ X, int64_t K,
                                                         const float* __restrict__ g, float eps,
                                                         int8_t* __restrict__ Xq,
                                                         float* __restrict__ x_scale,
                                                         int32_t* __restrict__ x_rowsum,
                                                         int* __restrict__ zero, int n_zero) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  __shared__ double red_d[4];
  const int64_t m = blockIdx.x;
  if (m == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
  const RowQuant rq = row_absmax_scale<DT, 256, NORM>(X, m, K, red_f, g, eps, red_d);
  const int sum = row_quantize_to<DT, 256, NORM>(X, m, K, rq.qs, Xq + m * K, red_i, g);
  if (threadIdx.x == 0) {
    const float s = rq.a_c / kQmax;
    x_scale[m] = NORM ? s * rq.r : s;
    if (x_rowsum) x_rowsum[m] = sum;
  }
}

// The same quantization in one pass for rows of at most KCH * 2048
// elements: every thread issues all of its loads at entry and keeps its
// chunks in registers through the max reduction, so a row costs one memory
// round trip instead of one per loop iteration and a second pass.  Same
// arithmetic, in the same order, as the two-pass kernel.
template <int DT, bool NORM, int KCH>
__global__ __launch_bounds__(256) void quant_acts_row_kernel(
    const void* __restrict__ X, int64_t K, const float* __restrict__ g, float eps,
    int8_t* __restrict__ Xq, float* __restrict__ x_scale, int32_t* __restrict__ x_rowsum,
    int* __restrict__ zero, int n_zero) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  __shared__ double red_d[4];
  __shared__ float s_scale;
  __shared__ int s_rowsum;
  const int m = blockIdx.x;
  Chunk<DT> ch[KCH];
  load_row<DT, 256, KCH>(X, m, (int)K, ch);
  Gains<256, KCH> gn;
  if constexpr (NORM) load_gains<256, KCH>(g, (int)K, gn);
  if (m == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
  quantize_row<DT, 256, KCH, NORM>(ch, (int)K, Xq + (int64_t)m * K, red_f, red_i, &s_scale,
                                   &s_rowsum, &gn, NORM, eps, red_d);
  if (threadIdx.x == 0) {  // thread 0 wrote both
    x_scale[m] = s_scale;
    if (x_rowsum) x_rowsum[m] = s_rowsum;
  }
}

template <int DT, bool NORM>
void launch_quant(const void* X, int64_t M, int64_t K, const float* g, float eps, int8_t* Xq,
                  float* x_scale, int32_t* x_rowsum, int* zero, int n_zero, hipStream_t s) {
  const dim3 grid((unsigned)M), block(256);
#define BL_QUANT_ROW(n)                                                                      \
  if (K <= (n) * 2048) {                                                                    \
    hipLaunchKernelGGL((quant_acts_row_kernel<DT, NORM, n>), grid, block, 0, s, X, K, g, eps, \
                       Xq, x_scale, x_rowsum, zero, n_zero);                                \
    return;                                                                                 \
  }
  BL_QUANT_ROW(1)
  BL_QUANT_ROW(2)
  BL_QUANT_ROW(4)
  BL_QUANT_ROW(6)
  BL_QUANT_ROW(8)
#undef BL_QUANT_ROW
  hipLaunchKernelGGL((quant_acts_kernel<DT, NORM>), grid, block, 0, s, X, K, g, eps, Xq,
                     x_scale, x_rowsum, zero, n_zero);
}

}  // namespace

hipError_t bl_launch_quant_acts(const void* X, int dtype, int64_t M, int64_t K, int8_t* Xq,
                                float* x_scale, int32_t* x_rowsum, int* zero, int n_zero,
                                hipStream_t s, const float* norm_gain, float norm_eps) {
  if (!zero) n_zero = 0;
  if (norm_gain)
    dtype == 1 ? launch_quant<1, true>(X, M, K, norm_gain, norm_eps, Xq, x_scale, x_rowsum, zero,
                                       n_zero, s)
               : launch_quant<0, true>(X, M, K, norm_gain, norm_eps, Xq, x_scale, x_rowsum, zero,
                                       n_zero, s);
  else
    dtype == 1 ? launch_quant<1, false>(X, M, K, norm_gain, norm_eps, Xq, x_scale, x_rowsum, zero,
                                        n_zero, s)
               : launch_quant<0, false>(X, M, K, norm_gain, norm_eps, Xq, x_scale, x_rowsum, zero,
                                        n_zero, s);
  return hipGetLastError();
}
