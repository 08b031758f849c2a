// Per-token absmax int8 quantization of activations (fishai news digest on
// BitNet b1.58 2B4T, activation-quantization item; "BitNet b1.58 2B4T
// Technical Report" card, Method Adaptation), optionally after subln read as
// an RMSNorm with a per-feature gain (fishai digest, list of BitLinear parts:
// normalization).  One workgroup per token.
#include "common.hpp"
#include "quant_row.hpp"

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

}  // namespace

hipError_t bl_launch_quant_acts(const void* X, int dtype, int64_t M, int64_t K, int8_t* Xq,
                                float* x_scale, int32_t* x_rowsum, int* zero, int n_zero,
                                hipStream_t s, const float* norm_gain, float norm_eps) {
  if (!zero) n_zero = 0;
  const dim3 grid((unsigned)M), block(256);
  if (norm_gain) {
    if (dtype == 1)
      hipLaunchKernelGGL((quant_acts_kernel<1, true>), grid, block, 0, s, X, K, norm_gain,
                         norm_eps, Xq, x_scale, x_rowsum, zero, n_zero);
    else
      hipLaunchKernelGGL((quant_acts_kernel<0, true>), grid, block, 0, s, X, K, norm_gain,
                         norm_eps, Xq, x_scale, x_rowsum, zero, n_zero);
  } else if (dtype == 1) {
    hipLaunchKernelGGL((quant_acts_kernel<1, false>), grid, block, 0, s, X, K, norm_gain,
                       norm_eps, Xq, x_scale, x_rowsum, zero, n_zero);
  } else {
    hipLaunchKernelGGL((quant_acts_kernel<0, false>), grid, block, 0, s, X, K, norm_gain,
                       norm_eps, Xq, x_scale, x_rowsum, zero, n_zero);
  }
  return hipGetLastError();
}
