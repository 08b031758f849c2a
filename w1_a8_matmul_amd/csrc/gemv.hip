// Small-M BitLinear forward (decode): one kernel per linear.
//
// The activation rows are quantized per token inside the kernel (absmax,
// int8) into LDS; the packed ternary weights stream from HBM in 16-byte
// lane loads (one 1 KiB tile per wave load), are unpacked in registers and
// contracted with v_dot4 (four int8 products per lane per instruction).  No
// MFMA: at M <= 4 the contraction is bound by HBM bytes, not by math.
//
// "Load the packed weights, unpack right before the product, multiply with
// int8 activations" is the kernel outline of the "BitNet b1.58 2B4T Technical
// Report" card, section "Method Adaptation"; the tiling here is gfx950's own.
#include "common.hpp"
#include "quant_row.hpp"

namespace {

using namespace bl;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// Codes are q+1 in {0,1,2}: sum_k code*x - sum_k x = sum_k q*x exactly.
template <int M, int DT, bool RELU2, bool DEBUG>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const void* __restrict__ X, int64_t K, int64_t N, const uint8_t* __restrict__ packed,
    const float* __restrict__ gamma_p, float* __restrict__ Y, int8_t* __restrict__ xq_out,
    float* __restrict__ xscale_out, int32_t* __restrict__ acc_out) {
  extern __shared__ __align__(16) int8_t xs[];  // [M][K] int8 activations
  __shared__ float red_f[kWaves];
  __shared__ int red_i[kWaves];
  __shared__ float s_scale[M];
  __shared__ int s_rowsum[M];
  __shared__ int partial[kWaves][M][kTileRows];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tile_row = blockIdx.x;
  const int64_t kblocks = K / kTileCols;
  const uint4* wp = reinterpret_cast<const uint4*>(packed + tile_row * kblocks * kTileBytes) + lane;

  // Issue the first weight loads before the activation prologue: the
  // weights do not depend on it.
  uint4 pre = make_uint4(0, 0, 0, 0);
  if (wave < kblocks) pre = wp[(int64_t)wave * 64];

  // Prologue: per-token absmax quantization into LDS.
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const RowQuant rq = row_absmax_scale<DT, kThreads>(X, m, K, red_f);
    const int sum = row_quantize_to<DT, kThreads>(X, m, K, rq.qs, xs + m * K, red_i);
    if (tid == 0) {
      s_scale[m] = rq.a_c / kQmax;
      s_rowsum[m] = sum;
    }
  }
  __syncthreads();

  int acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0;

  const int sub = lane >> 4;  // which 64-column quarter of the 256-column block
  for (int64_t b = wave; b < kblocks; b += kWaves) {
    const uint4 wv = (b == wave) ? pre : wp[b * 64];
    const uint32_t words[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int4* xp = reinterpret_cast<const int4*>(xs + m * K + b * kTileCols + sub * 64);
      const int4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
      const int xd[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                          x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
      int a = acc[m];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int f = 0; f < 4; ++f)
          a = __builtin_amdgcn_sdot4((int)codes(words[g], f), xd[4 * g + f], a, false);
      }
      acc[m] = a;
    }
  }

  // Lanes l, l^16, l^32, l^48 hold the same row; fold them, then the waves.
#pragma unroll
  for (int m = 0; m < M; ++m) {
    int a = acc[m];
    a += __shfl_xor(a, 16, kWave);
    a += __shfl_xor(a, 32, kWave);
    if (lane < kTileRows) partial[wave][m][lane] = a;
  }
  __syncthreads();

  if (tid < M * kTileRows) {
    const int m = tid / kTileRows, i = tid % kTileRows;
    int s = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += partial[w][m][i];
    const int acc_true = s - s_rowsum[m];
    const int64_t n = tile_row * kTileRows + i;
    Y[m * N + n] = rescale(acc_true, s_scale[m], *gamma_p, RELU2);
    if constexpr (DEBUG) {
      if (acc_out) acc_out[m * N + n] = acc_true;
    }
  }
  if constexpr (DEBUG) {
    if (blockIdx.x == 0) {
      for (int64_t i = tid; i < (int64_t)M * K; i += kThreads)
        if (xq_out) xq_out[i] = xs[i];
      if (tid < M && xscale_out) xscale_out[tid] = s_scale[tid];
    }
  }
}

constexpr int kMaxM = 4;
constexpr int64_t kMaxLds = 48 * 1024;

template <int M, int DT, bool RELU2, bool DEBUG>
hipError_t launch_one(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                      const float* gamma, float* Y, int8_t* xq, float* xs, int32_t* acc,
                      hipStream_t s) {
  const size_t lds = (size_t)M * (size_t)K;
  hipLaunchKernelGGL((gemv_kernel<M, DT, RELU2, DEBUG>), dim3((unsigned)(N / kTileRows)),
                     dim3(kThreads), lds, s, X, K, N, packed, gamma, Y, xq, xs, acc);
  return hipGetLastError();
}

template <int M, int DT>
hipError_t launch_m(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                    const float* gamma, float* Y, bool relu2, int8_t* xq, float* xs,
                    int32_t* acc, hipStream_t s) {
  const bool dbg = xq || xs || acc;
  if (relu2)
    return dbg ? launch_one<M, DT, true, true>(X, K, N, packed, gamma, Y, xq, xs, acc, s)
               : launch_one<M, DT, true, false>(X, K, N, packed, gamma, Y, xq, xs, acc, s);
  return dbg ? launch_one<M, DT, false, true>(X, K, N, packed, gamma, Y, xq, xs, acc, s)
             : launch_one<M, DT, false, false>(X, K, N, packed, gamma, Y, xq, xs, acc, s);
}

template <int DT>
hipError_t launch_dt(const void* X, int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                     const float* gamma, float* Y, bool relu2, int8_t* xq, float* xs,
                     int32_t* acc, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, DT>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
    case 2: return launch_m<2, DT>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
    case 3: return launch_m<3, DT>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
    case 4: return launch_m<4, DT>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool bl_gemv_supports(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxM && M * K <= kMaxLds;
}

hipError_t bl_launch_gemv(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                          const uint8_t* packed, const float* gamma, float* Y, bool relu2,
                          int8_t* xq_out, float* xscale_out, int32_t* acc_out, hipStream_t s) {
  if (dtype == 1)
    return launch_dt<1>(X, M, K, N, packed, gamma, Y, relu2, xq_out, xscale_out, acc_out, s);
  return launch_dt<0>(X, M, K, N, packed, gamma, Y, relu2, xq_out, xscale_out, acc_out, s);
}
