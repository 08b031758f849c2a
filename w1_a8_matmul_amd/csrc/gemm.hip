// BitLinear forward from int8 activations on the CDNA4 int8 matrix cores
// (v_mfma_i32_16x16x64_i8): for larger M the ternary x int8 product is a
// dense contraction, so the packed tiles are unpacked in registers into
// MFMA B operands and multiplied against int8 activation tiles.
#include "common.hpp"

namespace {

using namespace bl;

constexpr int kThreads = 256;

// Wave tile: TM x TN blocks of 16x16 outputs; 2x2 waves per workgroup.
template <int TM, int TN, bool RELU2, bool DEBUG>
__global__ __launch_bounds__(kThreads) void gemm_q_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_rowsum, int64_t M, int64_t K, int64_t N,
    const uint8_t* __restrict__ packed, const float* __restrict__ gamma_p,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m_base = ((int64_t)blockIdx.y * 2 + wm) * (16 * TM);
  const int64_t ntile_base = ((int64_t)blockIdx.x * 2 + wn) * TN;  // in 16-row tiles
  const int64_t ntiles = N / kTileRows;
  const int64_t kblocks = K / kTileCols;
  const int r16 = lane & 15, grp = lane >> 4;

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  for (int64_t b = 0; b < kblocks; ++b) {
    uint4 bw[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nt = ntile_base + j;
      bw[j] = nt < ntiles ? reinterpret_cast<const uint4*>(
                                packed + (nt * kblocks + b) * kTileBytes)[lane]
                          : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    }
    v4i a[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m_base + i * 16 + r16;
      if (m < M) {
        const v4i* p = reinterpret_cast<const v4i*>(Xq + m * K + b * kTileCols + grp * 64);
#pragma unroll
        for (int g = 0; g < 4; ++g) a[i][g] = p[g];
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) a[i][g] = v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v4i bop[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t w = g == 0 ? bw[j].x : g == 1 ? bw[j].y : g == 2 ? bw[j].z : bw[j].w;
        bop[j] = v4i{(int)codes(w, 0), (int)codes(w, 1), (int)codes(w, 2), (int)codes(w, 3)};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][g], bop[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of a 16x16 int32 MFMA tile: lane holds column (lane % 16) and
  // rows 4*(lane / 16) + r, r = 0..3.
  const float gamma = *gamma_p;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m_base + i * 16 + grp * 4 + r;
      if (m >= M) continue;
      const float sx = x_scale[m];
      const int rs = x_rowsum[m];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t nt = ntile_base + j;
        if (nt >= ntiles) continue;
        const int64_t n = nt * kTileRows + r16;
        const int v = acc[i][j][r] - rs;
        Y[m * N + n] = rescale(v, sx, gamma, RELU2);
        if constexpr (DEBUG) acc_out[m * N + n] = v;
      }
    }
  }
}

constexpr int kTM = 4, kTN = 4;

template <bool RELU2, bool DEBUG>
hipError_t launch(const int8_t* Xq, const float* sx, const int32_t* rs, int64_t M, int64_t K,
                  int64_t N, const uint8_t* packed, const float* gamma, float* Y,
                  int32_t* acc_out, hipStream_t s) {
  const int64_t rows_per_wg = 2 * 16 * kTM;
  const int64_t ntiles_per_wg = 2 * kTN;
  const dim3 grid((unsigned)((N / kTileRows + ntiles_per_wg - 1) / ntiles_per_wg),
                  (unsigned)((M + rows_per_wg - 1) / rows_per_wg));
  hipLaunchKernelGGL((gemm_q_kernel<kTM, kTN, RELU2, DEBUG>), grid, dim3(kThreads), 0, s, Xq,
                     sx, rs, M, K, N, packed, gamma, Y, acc_out);
  return hipGetLastError();
}

}  // namespace

hipError_t bl_launch_gemm_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, bool relu2, int32_t* acc_out,
                            hipStream_t s) {
  if (relu2)
    return acc_out ? launch<true, true>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y,
                                        acc_out, s)
                   : launch<true, false>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y,
                                         acc_out, s);
  return acc_out ? launch<false, true>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y,
                                       acc_out, s)
                 : launch<false, false>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y,
                                        acc_out, s);
}
