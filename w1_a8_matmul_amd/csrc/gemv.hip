// Small-M BitLinear forward (decode): one kernel per linear, no MFMA.
//
// One workgroup owns a 16-row tile of the output.  At entry each thread
// issues its activation loads, then every lane issues all of its packed
// weight loads (16 bytes each; the 64 lanes of a wave read one whole 1 KiB
// tile per load): the weights do not depend on the activations, and loading
// the activations first lets their quantization (per-token absmax to int8,
// into LDS) run while the weights are still in flight.  Each lane then
// unpacks its 2-bit codes in registers and contracts them with v_dot4 (four
// int8 products per instruction); partial sums are folded through LDS and
// rescaled.
//
// "Load the packed weights, unpack right before the product, multiply with
// int8 activations" is the kernel outline of the "BitNet b1.58 2B4T
// Technical Report" card, section "Method Adaptation"; the tiling and the
// unpacking below are this library's own, for gfx950.
#include "common.hpp"
#include "quant_row.hpp"

namespace {

using namespace bl;

constexpr int kMaxM = 4;
constexpr int kMaxLoads = 12;  // weight loads per lane
constexpr int kPreloadRegs = 64;  // VGPRs allowed for activations loaded early

// Codes of a packed word, kept at their bit positions where that still fits
// a signed byte: field 0 as is, field 1 times 4, fields 2 and 3 times 16.
// Three accumulators at scales 1, 4 and 16 then give the exact sum
// acc0 + acc1/4 + acc2/16 (each accumulator is an exact multiple of its
// scale).  Five bit operations unpack 16 codes.
__device__ __forceinline__ void dot_word(uint32_t w, const int* x4, int& a0, int& a1, int& a2) {
  a0 = __builtin_amdgcn_sdot4((int)(w & 0x03030303u), x4[0], a0, false);
  a1 = __builtin_amdgcn_sdot4((int)(w & 0x0c0c0c0cu), x4[1], a1, false);
  a2 = __builtin_amdgcn_sdot4((int)(w & 0x30303030u), x4[2], a2, false);
  a2 = __builtin_amdgcn_sdot4((int)((w >> 2) & 0x30303030u), x4[3], a2, false);
}

// Raw activation chunk: 8 consecutive elements (bf16: one uint4; f32: two).
template <int DT>
struct Chunk {
  uint4 a, b;
};

// Loads of one activation row go through a buffer resource over that row,
// so chunks past its end read as zero without a branch (branches around
// loads make the compiler wait for them early) and without memory traffic.
template <int DT, int NT, int KCH>
__device__ __forceinline__ void load_row(const void* __restrict__ X, int m, int K,
                                         Chunk<DT> ch[KCH]) {
  constexpr uint32_t elt = DT == 1 ? 2 : 4;
  const auto r = make_rsrc(reinterpret_cast<const char*>(X) + (int64_t)m * K * elt, K * elt);
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const uint32_t off = (threadIdx.x + c * NT) * 8 * elt;
    ch[c].a = buf_load16(r, off, 0);
    ch[c].b = DT == 1 ? make_uint4(0, 0, 0, 0) : buf_load16(r, off + 16, 0);
  }
}

template <int DT>
__device__ __forceinline__ void widen(const Chunk<DT>& c, float v[8]) {
  if constexpr (DT == 1) {
    const uint32_t d[4] = {c.a.x, c.a.y, c.a.z, c.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_float(d[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_float(d[i] >> 16);
    }
  } else {
    v[0] = __uint_as_float(c.a.x); v[1] = __uint_as_float(c.a.y);
    v[2] = __uint_as_float(c.a.z); v[3] = __uint_as_float(c.a.w);
    v[4] = __uint_as_float(c.b.x); v[5] = __uint_as_float(c.b.y);
    v[6] = __uint_as_float(c.b.z); v[7] = __uint_as_float(c.b.w);
  }
}

// Quantizes one row held in registers into xs[0..K); the scale and row sum
// go to s_scale / s_rowsum.  All NT threads take part.
template <int DT, int NT, int KCH>
__device__ __forceinline__ void quantize_row(const Chunk<DT> ch[KCH], int K, int8_t* xs,
                                             float* red_f, int* red_i, float* s_scale,
                                             int* s_rowsum) {
  constexpr int W = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Every chunk is used unconditionally (chunks past the row are zeros and
  // cannot raise the max), so the compiler keeps their loads where they
  // were issued instead of sinking them past the weight loads.
  float v[KCH][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    widen<DT>(ch[c], v[c]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
  }
  amax = wave_max(amax);
  if (lane == 0) red_f[wave] = amax;
  __syncthreads();
  float a = red_f[0];
#pragma unroll
  for (int w = 1; w < W; ++w) a = fmaxf(a, red_f[w]);
  const float a_c = a > kEps ? a : kEps;
  const float qs = kQmax / a_c;
  int sum = 0;
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const int k = (tid + c * NT) * 8;
    if (k < K) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = quant_i8(v[c][i] * qs);
        sum += q;
        if (i < 4)
          lo |= ((uint32_t)q & 0xffu) << (8 * i);
        else
          hi |= ((uint32_t)q & 0xffu) << (8 * (i - 4));
      }
      *reinterpret_cast<uint2*>(xs + k) = make_uint2(lo, hi);
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) red_i[wave] = sum;
  __syncthreads();  // also keeps the next row's red_f write after the reads above
  if (tid == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) t += red_i[w];
    *s_scale = a_c / kQmax;
    *s_rowsum = t;
  }
}

// Codes are q+1 in {0,1,2}: sum_k code*x - sum_k x = sum_k q*x exactly.
// NT threads (NT/64 waves) per 16-row tile; KCH = 8-element activation
// chunks per thread per row.
template <int M, int DT, int NT, int KCH, bool DEBUG>
__global__ __launch_bounds__(NT) void gemv_kernel(
    const void* __restrict__ X, int K, int64_t N, const uint8_t* __restrict__ packed,
    const float* __restrict__ gamma_p, float* __restrict__ Y, int relu2,
    int8_t* __restrict__ xq_out, float* __restrict__ xscale_out, int32_t* __restrict__ acc_out) {
  constexpr int W = NT / kWave;
  constexpr int kRegsPerRow = KCH * (DT == 1 ? 4 : 8);
  constexpr int P = (M * kRegsPerRow <= kPreloadRegs) ? M : (kRegsPerRow <= kPreloadRegs ? 1 : 0);
  extern __shared__ __align__(16) int8_t xs[];  // [M][K] int8 activations
  __shared__ float red_f[W];
  __shared__ int red_i[W];
  __shared__ float s_scale[M];
  __shared__ int s_rowsum[M];
  __shared__ int partial[M][W][kWave];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile_row = blockIdx.x;
  const int kblocks = K / kTileCols;

  // 1) activation rows 0..P-1, then 2) every weight load of this lane.
  Chunk<DT> pre[P > 0 ? P : 1][KCH];
#pragma unroll
  for (int m = 0; m < P; ++m) load_row<DT, NT, KCH>(X, m, K, pre[m]);

  // Blocks past the row tile's end read as zero (buffer range check).
  const auto wr = make_rsrc(packed + tile_row * (int64_t)kblocks * kTileBytes,
                            (uint32_t)kblocks * kTileBytes);
  uint4 wv[kMaxLoads];
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i)
    wv[i] = buf_load16(wr, lane * 16, (uint32_t)(wave + W * i) * kTileBytes);

  // 3) per-token quantization into LDS while the weights arrive.
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m < P) {
      quantize_row<DT, NT, KCH>(pre[m < P ? m : 0], K, xs + m * K, red_f, red_i, s_scale + m,
                                s_rowsum + m);
    } else {
      Chunk<DT> ch[KCH];
      load_row<DT, NT, KCH>(X, m, K, ch);
      quantize_row<DT, NT, KCH>(ch, K, xs + m * K, red_f, red_i, s_scale + m, s_rowsum + m);
    }
  }
  __syncthreads();

  // 4) unpack + v_dot4 over this lane's column blocks.
  int a0[M], a1[M], a2[M];
#pragma unroll
  for (int m = 0; m < M; ++m) a0[m] = a1[m] = a2[m] = 0;
  const int sub = lane >> 4;  // 64-column quarter of the 256-column block
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i) {
    const int b = wave + W * i;
    if (b < kblocks) {
      const uint32_t words[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int4* xp = reinterpret_cast<const int4*>(xs + m * K + b * kTileCols + sub * 64);
        const int4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
        const int xd[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                            x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) dot_word(words[g], xd + 4 * g, a0[m], a1[m], a2[m]);
      }
    }
  }

  // 5) lane l holds row (l mod 16) of the tile; fold lanes and waves in LDS.
#pragma unroll
  for (int m = 0; m < M; ++m) partial[m][wave][lane] = a0[m] + (a1[m] >> 2) + (a2[m] >> 4);
  __syncthreads();

  if (tid < M * kTileRows) {
    const int m = tid / kTileRows, i = tid % kTileRows;
    int s = 0;
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += partial[m][w][q * 16 + i];
    const int acc_true = s - s_rowsum[m];
    const int64_t n = tile_row * kTileRows + i;
    Y[m * N + n] = rescale(acc_true, s_scale[m], *gamma_p, relu2 != 0);
    if constexpr (DEBUG) {
      if (acc_out) acc_out[m * N + n] = acc_true;
    }
  }
  if constexpr (DEBUG) {
    if (blockIdx.x == 0) {
      for (int i = tid; i < M * K; i += NT)
        if (xq_out) xq_out[i] = xs[i];
      if (tid < M && xscale_out) xscale_out[tid] = s_scale[tid];
    }
  }
}

template <int M, int DT, int NT, int KCH>
hipError_t launch_one(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                      const float* gamma, float* Y, bool relu2, int8_t* xq, float* xs,
                      int32_t* acc, hipStream_t s) {
  const size_t lds = (size_t)M * (size_t)K;
  const dim3 grid((unsigned)(N / kTileRows)), block(NT);
  if (xq || xs || acc)
    hipLaunchKernelGGL((gemv_kernel<M, DT, NT, KCH, true>), grid, block, lds, s, X, (int)K, N,
                       packed, gamma, Y, relu2 ? 1 : 0, xq, xs, acc);
  else
    hipLaunchKernelGGL((gemv_kernel<M, DT, NT, KCH, false>), grid, block, lds, s, X, (int)K,
                       N, packed, gamma, Y, relu2 ? 1 : 0, xq, xs, acc);
  return hipGetLastError();
}

// Launch shape: 8 waves per tile when there are fewer tiles than CUs (more
// loads in flight per CU), else 4.  K <= 4096 fits a shorter chunk loop.
template <int M, int DT>
hipError_t launch_m(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                    const float* gamma, float* Y, bool relu2, int8_t* xq, float* xs,
                    int32_t* acc, hipStream_t s) {
  const bool wide = (N / kTileRows) < 256;
  if (wide) {
    if (K <= 4096)
      return launch_one<M, DT, 512, 1>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
    return launch_one<M, DT, 512, 3>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
  }
  if (K <= 4096)
    return launch_one<M, DT, 256, 2>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
  return launch_one<M, DT, 256, 6>(X, K, N, packed, gamma, Y, relu2, xq, xs, acc, s);
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

// Largest K: 12 loads per lane with 4 waves (each load is one 256-column block).
bool bl_gemv_supports(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxM && K <= (int64_t)kMaxLoads * 4 * kTileCols;
}

hipError_t bl_launch_gemv(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                          const uint8_t* packed, const float* gamma, float* Y, bool relu2,
                          int8_t* xq_out, float* xscale_out, int32_t* acc_out, hipStream_t s) {
  if (dtype == 1)
    return launch_dt<1>(X, M, K, N, packed, gamma, Y, relu2, xq_out, xscale_out, acc_out, s);
  return launch_dt<0>(X, M, K, N, packed, gamma, Y, relu2, xq_out, xscale_out, acc_out, s);
}
