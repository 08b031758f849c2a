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
#include "gemv_tile.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

constexpr int kMaxM = 4;
constexpr int kNT = 256;
constexpr int kMaxLoadsPerLane = 12;

// After this workgroup's h values are stored: count in; the last workgroup
// quantizes every token's row of h [M][F] (R4, as the activation
// quantizer: a = max|h|, codes rint(h * (127 / a_c)), scale a_c / 127, row
// sum of the codes).  It reads h device-coherently (sc1) in 16-byte loads,
// kHq per thread issued together: rows up to kHq * 1024 values stay in
// registers between the max and the codes; longer rows are read twice.
constexpr int kHq = 12;
constexpr int kCoherentLoad = 16;  // cache policy sc1

template <int M>
__device__ __forceinline__ void quantize_h_if_last(const float* __restrict__ H, int64_t F,
                                                   int64_t ntiles, int* __restrict__ counter,
                                                   int8_t* __restrict__ hq,
                                                   float* __restrict__ h_scale,
                                                   int32_t* __restrict__ h_rowsum,
                                                   float* red_f, int* red_i) {
  constexpr int W = kNT / kWave;
  constexpr int kChunk = kHq * kNT * 4;  // floats per chunk of a row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's h stores have completed
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == (int)ntiles - 1 ? 1 : 0;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  for (int m = 0; m < M; ++m) {
    const float* row = H + m * F;
    auto load_chunk = [&](int64_t c0, v4u (&v)[kHq]) {
      const auto r = make_rsrc(row + c0, (uint32_t)(min((int64_t)kChunk, F - c0) * 4));
#pragma unroll
      for (int j = 0; j < kHq; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (tid + j * kNT) * 16, 0, kCoherentLoad);
    };
    v4u v[kHq];
    float amax = 0.0f;
    for (int64_t c0 = 0; c0 < F; c0 += kChunk) {
      load_chunk(c0, v);  // past the row: zeros
#pragma unroll
      for (int j = 0; j < kHq; ++j)
        amax = fmaxf(fmaxf(fmaxf(fmaxf(amax, fabsf(__uint_as_float(v[j].x))),
                                 fabsf(__uint_as_float(v[j].y))),
                           fabsf(__uint_as_float(v[j].z))),
                     fabsf(__uint_as_float(v[j].w)));
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
    for (int64_t c0 = 0; c0 < F; c0 += kChunk) {
      if (F > kChunk) load_chunk(c0, v);  // one chunk: still in registers
#pragma unroll
      for (int j = 0; j < kHq; ++j) {
        const int64_t k = c0 + (int64_t)(tid + j * kNT) * 4;
        if (k < F) {
          const int q0 = quant_i8(__uint_as_float(v[j].x) * qs);
          const int q1 = quant_i8(__uint_as_float(v[j].y) * qs);
          const int q2 = quant_i8(__uint_as_float(v[j].z) * qs);
          const int q3 = quant_i8(__uint_as_float(v[j].w) * qs);
          sum += q0 + q1 + q2 + q3;
          *reinterpret_cast<uint32_t*>(hq + m * F + k) =
              ((uint32_t)q0 & 0xffu) | (((uint32_t)q1 & 0xffu) << 8) |
              (((uint32_t)q2 & 0xffu) << 16) | ((uint32_t)q3 << 24);
        }
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) red_i[wave] = sum;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) t += red_i[w];
      h_scale[m] = a_c / kQmax;
      h_rowsum[m] = t;
    }
    __syncthreads();  // red_f / red_i are reused by the next token
  }
}

// Codes are q+1 in {0,1,2}: sum_k code*x - sum_k x = sum_k q*x exactly.
// 256 threads (4 waves) per TPW 16-row tiles (tiles TPW*g .. TPW*g+TPW-1;
// a tile past the last reads zeros and stores nothing); L = weight loads
// per lane and tile (K <= L*1024) and KCH = (L+1)/2 eight-element
// activation chunks per thread per row (K <= KCH*2048).  The debug outputs
// are written only when their pointers are set.  The library launches one
// tile per workgroup: measured on MI355X, two or four tiles per workgroup
// (fewer workgroups, less repeated quantization) and eight-wave workgroups
// were slower on both decode projections, and this form of the kernel was
// faster than one written for a single tile (3.2 vs 3.5 us for 2560->6912).
//
// PREQ: X holds int8 codes [M][K] already quantized (scales and row sums in
// pq_scale / pq_rowsum); they are copied into LDS instead of quantized.
// QOUT (with the gated epilogue): the outputs h [M][N/2] also leave as the
// int8 input of the next projection.  h is stored device-coherently (sc1,
// past the per-XCD L2s); each workgroup then counts itself in at q_counter,
// and the last to arrive quantizes the whole of h per token exactly as
// bitlinear_quantize_acts does (absmax, R4), into xq_out / xscale_out /
// q_rowsum, and puts the counter back to zero.  No workgroup waits for
// another.
template <int M, int DT, int L, int TPW, bool NORM, bool PREQ = false, bool QOUT = false>
__global__ __launch_bounds__(kNT) void gemv_kernel(
    const void* __restrict__ X, int K, int64_t N, const uint8_t* __restrict__ packed,
    const float* __restrict__ gamma_p, float* __restrict__ Y, int epi,
    int8_t* __restrict__ xq_out, float* __restrict__ xscale_out, int32_t* __restrict__ acc_out,
    const float* __restrict__ norm_gain, float norm_eps,
    const float* __restrict__ pq_scale = nullptr, const int32_t* __restrict__ pq_rowsum = nullptr,
    int32_t* __restrict__ q_rowsum = nullptr, int* __restrict__ q_counter = nullptr) {
  static_assert(!(PREQ && NORM), "pre-quantized rows carry their norm already");
  static_assert(!QOUT || TPW == 1, "one tile per workgroup when h is quantized in the kernel");
  constexpr int W = kNT / kWave;
  constexpr int KCH = (L + 1) / 2;
  constexpr int kRegsPerRow = KCH * (DT == 1 ? 4 : 8);
  constexpr int P = PREQ ? 0
                         : ((M * kRegsPerRow <= kPreloadRegs)
                                ? M
                                : (kRegsPerRow <= kPreloadRegs ? 1 : 0));
  // 16-byte pieces of the int8 rows per thread (PREQ): M K / 16 over kNT.
  constexpr int PC = PREQ ? (M * L * kTileCols * W / 16 + kNT - 1) / kNT : 1;
  extern __shared__ __align__(16) int8_t xs[];  // [M][K] int8 activations
  __shared__ float red_f[W];
  __shared__ int red_i[W];
  __shared__ double red_d[W];
  __shared__ float s_scale[M];
  __shared__ int s_rowsum[M];
  __shared__ int partial[TPW][M][W][kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ntiles = N / kTileRows;
  const int kblocks = K / kTileCols;
  // 1) activation rows 0..P-1 (and the subln gains), then 2) every weight
  // load of this lane.
  Chunk<DT> pre[P > 0 ? P : 1][KCH];
#pragma unroll
  for (int m = 0; m < P; ++m) load_row<DT, kNT, KCH>(X, m, K, pre[m]);
  Gains<kNT, KCH> gn;
  if constexpr (NORM) load_gains<kNT, KCH>(norm_gain, K, gn);
  uint4 xv[PC];
  if constexpr (PREQ) {
    // the int8 rows, 16 bytes per piece (pieces past M K read zero)
    const auto xr = make_rsrc(X, (uint32_t)(M * K));
#pragma unroll
    for (int c = 0; c < PC; ++c) xv[c] = buf_load16(xr, (uint32_t)(tid + c * kNT) * 16u, 0);
  }
  uint4 wv[TPW][L];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t tile = (int64_t)blockIdx.x * TPW + t;
    load_tile_weights<W, L>(packed, tile < ntiles ? tile : 0, tile < ntiles ? kblocks : 0,
                            wave, lane, wv[t]);
  }

  // 3) per-token quantization into LDS while the weights arrive (or the
  // copy of the pre-quantized rows).
  if constexpr (PREQ) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      const int i = tid + c * kNT;
      if (i * 16 < M * K) *reinterpret_cast<uint4*>(xs + i * 16) = xv[c];
    }
    if (tid < M) {
      s_scale[tid] = pq_scale[tid];
      s_rowsum[tid] = pq_rowsum[tid];
    }
  }
#pragma unroll
  for (int m = 0; m < (PREQ ? 0 : M); ++m) {
    if (m < P) {
      quantize_row<DT, kNT, KCH, NORM>(pre[m < P ? m : 0], K, xs + m * K, red_f, red_i,
                                       s_scale + m, s_rowsum + m, &gn, true, norm_eps, red_d);
    } else {
      Chunk<DT> ch[KCH];
      load_row<DT, kNT, KCH>(X, m, K, ch);
      quantize_row<DT, kNT, KCH, NORM>(ch, K, xs + m * K, red_f, red_i, s_scale + m,
                                       s_rowsum + m, &gn, true, norm_eps, red_d);
    }
  }
  __syncthreads();

  // 4) unpack + v_dot4 over this lane's column blocks, 5) fold the lanes'
  // partial sums of all waves through LDS (lanes l, l+16, l+32, l+48 hold
  // tile row l%16) and rescale.
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    int part[M];
    contract_tile<M, W, L>(wv[t], xs, K, kblocks, wave, lane, part);
#pragma unroll
    for (int m = 0; m < M; ++m) partial[t][m][wave][lane] = part[m];
  }
  __syncthreads();
  if (tid < TPW * M * kTileRows) {
    const int t = tid / (M * kTileRows), r = tid % (M * kTileRows);
    const int m = r / kTileRows, i = r % kTileRows;
    const int64_t tile = (int64_t)blockIdx.x * TPW + t;
    int s = 0;
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += partial[t][m][w][q * 16 + i];
    if (tile < ntiles) {
      const int acc_true = s - s_rowsum[m];
      const int64_t n = tile * kTileRows + i;
      if (epi == kEpiGlu) {
        // rows i < 8 of the tile are gates, rows i + 8 their up rows
        if (i < 8) {
          int su = 0;
#pragma unroll
          for (int w = 0; w < W; ++w)
#pragma unroll
            for (int q = 0; q < 4; ++q) su += partial[t][m][w][q * 16 + i + 8];
          const float yg = rescale(acc_true, s_scale[m], *gamma_p, false);
          const float yu = rescale(su - s_rowsum[m], s_scale[m], *gamma_p, false);
          const float h = glu_relu2(yg, yu);
          if constexpr (QOUT)
            __hip_atomic_store(Y + m * (N / 2) + tile * 8 + i, h, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);  // sc1: past this XCD's L2
          else
            Y[m * (N / 2) + tile * 8 + i] = h;
        }
        if (acc_out) acc_out[m * N + glu_source_row(n, N)] = acc_true;
      } else {
        Y[m * N + n] = rescale(acc_true, s_scale[m], *gamma_p, epi == kEpiRelu2);
        if (acc_out) acc_out[m * N + n] = acc_true;
      }
    }
  }
  if constexpr (QOUT) {
    quantize_h_if_last<M>(Y, N / 2, ntiles, q_counter, xq_out, xscale_out, q_rowsum, red_f,
                          red_i);
    return;
  }
  if (blockIdx.x == 0) {
    if (xq_out)
      for (int i = tid; i < M * K; i += kNT) xq_out[i] = xs[i];
    if (xscale_out && tid < M) xscale_out[tid] = s_scale[tid];
  }
}

// Arguments every launch passes through.
struct GemvArgs {
  const void* X;
  int64_t K, N;
  const uint8_t* packed;
  const float* gamma;
  float* Y;
  int epi;
  int8_t* xq;
  float* xs;
  int32_t* acc;
  const float* norm_gain;
  float norm_eps;
  int mode;  // 0 plain, 1 pre-quantized rows (PREQ), 2 h quantized in the kernel (QOUT)
  const float* pq_scale;
  const int32_t* pq_rowsum;
  int32_t* q_rowsum;
  int* q_counter;
};

template <int M, int DT, int L>
hipError_t launch_one(const GemvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)M * (size_t)a.K;
  constexpr int kTilesPerWorkgroup = 1;
  const dim3 grid((unsigned)(a.N / kTileRows / kTilesPerWorkgroup)), block(kNT);
  if (a.mode == 1) {
    if constexpr (DT == 0)  // the rows are int8 whatever the source dtype was
      hipLaunchKernelGGL((gemv_kernel<M, 0, L, kTilesPerWorkgroup, false, true, false>), grid,
                         block, lds, s, a.X, (int)a.K, a.N, a.packed, a.gamma, a.Y, a.epi,
                         nullptr, nullptr, a.acc, nullptr, 0.0f, a.pq_scale, a.pq_rowsum,
                         nullptr, nullptr);
    else
      return hipErrorInvalidValue;
  } else if (a.mode == 2)
    hipLaunchKernelGGL((gemv_kernel<M, DT, L, kTilesPerWorkgroup, false, false, true>), grid,
                       block, lds, s, a.X, (int)a.K, a.N, a.packed, a.gamma, a.Y, kEpiGlu,
                       a.xq, a.xs, nullptr, nullptr, 0.0f, nullptr, nullptr, a.q_rowsum,
                       a.q_counter);
  else if (a.norm_gain)
    hipLaunchKernelGGL((gemv_kernel<M, DT, L, kTilesPerWorkgroup, true>), grid, block, lds, s,
                       a.X, (int)a.K, a.N, a.packed, a.gamma, a.Y, a.epi, a.xq, a.xs,
                       a.acc, a.norm_gain, a.norm_eps);
  else
    hipLaunchKernelGGL((gemv_kernel<M, DT, L, kTilesPerWorkgroup, false>), grid, block, lds, s,
                       a.X, (int)a.K, a.N, a.packed, a.gamma, a.Y, a.epi, a.xq, a.xs,
                       a.acc, a.norm_gain, a.norm_eps);
  return hipGetLastError();
}

// L = ceil(kblocks / 4), rounded up to an instantiated count.
template <int M, int DT>
hipError_t launch_m(const GemvArgs& a, hipStream_t s) {
  const int64_t loads = (a.K / kTileCols + 3) / 4;
#define BL_GEMV_CASE(n) \
  if (loads <= n) return launch_one<M, DT, n>(a, s);
  BL_GEMV_CASE(1)
  BL_GEMV_CASE(2)
  BL_GEMV_CASE(3)
  BL_GEMV_CASE(4)
  BL_GEMV_CASE(5)
  BL_GEMV_CASE(6)
  BL_GEMV_CASE(7)
  BL_GEMV_CASE(8)
  BL_GEMV_CASE(10)
  BL_GEMV_CASE(12)
#undef BL_GEMV_CASE
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(int64_t M, const GemvArgs& a, hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1, DT>(a, s);
    case 2: return launch_m<2, DT>(a, s);
    case 3: return launch_m<3, DT>(a, s);
    case 4: return launch_m<4, DT>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Largest K: 12 loads per lane with 4 waves (each load is one 256-column block).
bool bl_gemv_supports(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxM && K <= (int64_t)kMaxLoadsPerLane * 4 * kTileCols;
}

hipError_t bl_launch_gemv(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                          const uint8_t* packed, const float* gamma, float* Y, int epi,
                          int8_t* xq_out, float* xscale_out, int32_t* acc_out, hipStream_t s,
                          const float* norm_gain, float norm_eps) {
  const GemvArgs a{X,        K,       N,         packed,  gamma,   Y,       epi,
                   xq_out,   xscale_out, acc_out, norm_gain, norm_eps, 0,     nullptr,
                   nullptr,  nullptr, nullptr};
  return dtype == 1 ? launch_dt<1>(M, a, s) : launch_dt<0>(M, a, s);
}

hipError_t bl_launch_gemv_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, int epi, int32_t* acc_out,
                            hipStream_t s) {
  const GemvArgs a{Xq,      K,       N,        packed,  gamma,   Y,       epi,
                   nullptr, nullptr, acc_out,  nullptr, 0.0f,    1,       x_scale,
                   x_rowsum, nullptr, nullptr};
  return launch_dt<0>(M, a, s);
}

hipError_t bl_launch_gemv_glu_quant(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                                    const uint8_t* packed, const float* gamma, float* H,
                                    int8_t* hq, float* h_scale, int32_t* h_rowsum,
                                    int* counter, hipStream_t s) {
  const GemvArgs a{X,       K,        N,       packed,  gamma,   H,       kEpiGlu,
                   hq,      h_scale,  nullptr, nullptr, 0.0f,    2,       nullptr,
                   nullptr, h_rowsum, counter};
  return dtype == 1 ? launch_dt<1>(M, a, s) : launch_dt<0>(M, a, s);
}
