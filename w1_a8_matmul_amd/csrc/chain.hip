// The decode FFN of one to four tokens -- up projection, squared ReLU (plain
// or gated), down projection -- in one persistent launch.
//
// The squared ReLU between the up and down projections is the FFN's
// activation ("BitNet b1.58 2B4T Technical Report" card, Method Adaptation).
// Here both projections run in one launch: workgroup g computes 16-row tile g
// of the up projection, or, past those, a tile of the down projection.  An up tile is the one-launch
// decode GEMV (quantize the tokens, unpack, v_dot4, squared ReLU) and stores
// its slice of h device-coherently (sc1, past the per-XCD L2s), then raises
// its own flag.  A down tile issues its weight loads first, then waits until
// every up tile's flag is raised, reads h back coherently, quantizes it per
// token (as the activation quantizer, R4) and contracts.  Only down tiles
// wait, and only for up tiles, whose workgroups have lower indices: the
// dispatcher starts workgroups in index order, so those are running and
// wait for nothing.  A bounded poll (with an error flag) makes sure that a
// wait ends even so.  No shared atomic sits on the path: taking tiles from
// one queue counter and counting finished up tiles on another serialize on
// those addresses (measured on the decode pair: 29.7 us with both, 21.6 with
// the queue alone, 14.0 with neither); each up tile raises a flag of its own.  A flag holds the
// launch's generation + 1, so flags are never cleared: the last down tile to
// finish advances the generation.
#include "common.hpp"
#include "gemv_tile.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

constexpr int kNT = 256;
constexpr int kW = kNT / kWave;
constexpr int kCoherent = 16;               // cache policy sc1
constexpr uint32_t kPollLimit = 1u << 22;   // polls of the done counter before giving up

// The workspace: an unused word, down tiles finished, error flag (a poll
// that gave up), generation; then one flag per up tile.
struct ChainCounters {
  int unused, finished, error, gen;
};

// One row of h [M][F] (float) read device-coherently, as load_row reads an
// activation row (8 floats per chunk; chunks past F read zero).
template <int KCH>
__device__ __forceinline__ void load_h_row(const float* __restrict__ H, int m, int F,
                                           Chunk<0> ch[KCH]) {
  const auto r = make_rsrc(H + (int64_t)m * F, (uint32_t)F * 4u);
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const uint32_t off = (threadIdx.x + c * kNT) * 32u;
    const v4u a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent);
    const v4u b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, kCoherent);
    ch[c].a = make_uint4(a.x, a.y, a.z, a.w);
    ch[c].b = make_uint4(b.x, b.y, b.z, b.w);
  }
}

// Folds the lanes' partial sums of all waves (lanes l, l + 16, l + 32,
// l + 48 hold tile row l % 16) into the tile row's sum.
template <int M>
__device__ __forceinline__ int fold(const int (*partial)[kW][kWave], int m, int row) {
  int s = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w)
#pragma unroll
    for (int q = 0; q < 4; ++q) s += partial[m][w][q * 16 + row];
  return s;
}

// M tokens; DT the dtype of X; L weight loads per lane (for both
// projections: K and F up to L * 1024 columns).
template <int M, int DT, int L>
__global__ __launch_bounds__(kNT) void chain_kernel(
    const void* __restrict__ X, int K, int n_up, const uint8_t* __restrict__ packed_up,
    const float* __restrict__ gamma_up, int glu, float* __restrict__ H, int F, int n_down,
    const uint8_t* __restrict__ packed_down, const float* __restrict__ gamma_down,
    float* __restrict__ Y, ChainCounters* __restrict__ ctr) {
  constexpr int KCH = (L + 1) / 2;
  extern __shared__ __align__(16) int8_t xs[];  // [M][max(K, F)] int8 codes
  __shared__ float red_f[kW];
  __shared__ int red_i[kW];
  __shared__ float s_scale[M];
  __shared__ int s_rowsum[M];
  __shared__ int partial[M][kW][kWave];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t_up = n_up / kTileRows, t_down = n_down / kTileRows;
  __shared__ int s_gen;
  if (tid == 0) s_gen = __hip_atomic_load(&ctr->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int item = blockIdx.x;
  const int raised = s_gen + 1;  // an up tile's flag once its h is stored
  int* flags = reinterpret_cast<int*>(ctr + 1);  // [up tiles], after the counters
  uint4 wv[L];
  int part[M];

  if (item < t_up) {
    // Up tile: the one-launch decode GEMV with the squared ReLU (or the gated
    // one of a fused gate+up matrix, whose tile holds 8 gate rows, then their
    // 8 up rows).
    const int kblocks = K / kTileCols;
    // token 0's row, then the weights, then the quantization (token rows
    // after the first are loaded as they are quantized)
    Chunk<DT> ch[KCH];
    load_row<DT, kNT, KCH>(X, 0, K, ch);
    load_tile_weights<kW, L>(packed_up, item, kblocks, wave, lane, wv);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m > 0) load_row<DT, kNT, KCH>(X, m, K, ch);
      quantize_row<DT, kNT, KCH>(ch, K, xs + m * K, red_f, red_i, s_scale + m, s_rowsum + m);
    }
    __syncthreads();
    contract_tile<M, kW, L>(wv, xs, K, kblocks, wave, lane, part);
#pragma unroll
    for (int m = 0; m < M; ++m) partial[m][wave][lane] = part[m];
    __syncthreads();
    if (tid < M * kTileRows) {
      const int m = tid / kTileRows, i = tid % kTileRows;
      const float g = *gamma_up;
      const int acc = fold<M>(partial, m, i) - s_rowsum[m];
      if (glu) {
        if (i < 8) {
          const int acc_up = fold<M>(partial, m, i + 8) - s_rowsum[m];
          const float h = glu_relu2(rescale(acc, s_scale[m], g, false),
                                    rescale(acc_up, s_scale[m], g, false));
          __hip_atomic_store(H + (int64_t)m * F + item * 8 + i, h, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __hip_atomic_store(H + (int64_t)m * F + item * kTileRows + i,
                           rescale(acc, s_scale[m], g, true), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's h stores completed
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(&flags[item], raised, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // Down tile (item - t_up of the down projection): weights first.
  const int tile = item - t_up;
  const int fblocks = F / kTileCols;
  load_tile_weights<kW, L>(packed_down, tile, fblocks, wave, lane, wv);
  // Every thread waits for the flags of up tiles tid, tid + 256, ...
  {
    uint32_t polls = 0;
    for (int j = tid; j < t_up; j += kNT) {
      while (__hip_atomic_load(&flags[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
             raised) {
        if (++polls > kPollLimit) {
          __hip_atomic_store(&ctr->error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < M; ++m) {
    Chunk<0> ch[KCH];
    load_h_row<KCH>(H, m, F, ch);
    quantize_row<0, kNT, KCH>(ch, F, xs + m * F, red_f, red_i, s_scale + m, s_rowsum + m);
  }
  __syncthreads();
  contract_tile<M, kW, L>(wv, xs, F, fblocks, wave, lane, part);
#pragma unroll
  for (int m = 0; m < M; ++m) partial[m][wave][lane] = part[m];
  __syncthreads();
  if (tid < M * kTileRows) {
    const int m = tid / kTileRows, i = tid % kTileRows;
    const int acc = fold<M>(partial, m, i) - s_rowsum[m];
    Y[(int64_t)m * n_down + tile * kTileRows + i] = rescale(acc, s_scale[m], *gamma_down, false);
  }
  if (tid == 0 && __hip_atomic_fetch_add(&ctr->finished, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == t_down - 1) {
    // every down tile is past its wait
    __hip_atomic_store(&ctr->finished, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctr->gen, raised, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int M, int DT, int L>
hipError_t launch_one(const void* X, int64_t K, int64_t n_up, const uint8_t* pu,
                      const float* gu, bool glu, float* H, int64_t F, int64_t n_down,
                      const uint8_t* pd, const float* gd, float* Y, void* ws, hipStream_t s) {
  const size_t lds = (size_t)M * (size_t)(K > F ? K : F);
  const unsigned grid = (unsigned)(n_up / kTileRows + n_down / kTileRows);
  hipLaunchKernelGGL((chain_kernel<M, DT, L>), dim3(grid), dim3(kNT), lds, s, X, (int)K,
                     (int)n_up, pu, gu, glu ? 1 : 0, H, (int)F, (int)n_down, pd, gd, Y,
                     static_cast<ChainCounters*>(ws));
  return hipGetLastError();
}

template <int M, int DT>
hipError_t launch_m(int64_t K, int64_t n_up, const uint8_t* pu, const float* gu, bool glu,
                    float* H, int64_t F, int64_t n_down, const uint8_t* pd, const float* gd,
                    float* Y, void* ws, hipStream_t s, const void* X) {
  const int64_t kmax = K > F ? K : F;
  const int64_t loads = (kmax / kTileCols + kW - 1) / kW;
#define BL_CHAIN_CASE(n)                                                                   \
  if (loads <= n)                                                                          \
    return launch_one<M, DT, n>(X, K, n_up, pu, gu, glu, H, F, n_down, pd, gd, Y, ws, s);
  BL_CHAIN_CASE(2)
  BL_CHAIN_CASE(4)
  BL_CHAIN_CASE(8)
  BL_CHAIN_CASE(12)
#undef BL_CHAIN_CASE
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(int64_t M, int64_t K, int64_t n_up, const uint8_t* pu, const float* gu,
                     bool glu, float* H, int64_t F, int64_t n_down, const uint8_t* pd,
                     const float* gd, float* Y, void* ws, hipStream_t s, const void* X) {
  switch (M) {
    case 1: return launch_m<1, DT>(K, n_up, pu, gu, glu, H, F, n_down, pd, gd, Y, ws, s, X);
    case 2: return launch_m<2, DT>(K, n_up, pu, gu, glu, H, F, n_down, pd, gd, Y, ws, s, X);
    case 3: return launch_m<3, DT>(K, n_up, pu, gu, glu, H, F, n_down, pd, gd, Y, ws, s, X);
    case 4: return launch_m<4, DT>(K, n_up, pu, gu, glu, H, F, n_down, pd, gd, Y, ws, s, X);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t bl_chain_workspace_bytes(int64_t n_up) {
  return 16 + 4 * (size_t)(n_up / kTileRows);
}

hipError_t bl_launch_ffn_chain(const void* X, int dtype, int64_t M, int64_t K, int64_t n_up,
                               const uint8_t* packed_up, const float* gamma_up, bool glu,
                               float* H, int64_t n_down, const uint8_t* packed_down,
                               const float* gamma_down, float* Y, void* ws, hipStream_t s) {
  const int64_t F = glu ? n_up / 2 : n_up;
  return dtype == 1 ? launch_dt<1>(M, K, n_up, packed_up, gamma_up, glu, H, F, n_down,
                                   packed_down, gamma_down, Y, ws, s, X)
                    : launch_dt<0>(M, K, n_up, packed_up, gamma_up, glu, H, F, n_down,
                                   packed_down, gamma_down, Y, ws, s, X);
}
