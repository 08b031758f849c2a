// Grouped decode forward: many independent BitLinear layers (same token
// count M <= 4) in two launches instead of one per layer.
//
// Launch 1 quantizes every layer's activation rows per token (absmax, int8)
// into a workspace.  Launch 2 is persistent: each workgroup owns a
// contiguous, byte-balanced range of 16-row output tiles taken from the
// concatenation of all layers, stages the int8 activations of the layer it
// is working on in LDS, and its waves stream their tiles' packed weights
// (double-buffered chunks of 16-byte lane loads, one 1 KiB tile per wave
// load), unpack the 2-bit codes in registers and contract them with v_dot4.
// One launch then keeps HBM busy across layer boundaries, where one launch
// per layer pays its start-up and drain for every few megabytes.
//
// The per-layer arithmetic is that of the single-layer forward: absmean
// ternary weights and per-token absmax int8 activations ("BitNet b1.58 2B4T
// Technical Report" card, section "Method Adaptation"), exact int32 sums,
// ((float)acc * s_x) * gamma.
#include "common.hpp"
#include "group.hpp"
#include "quant_row.hpp"

namespace {

using namespace bl;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(256) void group_quant_kernel(const GroupOp* __restrict__ ops, int M,
                                                          int8_t* __restrict__ xq,
                                                          float* __restrict__ sx,
                                                          int32_t* __restrict__ rs) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  const int op = blockIdx.x / M, m = blockIdx.x % M;
  const GroupOp o = ops[op];
  int8_t* dst = xq + o.xq_off + (int64_t)m * o.K;
  RowQuant q;
  int sum;
  if (o.dtype == 1) {
    q = row_absmax_scale<1, 256>(o.X, m, o.K, red_f);
    sum = row_quantize_to<1, 256>(o.X, m, o.K, q.qs, dst, red_i);
  } else {
    q = row_absmax_scale<0, 256>(o.X, m, o.K, red_f);
    sum = row_quantize_to<0, 256>(o.X, m, o.K, q.qs, dst, red_i);
  }
  if (threadIdx.x == 0) {
    sx[op * M + m] = q.a_c / kQmax;
    rs[op * M + m] = sum;
  }
}

// Unpack and contract one 16-byte lane chunk (64 columns of one row) with
// the matching 64 int8 activations of every token; see the single-layer
// kernel for the scale-1/4/16 accumulator trick.
template <int M>
__device__ __forceinline__ void dot_chunk(const uint4 w, const int8_t* xs, int K, int col,
                                          int (&a0)[M], int (&a1)[M], int (&a2)[M]) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int4* xp = reinterpret_cast<const int4*>(xs + m * K + col);
    const int4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
    const int xd[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                        x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t wd = words[g];
      a0[m] = __builtin_amdgcn_sdot4((int)(wd & 0x03030303u), xd[4 * g + 0], a0[m], false);
      a1[m] = __builtin_amdgcn_sdot4((int)(wd & 0x0c0c0c0cu), xd[4 * g + 1], a1[m], false);
      a2[m] = __builtin_amdgcn_sdot4((int)(wd & 0x30303030u), xd[4 * g + 2], a2[m], false);
      a2[m] = __builtin_amdgcn_sdot4((int)((wd >> 2) & 0x30303030u), xd[4 * g + 3], a2[m], false);
    }
  }
}

// One wave works through tiles first, first+stride, ... < last of layer o.
// Each tile is cut into chunks of C column blocks; the loads of the next
// chunk are in flight while the current one is contracted.  Chunks past the
// end use an empty buffer range and read zeros.
template <int M, int C>
__device__ __forceinline__ void run_tiles(const GroupOp& o, int first, int last, int stride,
                                          const int8_t* xs, const float* s_sx, const int* s_rs,
                                          int lane) {
  const int K = o.K;
  const int kblocks = K / kTileCols;
  const int nc = (kblocks + C - 1) / C;
  const int n_mine = first < last ? (last - first + stride - 1) / stride : 0;
  const int total = n_mine * nc;
  if (total == 0) return;
  const float gamma = *o.gamma;
  const int sub = lane >> 4;

  auto issue = [&](uint4 (&buf)[C], int j) {
    const bool valid = j < total;
    const int it = first + (j / nc) * stride;
    const int c = j % nc;
    const int64_t tr = it - o.item_begin;
    const auto r = make_rsrc(o.packed + (valid ? tr * (int64_t)kblocks * kTileBytes : 0),
                             valid ? (uint32_t)kblocks * kTileBytes : 0u);
#pragma unroll
    for (int i = 0; i < C; ++i) buf[i] = buf_load16(r, lane * 16, (uint32_t)(c * C + i) * kTileBytes);
  };

  int a0[M], a1[M], a2[M];
#pragma unroll
  for (int m = 0; m < M; ++m) a0[m] = a1[m] = a2[m] = 0;

  auto consume = [&](const uint4 (&buf)[C], int j) {
    const int c = j % nc;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int b = min(c * C + i, kblocks - 1);  // past the end: zero codes, any x
      dot_chunk<M>(buf[i], xs, K, b * kTileCols + sub * 64, a0, a1, a2);
    }
    if (c == nc - 1) {
      const int it = first + (j / nc) * stride;
      const int64_t tr = it - o.item_begin;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        int v = a0[m] + (a1[m] >> 2) + (a2[m] >> 4);
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        if (lane < kTileRows && j < total) {
          const int64_t n = tr * kTileRows + lane;
          o.Y[m * (int64_t)o.N + n] = rescale(v - s_rs[m], s_sx[m], gamma, o.relu2 != 0);
        }
        a0[m] = a1[m] = a2[m] = 0;
      }
    }
  };

  uint4 bufA[C], bufB[C];
  issue(bufA, 0);
  for (int j = 0; j < total; j += 2) {
    issue(bufB, j + 1);
    consume(bufA, j);
    issue(bufA, j + 2);
    consume(bufB, j + 1);
  }
}

template <int M, int C>
__device__ void run_tiles_c(const GroupOp& o, int first, int last, const int8_t* xs,
                            const float* s_sx, const int* s_rs, int wave, int lane) {
  run_tiles<M, C>(o, first + wave, last, kWaves, xs, s_sx, s_rs, lane);
}

template <int M>
__global__ __launch_bounds__(kThreads) void group_gemv_kernel(
    const GroupOp* __restrict__ ops, int n_ops, const int* __restrict__ wg_begin,
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int* __restrict__ rs) {
  extern __shared__ __align__(16) int8_t xs[];  // [M][K] of the current layer
  __shared__ float s_sx[M];
  __shared__ int s_rs[M];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int item = wg_begin[blockIdx.x];
  const int end = wg_begin[blockIdx.x + 1];
  int op = 0;
  while (op + 1 < n_ops && ops[op + 1].item_begin <= item) ++op;

  while (item < end) {
    const GroupOp o = ops[op];
    const int seg_end = min(end, o.item_begin + o.N / kTileRows);
    // Stage this layer's int8 activations (M*K bytes, a multiple of 256).
    const int bytes = M * o.K;
    const uint4* src = reinterpret_cast<const uint4*>(xq + o.xq_off);
    for (int i = tid; i < bytes / 16; i += kThreads) reinterpret_cast<uint4*>(xs)[i] = src[i];
    if (tid < M) {
      s_sx[tid] = sx[op * M + tid];
      s_rs[tid] = rs[op * M + tid];
    }
    __syncthreads();
    switch (o.chunk) {
      case 1: run_tiles_c<M, 1>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 2: run_tiles_c<M, 2>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 3: run_tiles_c<M, 3>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 4: run_tiles_c<M, 4>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 5: run_tiles_c<M, 5>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 6: run_tiles_c<M, 6>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 7: run_tiles_c<M, 7>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 8: run_tiles_c<M, 8>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 9: run_tiles_c<M, 9>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 10: run_tiles_c<M, 10>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      case 11: run_tiles_c<M, 11>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
      default: run_tiles_c<M, 12>(o, item, seg_end, xs, s_sx, s_rs, wave, lane); break;
    }
    __syncthreads();  // before the next layer overwrites xs
    item = seg_end;
    ++op;
  }
}

}  // namespace

hipError_t bl_launch_group(const GroupOp* ops, int n_ops, int M, const int* wg_begin, int G,
                           int max_k, int8_t* xq, float* sx, int32_t* rs, hipStream_t s) {
  hipLaunchKernelGGL(group_quant_kernel, dim3((unsigned)(n_ops * M)), dim3(256), 0, s, ops, M,
                     xq, sx, rs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)M * (size_t)max_k;
  switch (M) {
    case 1:
      hipLaunchKernelGGL(group_gemv_kernel<1>, dim3(G), dim3(kThreads), lds, s, ops, n_ops,
                         wg_begin, xq, sx, rs);
      break;
    case 2:
      hipLaunchKernelGGL(group_gemv_kernel<2>, dim3(G), dim3(kThreads), lds, s, ops, n_ops,
                         wg_begin, xq, sx, rs);
      break;
    case 3:
      hipLaunchKernelGGL(group_gemv_kernel<3>, dim3(G), dim3(kThreads), lds, s, ops, n_ops,
                         wg_begin, xq, sx, rs);
      break;
    default:
      hipLaunchKernelGGL(group_gemv_kernel<4>, dim3(G), dim3(kThreads), lds, s, ops, n_ops,
                         wg_begin, xq, sx, rs);
      break;
  }
  return hipGetLastError();
}
