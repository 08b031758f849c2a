// Context probes for the benchmark: what this MI355X sustains for a plain
// streaming read and for int8 matrix-core work, measured the same way as the
// BitLinear kernels.  They are reported beside the BitLinear numbers and are
// not a denominator: the roofline fractions use the published peaks.
// Built into a library of their own; nothing on the BitLinear path uses them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Streaming read: workgroup g reads the 16-byte chunks g*256 + t, advancing
// by the whole grid, ten loads in flight per lane.  Each workgroup writes
// one word so that the loads stay live.  `bytes` is a multiple of 16.  NT:
// the loads carry the non-temporal (streaming) policy, as the decode
// kernels' weight loads do.
template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const v4u* __restrict__ src, uint64_t n16,
                                                   uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 9 * stride < n16; i += 10 * stride) {
    v4u v[10];
#pragma unroll
    for (int u = 0; u < 10; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 10; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const v4u v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // practically never; keeps the loads
}

// Matrix-core loop: eight independent accumulators per wave, operands in
// registers (loaded once from `src`, which holds 1024 v4i).
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_kernel(const v4i* __restrict__ src, int iters,
                                                   int* __restrict__ sink) {
  const int t = threadIdx.x;
  const v4i a0 = src[t], a1 = src[t + 256], b0 = src[t + 512], b1 = src[t + 768];
  if constexpr (SHAPE == 0) {
    v4i c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = v4i{0, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        c[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8((k & 2) ? a1 : a0, (k & 1) ? b1 : b0, c[k],
                                                     0, 0, 0);
    }
    v4i s = c[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) s += c[k];
    if (s.x == 0x7fffffff) sink[blockIdx.x] = s.y;
  } else {
    v16i c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[k][e] = 0;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        c[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8((k & 2) ? a1 : a0, (k & 1) ? b1 : b0, c[k],
                                                     0, 0, 0);
    }
    v16i s = c[0] + c[1] + c[2] + c[3];
    if (s[0] == 0x7fffffff) sink[blockIdx.x] = s[1];
  }
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device buffer `src` with `grid`
// workgroups of 256 threads; `sink` holds `grid` words.  0 or a hipError_t.
int probe_stream_read(const void* src, uint64_t bytes, void* sink, int grid, void* stream) {
  if (!src || !sink || grid < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const v4u*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// The same read with non-temporal loads.
int probe_stream_read_nt(const void* src, uint64_t bytes, void* sink, int grid, void* stream) {
  if (!src || !sink || grid < 1 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const v4u*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `iters` rounds of int8 MFMAs per wave: shape 0 = 8 x v_mfma_i32_16x16x64_i8
// (16x16x64 multiply-adds each), shape 1 = 4 x v_mfma_i32_32x32x32_i8
// (32x32x32 each).  `src` holds 1024 v4i of operand bytes, `sink` `grid` ints.
int probe_mfma_i8(int shape, const void* src, int iters, void* sink, int grid, void* stream) {
  if (!src || !sink || grid < 1 || iters < 1 || (shape != 0 && shape != 1))
    return (int)hipErrorInvalidValue;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_kernel<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const v4i*>(src), iters, static_cast<int*>(sink));
  else
    hipLaunchKernelGGL(mfma_kernel<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const v4i*>(src), iters, static_cast<int*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
