// Shared device helpers and launch declarations for the BitLinear kernels.
// gfx950 (CDNA4) only: 64-wide wavefronts, int8 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;
constexpr float kEps = 1e-5f;       // guard for all-zero weights / tokens
constexpr float kQmax = 127.0f;     // symmetric int8 range [-127, 127]
constexpr uint32_t kCodeMask = 0x03030303u;

// Packed tile geometry (16 rows x 256 columns, 1 KiB).
constexpr int kTileRows = 16;
constexpr int kTileCols = 256;
constexpr int kTileBytes = 1024;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// rint(v) clamped to [-127, 127] as an int; v is x * qs.
__device__ __forceinline__ int quant_i8(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -kQmax), kQmax);
  return (int)r;
}

// Epilogue: ((float)acc * s_x) * gamma, then the optional ReLU^2.  Written as
// separate statements; the library is compiled with -ffp-contract=off.
__device__ __forceinline__ float rescale(int acc, float sx, float gamma, bool relu2) {
  float t = (float)acc * sx;
  float y = t * gamma;
  if (relu2) {
    float r = y > 0.0f ? y : 0.0f;
    y = r * r;
  }
  return y;
}

// Codes of field f (0..3) of a packed word: four bytes, each 0, 1 or 2.
__device__ __forceinline__ uint32_t codes(uint32_t w, int f) {
  return (w >> (2 * f)) & kCodeMask;
}

}  // namespace bl

// Host-side launchers (defined in the .hip files).  All return hipError_t of
// the launch; shapes were validated by the ABI layer.
hipError_t bl_launch_absmean_rows(const float* W, int64_t N, int64_t K, double* row_sum,
                                  hipStream_t s);
hipError_t bl_launch_absmean_final(const double* row_sum, int64_t N, int64_t K,
                                   float* gamma, hipStream_t s);
hipError_t bl_launch_quant_pack(const float* W, int64_t N, int64_t K, const float* gamma,
                                uint8_t* packed, hipStream_t s);
hipError_t bl_launch_pack(const int8_t* Wq, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t s);
hipError_t bl_launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wq,
                            hipStream_t s);
hipError_t bl_launch_quant_acts(const void* X, int dtype, int64_t M, int64_t K, int8_t* Xq,
                                float* x_scale, int32_t* x_rowsum, hipStream_t s);
// Small-M fused forward (activation quantization inside the kernel).
bool bl_gemv_supports(int64_t M, int64_t K);
hipError_t bl_launch_gemv(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                          const uint8_t* packed, const float* gamma, float* Y, bool relu2,
                          int8_t* xq_out, float* xscale_out, int32_t* acc_out,
                          hipStream_t s);
// Forward from quantized activations on the int8 MFMA units.
hipError_t bl_launch_gemm_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, bool relu2, int32_t* acc_out,
                            hipStream_t s);
