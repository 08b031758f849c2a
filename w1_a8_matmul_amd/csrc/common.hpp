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
// The base-3 layout (five codes per byte): tiles of 16 rows x 320 columns,
// also 1 KiB; K padded up to a multiple of 320 with code 0.
constexpr int kB3TileCols = 320;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Raw buffer resource over [p, p + bytes): loads at offsets at or past
// `bytes` return zero and do not touch memory, so loads need no branches.
// The third descriptor word is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte load at byte offset voff (per lane) + soff (wave-uniform).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same load with the non-temporal policy (cache-policy bit NT, value 2
// on gfx950), for weights that are read exactly once: the caches do not keep
// them.  Streaming a decode step's weights this way raised the grouped
// forward from 5.1 to 5.3 TB/s (2B step, M = 1).  Not for data that other
// workgroups read again (activations).
__device__ __forceinline__ uint4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// DPP lane moves inside each 16-lane row: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.  After the four steps every lane
// of a row holds the row's reduction.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(dpp<0xb1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<0x4e>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<0x141>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<0x140>(__float_as_int(v))));
  return v;
}

__device__ __forceinline__ int row_sum16(int v) {
  v += dpp<0xb1>(v);
  v += dpp<0x4e>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// Whole-wave reductions (all 64 lanes active); the result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int wave_sum(int v) {
  v = row_sum16(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Sum over the wave in double (the subln sum of squares): the same DPP row
// steps on both halves of the double, then the four rows (cross-lane
// bpermutes cost several times more).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)dpp<CTRL>((int)(unsigned)u);
  const unsigned hi = (unsigned)dpp<CTRL>((int)(unsigned)(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xb1>(v);
  v += dpp_f64<0x4e>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// subln's RMS factor of a row whose squares sum to S (double): one rounding
// of 1 / sqrt(S / K + eps) to float, the rest in double.
__device__ __forceinline__ float rms_factor(double S, int64_t K, float eps) {
  return (float)(1.0 / sqrt(S / (double)K + (double)eps));
}

// rint(v) clamped to [-127, 127] as an int; v is x * qs.
__device__ __forceinline__ int quant_i8(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -kQmax), kQmax);
  return (int)r;
}

// Epilogue modes: none, ReLU^2, and the gated ReLU^2 of a fused gate+up
// matrix packed with its halves interleaved (16-row tile t: gate rows
// 8t..8t+7, then their up rows), whose output has N/2 columns.
constexpr int kEpiNone = 0, kEpiRelu2 = 1, kEpiGlu = 2;

// h = max(gate, 0)^2 * up, left to right (no fused multiply-add).
__device__ __forceinline__ float glu_relu2(float yg, float yu) {
  const float r = yg > 0.0f ? yg : 0.0f;
  const float t = r * r;
  return t * yu;
}

// Row of the unpermuted gate+up matrix held at interleaved packed row n.
__device__ __forceinline__ int64_t glu_source_row(int64_t n, int64_t N) {
  const int64_t t = n / 16, i = n % 16;
  return i < 8 ? 8 * t + i : N / 2 + 8 * t + (i - 8);
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
