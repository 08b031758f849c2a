// Building blocks of the small-M (decode) forward of one 16-row output tile,
// (used by the one-linear decode kernel).
//
// A workgroup of NT threads (W = NT/64 waves) owns a tile.  Wave w streams
// the tile's column blocks w, w+W, ... (each 16-byte lane load of a wave is
// one whole 1 KiB packed block), unpacks the 2-bit codes in registers and
// contracts them with the int8 activations in LDS using v_dot4; partial sums
// are folded across lanes and waves through LDS.
#pragma once

#include "common.hpp"

namespace bl {

constexpr int kPreloadRegs = 64;   // VGPRs allowed for activations loaded early

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
// With valid false the range is empty and the whole row reads as zero.
template <int DT, int NT, int KCH>
__device__ __forceinline__ void load_row(const void* __restrict__ X, int m, int K,
                                         Chunk<DT> ch[KCH], bool valid = true) {
  constexpr uint32_t elt = DT == 1 ? 2 : 4;
  const auto r = make_rsrc(reinterpret_cast<const char*>(X) + (int64_t)m * K * elt,
                           valid ? K * elt : 0u);
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

// subln gains (float [K]) of the columns this thread's activation chunks
// cover, loaded with the activation row so that waiting for them never
// waits for the weight loads issued after it.  Gains past K read as zero.
template <int NT, int KCH>
struct Gains {
  uint4 lo[KCH], hi[KCH];
};

template <int NT, int KCH>
__device__ __forceinline__ void load_gains(const float* __restrict__ g, int K,
                                           Gains<NT, KCH>& gn) {
  const auto r = make_rsrc(g, g ? (uint32_t)K * 4u : 0u);
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    const uint32_t off = (threadIdx.x + c * NT) * 32u;
    gn.lo[c] = buf_load16(r, off, 0);
    gn.hi[c] = buf_load16(r, off + 16, 0);
  }
}

// Position of natural dword d of an int8 row in the field-transposed LDS
// layout: within each 64-byte group, dword 4j + f moves to 4f + j.
__device__ __forceinline__ int xs_ft_dword(int d) {
  return (d & ~15) | ((d & 3) << 2) | ((d >> 2) & 3);
}

// Quantizes one row held in registers into xs[0..K); the scale and row sum
// go to s_scale / s_rowsum.  All NT threads take part.  With NORM and
// gain_on, subln first: the codes are those of u = x * g and the scale
// carries the row's RMS factor (from the double sum of x^2; red_d holds
// NT/64 doubles of LDS).  With FT (field-transposed), the four dwords of
// each 16-column group are spread across the four 16-byte quarters of
// their 64-column group: natural dword 4j + f of a 64-byte group is stored
// at dword 4f + j (xs_ft_dword).
template <int DT, int NT, int KCH, bool NORM = false, bool FT = false>
__device__ __forceinline__ void quantize_row(const Chunk<DT> ch[KCH], int K, int8_t* xs,
                                             float* red_f, int* red_i, float* s_scale,
                                             int* s_rowsum,
                                             const Gains<NT, KCH>* gn = nullptr,
                                             bool gain_on = false, float eps = 0.0f,
                                             double* red_d = nullptr) {
  constexpr int W = NT / kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Every chunk is used unconditionally (chunks past the row are zeros and
  // cannot raise the max), so the compiler keeps their loads where they
  // were issued instead of sinking them past the weight loads.
  float v[KCH][8];
  float amax = 0.0f;
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < KCH; ++c) {
    widen<DT>(ch[c], v[c]);
    if constexpr (NORM) {
      const float gv[8] = {__uint_as_float(gn->lo[c].x), __uint_as_float(gn->lo[c].y),
                           __uint_as_float(gn->lo[c].z), __uint_as_float(gn->lo[c].w),
                           __uint_as_float(gn->hi[c].x), __uint_as_float(gn->hi[c].y),
                           __uint_as_float(gn->hi[c].z), __uint_as_float(gn->hi[c].w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss = __builtin_fma((double)v[c][i], (double)v[c][i], ss);  // exact square: one rounding
        if (gain_on) v[c][i] = v[c][i] * gv[i];
      }
    }
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
      if constexpr (FT) {
        const int d = k >> 2;  // even: the pair d, d + 1 shares its group of 16 columns
        reinterpret_cast<uint32_t*>(xs)[xs_ft_dword(d)] = lo;
        reinterpret_cast<uint32_t*>(xs)[xs_ft_dword(d + 1)] = hi;
      } else {
        *reinterpret_cast<uint2*>(xs + k) = make_uint2(lo, hi);
      }
    }
  }
  sum = wave_sum(sum);
  // The sum of squares is needed only for the scale: reduced after the codes.
  if constexpr (NORM) ss = wave_sum_f64(ss);
  if (lane == 0) {
    red_i[wave] = sum;
    if constexpr (NORM) red_d[wave] = ss;
  }
  __syncthreads();  // also keeps the next row's red_f write after the reads above
  if (tid == 0) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) t += red_i[w];
    const float sc = a_c / kQmax;
    float rfac = 1.0f;
    if constexpr (NORM) {
      double S = red_d[0];
#pragma unroll
      for (int w = 1; w < W; ++w) S += red_d[w];
      if (gain_on) rfac = rms_factor(S, K, eps);
    }
    *s_scale = NORM && gain_on ? sc * rfac : sc;
    *s_rowsum = t;
  }
}

// Issues every packed-weight load of this lane for 16-row tile `tile`
// (kblocks <= L*W column blocks; wave w takes blocks w, w+W, ...).  Blocks
// past the tile's end read as zero through the buffer range check.  L is
// the exact number of loads the shape needs: out-of-range loads return zeros
// but still occupy the address and data paths.  Above four loads per lane
// they stream (non-temporal): measured on MI355X, 6912->2560 (7 loads) went
// from 3.90 to 3.60 us, while 2560->6912 (3 loads) went from 3.18 to 3.35.
template <int W, int L>
__device__ __forceinline__ void load_tile_weights(const uint8_t* __restrict__ packed,
                                                  int64_t tile, int kblocks, int wave,
                                                  int lane, uint4 (&wv)[L]) {
  const auto wr = make_rsrc(packed + tile * (int64_t)kblocks * kTileBytes,
                            (uint32_t)kblocks * kTileBytes);
#pragma unroll
  for (int i = 0; i < L; ++i)
    wv[i] = L > 4 ? buf_load16_stream(wr, lane * 16, (uint32_t)(wave + W * i) * kTileBytes)
                  : buf_load16(wr, lane * 16, (uint32_t)(wave + W * i) * kTileBytes);
}

// Unpacks this lane's weights and contracts them with the int8 activations
// xs [M][K] in LDS.  Returns, per token, the lane's partial sum of code * x
// over its blocks for row (lane mod 16) of the tile.
template <int M, int W, int L>
__device__ __forceinline__ void contract_tile(const uint4 (&wv)[L], const int8_t* xs,
                                              int K, int kblocks, int wave, int lane,
                                              int (&part)[M]) {
  int a0[M], a1[M], a2[M];
#pragma unroll
  for (int m = 0; m < M; ++m) a0[m] = a1[m] = a2[m] = 0;
  const int sub = lane >> 4;  // 64-column quarter of the 256-column block
#pragma unroll
  for (int i = 0; i < L; ++i) {
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
#pragma unroll
  for (int m = 0; m < M; ++m) part[m] = a0[m] + (a1[m] >> 2) + (a2[m] >> 4);
}

}  // namespace bl
