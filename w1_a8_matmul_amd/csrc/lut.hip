// Lookup-table decode GEMV for one token (T-MAC style).
//
// The ternary kernels of bitnet.cpp rest on T-MAC's lookup-table method
// (dignews.cc article on BitNet b1.58 2B4T, section 3): instead of
// multiplying weights by activations, the sums a small group of weights can
// produce with the current activations are tabulated once, and each group of
// packed weight codes indexes its table.  Here a group is two columns: for
// every column pair of the token's int8 activations (x_a, x_b) a 16-entry
// int16 table T[n] = (n & 3) x_a + (n >> 2) x_b sits in LDS, so a 4-bit field
// of the packed 2-bit layout (the codes of two columns) is its own index.
// A lane then reads one table entry per two weights instead of unpacking and
// multiplying.  The integer sum is the same as the dot-product kernels', so
// the outputs are bit-identical; what differs is the cost per weight.
//
// Layout facts this relies on: in a packed word, byte b holds the codes of
// columns 4f + b (f = 0..3) of its 16-column group, field f in bits 2f..2f+1;
// so the low nibble of byte b is the pair (b, b + 4) and the high nibble the
// pair (b + 8, b + 12).
#include "common.hpp"
#include "gemv_tile.hpp"
#include "launch.hpp"

#include <atomic>

namespace {

using namespace bl;

using lds_i16 = const __attribute__((address_space(3))) int16_t*;

constexpr int kNT = 256;
constexpr int kW = kNT / kWave;

// Byte offset of the table of column pair P (32 bytes each).  After every 32
// pairs (one 64-column quarter of a 256-column block) 32 bytes are skipped,
// so that the four quarters one wave reads at once start 8 banks apart; the
// 16 lanes of one quarter share its table and read entries of one 8-bank row.
__host__ __device__ constexpr int64_t lut_offset(int64_t P) { return 32 * (P + (P >> 5)); }

// Pair P of column block bk (128 pairs per block): quarter q = (P >> 5) & 3,
// word g = (P >> 3) & 3, byte b = (P >> 1) & 3, nibble h = P & 1; its first
// column is 256 bk + 64 q + 16 g + 8 h + b and the second is 4 further on.
__device__ __forceinline__ int pair_first_column(int P) {
  const int bk = P >> 7, q = (P >> 5) & 3, g = (P >> 3) & 3, b = (P >> 1) & 3, h = P & 1;
  return bk * kTileCols + q * 64 + g * 16 + h * 8 + b;
}

// base + byte b of v, in one instruction: the byte is selected by the
// operand's sub-dword select (SDWA), which the compiler does not form here
// by itself (it re-derives each byte from the packed word with a shift and
// a mask instead).
__device__ __forceinline__ uint32_t add_byte(int b, uint32_t base, uint32_t v) {
  uint32_t r;
  switch (b) {
    case 0:
      asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
          "src1_sel:BYTE_0" : "=v"(r) : "v"(base), "v"(v));
      break;
    case 1:
      asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
          "src1_sel:BYTE_1" : "=v"(r) : "v"(base), "v"(v));
      break;
    case 2:
      asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
          "src1_sel:BYTE_2" : "=v"(r) : "v"(base), "v"(v));
      break;
    default:
      asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "
          "src1_sel:BYTE_3" : "=v"(r) : "v"(base), "v"(v));
      break;
  }
  return r;
}

// One workgroup of 4 waves per 16-row tile, as the dot-product GEMV: wave w
// streams the tile's column blocks w, w + 4, ... (L loads per lane).  The
// weight loads are issued at entry; the token is quantized and the tables
// built while they are in flight.
template <int DT, int L>
__global__ __launch_bounds__(kNT) void lut_gemv_kernel(
    const void* __restrict__ X, int K, int64_t N, const uint8_t* __restrict__ packed,
    const float* __restrict__ gamma_p, float* __restrict__ Y, int epi,
    int8_t* __restrict__ xq_out, float* __restrict__ xscale_out,
    int32_t* __restrict__ acc_out) {
  constexpr int KCH = (L + 1) / 2;
  // All of LDS is the dynamic array, so that it starts at address 0 and the
  // table addresses need no further add: the tables, then the K int8 codes,
  // then the fold and reduction slots.
  extern __shared__ __align__(16) int8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile = blockIdx.x;
  const int kblocks = K / kTileCols;
  const int pairs = K / 2;
  int8_t* xs = smem + lut_offset(pairs);
  int(*partial)[kWave] = reinterpret_cast<int(*)[kWave]>(xs + K);
  float* red_f = reinterpret_cast<float*>(xs + K + kW * kWave * 4);
  int* red_i = reinterpret_cast<int*>(red_f + kW);
  float& s_scale = *reinterpret_cast<float*>(red_i + kW);
  int& s_rowsum = *reinterpret_cast<int*>(red_i + kW + 1);

  Chunk<DT> ch[KCH];
  load_row<DT, kNT, KCH>(X, 0, K, ch);
  uint4 wv[L];
  load_tile_weights<kW, L>(packed, tile, kblocks, wave, lane, wv);

  quantize_row<DT, kNT, KCH>(ch, K, xs, red_f, red_i, &s_scale, &s_rowsum);
  __syncthreads();

  // Tables: entry n of pair P is (n & 3) x_a + (n >> 2) x_b; entries with a
  // field of 3 are never indexed (codes are 0..2) and hold harmless values.
  for (int P = tid; P < pairs; P += kNT) {
    const int c = pair_first_column(P);
    const int xa = xs[c], xb = xs[c + 4];
    uint32_t d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int lo = ((2 * e) & 3) * xa + ((2 * e) >> 2) * xb;
      const int hi = ((2 * e + 1) & 3) * xa + ((2 * e + 1) >> 2) * xb;
      d[e] = ((uint32_t)lo & 0xffffu) | ((uint32_t)hi << 16);
    }
    uint4* t = reinterpret_cast<uint4*>(smem + lut_offset(P));
    t[0] = make_uint4(d[0], d[1], d[2], d[3]);
    t[1] = make_uint4(d[4], d[5], d[6], d[7]);
  }
  __syncthreads();

  // Lookups: per packed word, the low and high nibble of each byte, doubled
  // into byte offsets (two masks and two shifts per word), then one int16
  // read per nibble at the table of its pair.
  const int sub = lane >> 4;
  // LDS byte address of the array (a 32-bit local address), so that a table
  // address is one add from the packed byte.
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t*)smem;
  int acc = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int bk = wave + kW * i;
    if (bk < kblocks) {
      const uint32_t base_off = lds0 + (uint32_t)lut_offset((int64_t)bk * 128 + 32 * sub);
      const uint32_t words[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo2 = (words[g] << 1) & 0x1e1e1e1eu;  // 2 x low nibbles
        const uint32_t hi2 = (words[g] >> 3) & 0x1e1e1e1eu;  // 2 x high nibbles
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int j = 8 * g + 2 * b;  // pair of the low nibble within the quarter
          const int v0 = *reinterpret_cast<lds_i16>(
              (uintptr_t)(add_byte(b, base_off, lo2) + 32 * j));
          const int v1 = *reinterpret_cast<lds_i16>(
              (uintptr_t)(add_byte(b, base_off, hi2) + 32 * (j + 1)));
          acc += v0 + v1;
        }
      }
    }
  }
  partial[wave][lane] = acc;
  __syncthreads();

  // Lanes l, l + 16, l + 32, l + 48 of every wave hold tile row l % 16.
  if (tid < kTileRows) {
    const int r = tid;
    auto row_sum = [&](int row) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kW; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) s += partial[w][q * 16 + row];
      return s - s_rowsum;
    };
    const int acc_true = row_sum(r);
    const int64_t n = tile * kTileRows + r;
    const float gamma = *gamma_p;
    if (epi == kEpiGlu) {
      // rows r < 8 of the tile are gates, rows r + 8 their up rows
      if (r < 8) {
        const float yg = rescale(acc_true, s_scale, gamma, false);
        const float yu = rescale(row_sum(r + 8), s_scale, gamma, false);
        Y[tile * 8 + r] = glu_relu2(yg, yu);
      }
      if (acc_out) acc_out[glu_source_row(n, N)] = acc_true;
    } else {
      Y[n] = rescale(acc_true, s_scale, gamma, epi == kEpiRelu2);
      if (acc_out) acc_out[n] = acc_true;
    }
  }
  if (blockIdx.x == 0) {
    if (xq_out)
      for (int i = tid; i < K; i += kNT) xq_out[i] = xs[i];
    if (xscale_out && tid == 0) xscale_out[0] = s_scale;
  }
}

template <int DT, int L>
hipError_t launch_one(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                      const float* gamma, float* Y, int epi, int8_t* xq, float* xsc,
                      int32_t* acc, hipStream_t s) {
  const size_t lds = bl_lut_lds_bytes(K);
  // Above 64 KiB of LDS the kernel needs the attribute, once per device (a
  // bit per device; two threads may both set it, which is harmless).
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (lds > 65536 && !(attr_set.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lut_gemv_kernel<DT, L>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bl_lut_max_lds_bytes());
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((lut_gemv_kernel<DT, L>), dim3((unsigned)(N / kTileRows)), dim3(kNT), lds,
                     s, X, (int)K, N, packed, gamma, Y, epi, xq, xsc, acc);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const void* X, int64_t K, int64_t N, const uint8_t* packed,
                     const float* gamma, float* Y, int epi, int8_t* xq, float* xsc,
                     int32_t* acc, hipStream_t s) {
  const int64_t loads = (K / kTileCols + kW - 1) / kW;
#define BL_LUT_CASE(n) \
  if (loads <= n) return launch_one<DT, n>(X, K, N, packed, gamma, Y, epi, xq, xsc, acc, s);
  BL_LUT_CASE(1)
  BL_LUT_CASE(2)
  BL_LUT_CASE(3)
  BL_LUT_CASE(4)
  BL_LUT_CASE(5)
  BL_LUT_CASE(6)
  BL_LUT_CASE(7)
  BL_LUT_CASE(8)
#undef BL_LUT_CASE
  return hipErrorInvalidValue;
}

}  // namespace

size_t bl_lut_lds_bytes(int64_t K) {
  return (size_t)lut_offset(K / 2) + (size_t)K + kW * kWave * 4 + 2 * kW * 4 + 16;
}

size_t bl_lut_max_lds_bytes() { return bl_lut_lds_bytes(kLutMaxK); }

hipError_t bl_launch_lut_gemv(const void* X, int dtype, int64_t K, int64_t N,
                              const uint8_t* packed, const float* gamma, float* Y, int epi,
                              int8_t* xq_out, float* xscale_out, int32_t* acc_out,
                              hipStream_t s) {
  return dtype == 1 ? launch_dt<1>(X, K, N, packed, gamma, Y, epi, xq_out, xscale_out, acc_out, s)
                    : launch_dt<0>(X, K, N, packed, gamma, Y, epi, xq_out, xscale_out, acc_out, s);
}
