// Grouped decode forward: many independent BitLinear layers (same token
// count M <= 16) in one persistent launch instead of one launch per layer.
//
// Each workgroup owns a contiguous, byte-balanced range of 16-row output
// tiles taken from the concatenation of all layers.  Whenever it starts on a
// layer, the workgroup quantizes that layer's activation rows per token
// (absmax, int8) into LDS itself -- a few kilobytes read from L2, cheaper
// than a separate quantization launch -- while its waves' first weight
// loads are already in flight (above kGroupInlineQuantMaxM tokens a
// quantization launch does this once per layer and token, and workgroups
// copy the int8 rows instead).  Its waves then stream their tiles' packed
// weights in chunks of 16-byte lane loads (one 1 KiB block per wave load,
// chunks through two register buffers), unpack the 2-bit codes in registers
// and contract them on the int8 matrix cores (v_mfma_i32_16x16x64_i8, the
// tokens in the A rows; at one token the 16 rows repeat it).  Measured on
// MI355X, this beats the same loop contracting with v_dot4 on the vector ALU
// even at one token (2B step: 94.4-95.2 us against 101.3-101.7 us, same
// occupancy).  One launch keeps HBM busy across layer boundaries, where one
// launch per layer pays its start-up and drain for every few megabytes.
//
// The per-layer arithmetic is that of the single-layer forward: absmean
// ternary weights and per-token absmax int8 activations ("BitNet b1.58 2B4T
// Technical Report" card, section "Method Adaptation"), exact int32 sums,
// ((float)acc * s_x) * gamma.  The same loop also runs on weights in the
// base-3 layout (five codes per byte, B3 instantiations).
#include "common.hpp"
#include "gemv_tile.hpp"
#include "group.hpp"
#include "quant_row.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

constexpr int kChunk = 6;        // column blocks per streamed chunk
constexpr int kSegTiles = kGroupSegTiles;

// One 1 KiB block of a 16-row tile on the matrix cores.  Lane l loaded
// row l%16 of the tile, columns 64q .. 64q+63 of the block (q = l/16), as
// four words; word j holds the codes of columns 64q + 16j .. +15, field f of
// its byte b being column 64q + 16j + 4f + b.  MFMA f takes field f of all
// four words, left in place (codes times 1, 4 or 16; field 3 shifted down
// to times 1), so each operand costs one AND (two for field 3) instead of a
// shift and an AND per field.  Its 16 activation bytes are columns
// 64q + 16j + 4f .. +3 for j = 0..3, which the field-transposed LDS row
// (xs_ft_dword) keeps as one 16-byte read at 16f.  The four MFMAs cover the
// block's 256 columns for all 16 x 16 (token, row) pairs; acc4 and acc16
// hold 4 and 16 times their fields' sums (exact multiples, well inside int32
// for K <= 12288), so the tile's sum is acc1 + acc4 / 4 + acc16 / 16, taken
// with arithmetic shifts at the tile's end.
__device__ __forceinline__ void mfma_block(const uint4 w, const int8_t* xa, v4i& acc1,
                                           v4i& acc4, v4i& acc16) {
  auto operand = [&](uint32_t mask) {
    return v4i{(int)(w.x & mask), (int)(w.y & mask), (int)(w.z & mask), (int)(w.w & mask)};
  };
  const v4i* a = reinterpret_cast<const v4i*>(xa);
  acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], operand(kCodeMask), acc1, 0, 0, 0);
  acc4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], operand(kCodeMask << 2), acc4, 0, 0, 0);
  acc16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2], operand(kCodeMask << 4), acc16, 0, 0, 0);
  const v4i b3 = v4i{(int)((w.x >> 6) & kCodeMask), (int)((w.y >> 6) & kCodeMask),
                     (int)((w.z >> 6) & kCodeMask), (int)((w.w >> 6) & kCodeMask)};
  acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[3], b3, acc1, 0, 0, 0);
}

// The same block with the activation row in natural order: MFMA j takes
// word j, its four fields shifted down (dword f = field f, columns
// 64q + 16j + 4f .. +3) against the 16 activation bytes at 16j; two
// accumulators halve the dependent chain.  Seven VALU operations per word
// against five, but fewer registers: the multi-row inline quantization
// (two or three tokens) keeps three waves per SIMD with it, and drops to two
// with the in-place fields (2B step at M = 2: 101.7-105.1 against
// 104.5-106.5 us).
__device__ __forceinline__ void mfma_block_shifted(const uint4 w, const int8_t* xa, v4i& acc0,
                                                   v4i& acc1) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v4i a = *reinterpret_cast<const v4i*>(xa + 16 * k);
    const uint32_t wd = words[k];
    const v4i b = v4i{(int)codes(wd, 0), (int)codes(wd, 1), (int)codes(wd, 2), (int)codes(wd, 3)};
    if (k % 2 == 0)
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc0, 0, 0, 0);
    else
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc1, 0, 0, 0);
  }
}

// The base-3 layout (five codes per byte): the lane's 16 bytes (row l % 16,
// columns 80q .. 80q + 79 of a 320-column block) decode into 20 dwords of
// four int8 codes, dword t holding columns 4t .. 4t + 3 (byte b of packed
// word j carries columns 20j + 4i + b as its base-3 digits i).  MFMA m
// contracts dwords 4m .. 4m + 3, columns 16m .. 16m + 15, with the same 16
// activation bytes.  Digits come two bytes at a time in 16-bit lanes:
// v / 3 = (v * 171) >> 9 exactly for v <= 255, digit = v - 3 (v / 3).
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t us2_bits(us2 v) { return __builtin_bit_cast(uint32_t, v); }

// The five digit dwords of one packed word: d_i holds digit i of its four
// bytes (codes of four consecutive columns).
struct B3Digits {
  uint32_t d0, d1, d2, d3, d4;
};

__device__ __forceinline__ B3Digits b3_word_digits(uint32_t w) {
  us2 lo = __builtin_bit_cast(us2, w & 0x00ff00ffu);         // bytes 0 and 2
  us2 hi = __builtin_bit_cast(us2, (w >> 8) & 0x00ff00ffu);  // bytes 1 and 3
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const us2 ql = (lo * (unsigned short)171) >> (unsigned short)9;
    const us2 qh = (hi * (unsigned short)171) >> (unsigned short)9;
    const us2 dl = lo - ql * (unsigned short)3, dh = hi - qh * (unsigned short)3;
    d[i] = us2_bits(dl) | (us2_bits(dh) << 8);
    lo = ql;
    hi = qh;
  }
  return B3Digits{d[0], d[1], d[2], d[3], us2_bits(lo) | (us2_bits(hi) << 8)};
}

// Five MFMAs per block, each fed as soon as its 16 codes are decoded: the
// 20 digit dwords run through the four words in order, four per MFMA.
__device__ __forceinline__ void mfma_block_b3(const uint4 w, const int8_t* xa, v4i& acc0,
                                              v4i& acc1) {
  auto mma = [&](int m, uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, v4i& acc) {
    const v4i a = *reinterpret_cast<const v4i*>(xa + 16 * m);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, v4i{(int)c0, (int)c1, (int)c2, (int)c3},
                                                acc, 0, 0, 0);
  };
  const B3Digits x = b3_word_digits(w.x);
  mma(0, x.d0, x.d1, x.d2, x.d3, acc0);
  const B3Digits y = b3_word_digits(w.y);
  mma(1, x.d4, y.d0, y.d1, y.d2, acc1);
  const B3Digits z = b3_word_digits(w.z);
  mma(2, y.d3, y.d4, z.d0, z.d1, acc0);
  const B3Digits t = b3_word_digits(w.w);
  mma(3, z.d2, z.d3, z.d4, t.d0, acc1);
  mma(4, t.d1, t.d2, t.d3, t.d4, acc0);
}

template <int NT>
struct Smem {
  float red_f[NT / kWave];
  int red_i[NT / kWave];
  double red_d[NT / kWave];
};

// One layer segment: tiles first, first+stride, ... < last of layer o for
// this wave.  Each tile is cut into chunks of kChunk column blocks.
// Chunks past the end of a tile or of the wave's work use an empty or short
// buffer range and read zeros.
// PREQ: the activations were quantized by the separate launch; the
// segment copies its layer's int8 rows, scales and row sums into LDS instead.
// NORM (inline quantization only): layers with a subln gain get it applied
// before their quantization.  MR (inline quantization, M > 1): the next
// token row is loaded while the current one is quantized.  B3: the weights
// use the base-3 layout (blocks of 16 rows x 320 columns, K padded to 320).
template <int NT, int KCH, int DT, bool PREQ, bool NORM, bool MR, bool B3>
__device__ __forceinline__ void run_segment(const GroupOp& o, int M, int first, int last,
                                            bool quantize, int8_t* xs, int xstride,
                                            float* s_sx, int* s_rs, float* s_y, Smem<NT>& sm,
                                            const int8_t* __restrict__ xq,
                                            const float* __restrict__ sx,
                                            const int* __restrict__ rs, int op, int wave,
                                            int lane) {
  constexpr int kThreads = NT;
  constexpr int kWaves = NT / kWave;
  constexpr int C = kChunk;
  constexpr int kBlockCols = B3 ? kB3TileCols : kTileCols;  // columns per 1 KiB block
  // Field-transposed activation rows and the in-place field MFMAs, except
  // for the base-3 layout and the multi-row inline quantization.
  constexpr bool FT = !B3 && !MR;
  const int K = o.K;
  const int kblocks = B3 ? (K + kB3TileCols - 1) / kB3TileCols : K / kTileCols;
  const int nc = (kblocks + C - 1) / C;
  const int stride = kWaves;
  const int mine = first + wave;
  const int n_mine = mine < last ? (last - mine + stride - 1) / stride : 0;
  const int total = n_mine * nc;
  const int q16 = lane >> 4;                     // quarter of the block held by this lane
  const int arow = min(lane & 15, M - 1);        // token row of this lane's A operand

  // Chunk cursors (tile, chunk within the tile) advance with selects only:
  // a branch here, or a division the compiler skips with one, would make it
  // wait for every outstanding load where the paths join.
  struct Cursor {
    int it, c;
  };
  auto advance = [&](Cursor& q) {
    const bool wrap = q.c + 1 == nc;
    q.it = wrap ? q.it + stride : q.it;
    q.c = wrap ? 0 : q.c + 1;
  };
  auto issue = [&](uint4 (&buf)[C], int j, const Cursor& q) {
    const bool valid = j < total;
    const int tr = valid ? q.it - o.item_begin : 0;
    const auto r = make_rsrc(o.packed + (int64_t)tr * kblocks * kTileBytes,
                             valid ? (uint32_t)kblocks * kTileBytes : 0u);
#pragma unroll
    for (int i = 0; i < C; ++i)
      buf[i] = buf_load16_stream(r, lane * 16, (uint32_t)(q.c * C + i) * kTileBytes);
  };

  // Activation row 0 first, then the first weight chunk, then the
  // quantization (which waits for the row but not for the weights); or the
  // first weight chunk, then the copy of the quantized rows.
  uint4 bufA[C], bufB[C];
  Cursor qi{mine, 0};  // next chunk to issue
  Cursor qc{mine, 0};  // next chunk to consume
  if (PREQ) {
    issue(bufA, 0, qi);
    if (quantize) {
      // The layer's int8 rows, in batches of kCopyBatch 16-byte pieces per
      // thread: every load of a batch is issued before its LDS stores (loads
      // past the rows read zero through the buffer range, no branch), so a
      // batch costs one L2 round trip.  One piece per iteration made the
      // copy wait for a round trip per piece: 27 at M = 16, K = 6912.
      constexpr int kCopyBatch = 8;
      const int row16 = K / 16;  // 16-byte pieces per row
      const int n16 = M * row16;
      const auto xr = make_rsrc(xq + o.xq_off, (uint32_t)n16 * 16u);
      for (int b0 = 0; b0 < n16; b0 += kCopyBatch * kThreads) {
        uint4 v[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u)
          v[u] = buf_load16(xr, (uint32_t)(b0 + u * kThreads + (int)threadIdx.x) * 16u, 0);
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
          const int i = b0 + u * kThreads + (int)threadIdx.x;
          if (i < n16) {
            const int m = i / row16, c = i - m * row16;
            if constexpr (!FT) {
              *reinterpret_cast<uint4*>(xs + m * xstride + c * 16) = v[u];
            } else {  // field-transposed: dword 4c + t of the row goes to xs_ft_dword
              uint32_t* row = reinterpret_cast<uint32_t*>(xs + m * xstride);
              row[xs_ft_dword(4 * c)] = v[u].x;
              row[xs_ft_dword(4 * c + 1)] = v[u].y;
              row[xs_ft_dword(4 * c + 2)] = v[u].z;
              row[xs_ft_dword(4 * c + 3)] = v[u].w;
            }
          }
        }
      }
      if ((int)threadIdx.x < M) {
        s_sx[threadIdx.x] = sx[op * M + threadIdx.x];
        s_rs[threadIdx.x] = rs[op * M + threadIdx.x];
      }
    }
  } else if (quantize && MR) {
    // Up to four token rows (M <= kGroupInlineQuantMaxM), straight-line code:
    // rows 0 and 1 before the first weight chunk, row m + 2 issued before
    // row m + 1 is quantized, so no quantization waits for a round trip of
    // its own (rows past M read zero and are not quantized).  One row at a
    // time cost a round trip per row at every new layer.
    static_assert(kGroupInlineQuantMaxM <= 4, "the multi-row quantization handles four rows");
    Chunk<DT> ch[KCH], nx[KCH];
    load_row<DT, kThreads, KCH>(o.X, 0, K, ch);
    Gains<kThreads, KCH> gn;
    if constexpr (NORM) load_gains<kThreads, KCH>(o.norm_gain, K, gn);
    const bool gain_on = NORM && o.norm_gain != nullptr;
    load_row<DT, kThreads, KCH>(o.X, 1, K, nx, M > 1);
    issue(bufA, 0, qi);
    auto quant = [&](const Chunk<DT>(&c)[KCH], int m) {
      quantize_row<DT, kThreads, KCH, NORM, FT>(c, K, xs + m * xstride, sm.red_f, sm.red_i,
                                                s_sx + m, s_rs + m, &gn, gain_on, o.norm_eps,
                                                sm.red_d);
    };
    quant(ch, 0);
    load_row<DT, kThreads, KCH>(o.X, 2, K, ch, M > 2);
    if (M > 1) quant(nx, 1);
    load_row<DT, kThreads, KCH>(o.X, 3, K, nx, M > 3);
    if (M > 2) quant(ch, 2);
    if (M > 3) quant(nx, 3);
  } else if (quantize) {
    Chunk<DT> ch[KCH];
    load_row<DT, kThreads, KCH>(o.X, 0, K, ch);
    Gains<kThreads, KCH> gn;
    if constexpr (NORM) load_gains<kThreads, KCH>(o.norm_gain, K, gn);
    const bool gain_on = NORM && o.norm_gain != nullptr;
    issue(bufA, 0, qi);
    quantize_row<DT, kThreads, KCH, NORM, FT>(ch, K, xs, sm.red_f, sm.red_i, s_sx, s_rs, &gn,
                                              gain_on, o.norm_eps, sm.red_d);
    for (int m = 1; m < M; ++m) {
      Chunk<DT> chm[KCH];
      load_row<DT, kThreads, KCH>(o.X, m, K, chm);
      quantize_row<DT, kThreads, KCH, NORM, FT>(chm, K, xs + m * xstride, sm.red_f, sm.red_i,
                                                s_sx + m, s_rs + m, &gn, gain_on, o.norm_eps,
                                                sm.red_d);
    }
  } else {
    issue(bufA, 0, qi);
  }
  advance(qi);
  __syncthreads();

  const float gamma = *o.gamma;
  const int8_t* xrow = xs + arow * xstride + q16 * (kBlockCols / 4);
  v4i acc0 = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0}, acc2 = v4i{0, 0, 0, 0};

  // D layout: lane l holds tile row l%16 and tokens 4*(l/16) + r, r = 0..3.
  auto consume = [&](const uint4 (&buf)[C], int j, Cursor& q) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int b = min(q.c * C + i, kblocks - 1);  // past the end: zero codes, any x
      if constexpr (B3)
        mfma_block_b3(buf[i], xrow + b * kBlockCols, acc0, acc1);
      else if constexpr (FT)
        mfma_block(buf[i], xrow + b * kBlockCols, acc0, acc1, acc2);
      else
        mfma_block_shifted(buf[i], xrow + b * kBlockCols, acc0, acc1);
    }
    if (q.c == nc - 1) {
      const v4i d = FT ? acc0 + (acc1 >> 2) + (acc2 >> 4) : acc0 + acc1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * q16 + r;
        if (m < M && j < total)
          s_y[(m * kSegTiles + (q.it - first)) * kTileRows + (lane & 15)] =
              rescale(d[r] - s_rs[m], s_sx[m], gamma, o.epi == kEpiRelu2);
      }
      acc0 = v4i{0, 0, 0, 0};
      acc1 = v4i{0, 0, 0, 0};
      acc2 = v4i{0, 0, 0, 0};
    }
    advance(q);
  };

  // Rounds of four chunks through two buffers: while one chunk is
  // contracted the next is in flight.  Every load is consumed within its
  // round: a load whose result crosses a loop's back edge, or a branch
  // around loads, makes the compiler wait for every outstanding load before
  // the first use, which would serialize the chunks.  The first round (chunk
  // 0 already in flight since before the quantization) runs
  // unconditionally; a wave with no tiles reads zeros and stores nothing.
  auto rest_of_round = [&](int j) {
    issue(bufB, j + 1, qi);
    advance(qi);
    consume(bufA, j, qc);
    issue(bufA, j + 2, qi);
    advance(qi);
    consume(bufB, j + 1, qc);
    issue(bufB, j + 3, qi);
    advance(qi);
    consume(bufA, j + 2, qc);
    consume(bufB, j + 3, qc);
  };
  rest_of_round(0);
  for (int j = 4; j < total; j += 4) {
    issue(bufA, j, qi);
    advance(qi);
    rest_of_round(j);
  }

  // Outputs of the segment's tiles, from LDS, in row order.  Stores are kept
  // out of the streaming loop: with loads and stores outstanding together the
  // compiler can no longer count loads in order and waits for all of them.
  __syncthreads();
  const int rows = (last - first) * kTileRows;
  const int64_t n0 = (int64_t)(first - o.item_begin) * kTileRows;
  // Four consecutive outputs per thread and store (16 bytes): at 16 tokens
  // this took the 2B step from 139-140 to 133-136 us against one float per
  // store.
  if (o.epi == kEpiGlu) {
    // interleaved gate+up tiles: rows 0..7 gates, 8..15 their up rows;
    // output row r of the segment is gate row r (tile r/8) of N/2
    const int q4 = rows / 8;
    for (int i = threadIdx.x; i < M * q4; i += kThreads) {
      const int m = i / q4, r = (i - m * q4) * 4;
      const float* ty = s_y + m * kSegTiles * kTileRows + (r / 8) * kTileRows + (r % 8);
      const float4 g = *reinterpret_cast<const float4*>(ty);
      const float4 u = *reinterpret_cast<const float4*>(ty + 8);
      *reinterpret_cast<float4*>(o.Y + m * (int64_t)(o.N / 2) + n0 / 2 + r) =
          make_float4(glu_relu2(g.x, u.x), glu_relu2(g.y, u.y), glu_relu2(g.z, u.z),
                      glu_relu2(g.w, u.w));
    }
  } else {
    const int q4 = rows / 4;
    for (int i = threadIdx.x; i < M * q4; i += kThreads) {
      const int m = i / q4, r = (i - m * q4) * 4;
      *reinterpret_cast<float4*>(o.Y + m * (int64_t)o.N + n0 + r) =
          *reinterpret_cast<const float4*>(s_y + m * kSegTiles * kTileRows + r);
    }
  }
}

// Many layers.  Work is in two parts.  First a static, cost-balanced
// contiguous range of 16-row tiles per workgroup (wg_begin[g] ..
// wg_begin[g+1]-1), run in segments of at most kSegTiles tiles of one layer.
// Then units of about kGroupUnitBlocks weight blocks of one layer (the rest of the
// tiles, in layer order) taken from a queue as workgroups become free.  The
// workgroups of a compute unit do not stream at the same rate (the oldest
// wave wins arbitration), so static shares alone leave a long tail with few
// workgroups streaming; the queue keeps them all busy to the end, and the
// static part keeps the per-unit set-up (quantizing a new layer's
// activations) off most of the work.  queue[0] is the next unit, queue[1]
// counts the workgroups that found the queue empty; the last of them puts
// both back to zero for the next launch.  A layer's int8 activations are
// quantized (or copied) whenever a workgroup moves to a new layer.
template <int NT, int KCH, bool PREQ, bool NORM, bool MR, bool B3>
__global__ __launch_bounds__(NT) void group_kernel(const GroupOp* __restrict__ ops, int n_ops,
                                                   int M, int max_k,
                                                   const int* __restrict__ wg_begin,
                                                   const GroupUnit* __restrict__ units,
                                                   int n_units, int* __restrict__ queue,
                                                   const int8_t* __restrict__ xq,
                                                   const float* __restrict__ sx,
                                                   const int* __restrict__ rs) {
  extern __shared__ __align__(16) int8_t dyn[];
  __shared__ float s_sx[kGroupMaxM];
  __shared__ int s_rs[kGroupMaxM];
  __shared__ Smem<NT> sm;
  __shared__ int s_unit;
  // Dynamic LDS: int8 activations [M][max_k + 16] of the current layer (rows
  // padded by 16 bytes so that the 16 token rows of an A-operand read fall in
  // distinct banks), then a segment's outputs [M][kSegTiles][16] floats.
  const int xstride = max_k + 16;
  int8_t* xs = dyn;
  float* s_y = reinterpret_cast<float*>(dyn + (size_t)M * xstride);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int quantized_op = -1;
  // Tiles first .. end-1 of layer op (end - first <= kSegTiles).
  auto segment = [&](int op, int first, int end) __attribute__((always_inline)) {
    const GroupOp o = ops[op];
    const bool quantize = quantized_op != op;
    if (PREQ)
      run_segment<NT, KCH, 0, true, false, false, B3>(o, M, first, end, quantize, xs, xstride,
                                                      s_sx, s_rs, s_y, sm, xq, sx, rs, op, wave,
                                                      lane);
    else if (o.dtype == 1)
      run_segment<NT, KCH, 1, false, NORM, MR, B3>(o, M, first, end, quantize, xs, xstride, s_sx,
                                                   s_rs, s_y, sm, xq, sx, rs, op, wave, lane);
    else
      run_segment<NT, KCH, 0, false, NORM, MR, B3>(o, M, first, end, quantize, xs, xstride, s_sx,
                                                   s_rs, s_y, sm, xq, sx, rs, op, wave, lane);
    __syncthreads();  // before the next segment overwrites xs, the scales, s_y or s_unit
    quantized_op = op;
  };

  // Static part.
  int item = wg_begin[blockIdx.x];
  const int end = wg_begin[blockIdx.x + 1];
  int op = 0;
  while (op + 1 < n_ops && ops[op + 1].item_begin <= item) ++op;
  while (item < end) {
    const int op_end = ops[op].item_begin + ops[op].N / kTileRows;
    const int seg_end = min(min(end, op_end), item + kSegTiles);
    segment(op, item, seg_end);
    item = seg_end;
    if (item == op_end) ++op;
  }
  // Shared part.
  for (;;) {
    if (threadIdx.x == 0)
      s_unit = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int u = s_unit;
    if (u >= n_units) break;
    const GroupUnit un = units[u];
    segment(un.op, un.first, un.end);
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          (int)gridDim.x - 1) {
    // Every workgroup is past its last take from the queue.
    __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Per-token quantization of every layer's activations (one workgroup per
// layer and token) into the workspace, for the larger token counts.  This
// two-pass form serves layers wider than the one-pass kernel below takes.
__global__ __launch_bounds__(256) void group_quant_loop_kernel(const GroupOp* __restrict__ ops, int M,
                                                          int8_t* __restrict__ xq,
                                                          float* __restrict__ sx,
                                                          int* __restrict__ rs) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  __shared__ double red_d[4];
  const int op = blockIdx.x / M, m = blockIdx.x % M;
  const GroupOp o = ops[op];
  int8_t* dst = xq + o.xq_off + (int64_t)m * o.K;
  const float* g = o.norm_gain;
  RowQuant q;
  int sum;
  if (g && o.dtype == 1) {
    q = row_absmax_scale<1, 256, true>(o.X, m, o.K, red_f, g, o.norm_eps, red_d);
    sum = row_quantize_to<1, 256, true>(o.X, m, o.K, q.qs, dst, red_i, g);
  } else if (g) {
    q = row_absmax_scale<0, 256, true>(o.X, m, o.K, red_f, g, o.norm_eps, red_d);
    sum = row_quantize_to<0, 256, true>(o.X, m, o.K, q.qs, dst, red_i, g);
  } else if (o.dtype == 1) {
    q = row_absmax_scale<1, 256>(o.X, m, o.K, red_f);
    sum = row_quantize_to<1, 256>(o.X, m, o.K, q.qs, dst, red_i);
  } else {
    q = row_absmax_scale<0, 256>(o.X, m, o.K, red_f);
    sum = row_quantize_to<0, 256>(o.X, m, o.K, q.qs, dst, red_i);
  }
  if (threadIdx.x == 0) {
    const float sc = q.a_c / kQmax;
    sx[op * M + m] = g ? sc * q.r : sc;
    rs[op * M + m] = sum;
  }
}

// One pass for layers of at most KCH * 2048 columns: the row's chunks (and
// any subln gains) are loaded at entry and stay in registers through the
// max reduction; same arithmetic, in the same order, as the two-pass form.
// NORM: some layer of the group has a subln gain (a layer without one then
// reads an empty range of zeros and skips it).  Without it the kernel holds
// no gain registers: at 6 chunks 64 registers instead of 154 (8 waves per
// SIMD instead of 3), at 4 chunks 48 instead of 106.
template <int DT, int KCH, bool NORM>
__device__ __forceinline__ void group_quant_row(const GroupOp& o, int m, int8_t* dst,
                                                float* red_f, int* red_i, double* red_d,
                                                float* s_scale, int* s_rowsum) {
  Chunk<DT> ch[KCH];
  load_row<DT, 256, KCH>(o.X, m, o.K, ch);
  if constexpr (NORM) {
    Gains<256, KCH> gn;
    load_gains<256, KCH>(o.norm_gain, o.K, gn);  // no gain: an empty range, zeros
    if (o.norm_gain) {
      quantize_row<DT, 256, KCH, true>(ch, o.K, dst, red_f, red_i, s_scale, s_rowsum, &gn, true,
                                       o.norm_eps, red_d);
      return;
    }
  }
  quantize_row<DT, 256, KCH, false>(ch, o.K, dst, red_f, red_i, s_scale, s_rowsum);
}

template <int KCH, bool NORM>
__global__ __launch_bounds__(256) void group_quant_kernel(const GroupOp* __restrict__ ops, int M,
                                                          int8_t* __restrict__ xq,
                                                          float* __restrict__ sx,
                                                          int* __restrict__ rs) {
  __shared__ float red_f[4];
  __shared__ int red_i[4];
  __shared__ double red_d[4];
  __shared__ float s_scale;
  __shared__ int s_rowsum;
  const int op = blockIdx.x / M, m = blockIdx.x % M;
  const GroupOp o = ops[op];
  int8_t* dst = xq + o.xq_off + (int64_t)m * o.K;
  if (o.dtype == 1)
    group_quant_row<1, KCH, NORM>(o, m, dst, red_f, red_i, red_d, &s_scale, &s_rowsum);
  else
    group_quant_row<0, KCH, NORM>(o, m, dst, red_f, red_i, red_d, &s_scale, &s_rowsum);
  if (threadIdx.x == 0) {  // thread 0 wrote both
    sx[op * M + m] = s_scale;
    rs[op * M + m] = s_rowsum;
  }
}

// Activation chunks per thread: each covers NT * 8 elements of a row.
// Kernel modes: pre-quantized (the quantization launch applies any subln);
// inline quantization without or with subln gains, of one row or of
// several; each for the 2-bit and the base-3 weight layout.
template <int NT, bool PREQ, bool NORM, bool MR, bool B3>
const void* kernel_for(int max_k) {
  if (max_k <= NT * 8 * 2)
    return reinterpret_cast<const void*>(&group_kernel<NT, 2, PREQ, NORM, MR, B3>);
  if (max_k <= NT * 8 * 4)
    return reinterpret_cast<const void*>(&group_kernel<NT, 4, PREQ, NORM, MR, B3>);
  return reinterpret_cast<const void*>(&group_kernel<NT, 6, PREQ, NORM, MR, B3>);
}

template <int NT, bool NORM, bool B3>
const void* kernel_for(bool mr, int max_k) {
  return mr ? kernel_for<NT, false, NORM, true, B3>(max_k)
            : kernel_for<NT, false, NORM, false, B3>(max_k);
}

template <bool B3>
const void* kernel_for(int threads, int M, bool norm, int max_k) {
  const bool preq = bl_group_prequantizes(M), mr = M > 1;
  if (threads == 512) {
    if (preq) return kernel_for<512, true, false, false, B3>(max_k);
    return norm ? kernel_for<512, true, B3>(mr, max_k) : kernel_for<512, false, B3>(mr, max_k);
  }
  if (preq) return kernel_for<256, true, false, false, B3>(max_k);
  return norm ? kernel_for<256, true, B3>(mr, max_k) : kernel_for<256, false, B3>(mr, max_k);
}

// The kernel a launch for M tokens uses.
const void* kernel_for(int threads, int M, bool norm, bool b3, int max_k) {
  return b3 ? kernel_for<true>(threads, M, norm, max_k)
            : kernel_for<false>(threads, M, norm, max_k);
}

template <int NT, bool PREQ, bool NORM, bool MR, bool B3>
void launch(const GroupOp* ops, int n_ops, int M, const int* wg_begin, const GroupUnit* units,
            int n_units, int* queue, int G, int max_k, size_t lds, const int8_t* xq,
            const float* sx, const int* rs, hipStream_t s) {
  if (max_k <= NT * 8 * 2)
    hipLaunchKernelGGL((group_kernel<NT, 2, PREQ, NORM, MR, B3>), dim3(G), dim3(NT), lds, s,
                       ops, n_ops, M, max_k, wg_begin, units, n_units, queue, xq, sx, rs);
  else if (max_k <= NT * 8 * 4)
    hipLaunchKernelGGL((group_kernel<NT, 4, PREQ, NORM, MR, B3>), dim3(G), dim3(NT), lds, s,
                       ops, n_ops, M, max_k, wg_begin, units, n_units, queue, xq, sx, rs);
  else
    hipLaunchKernelGGL((group_kernel<NT, 6, PREQ, NORM, MR, B3>), dim3(G), dim3(NT), lds, s,
                       ops, n_ops, M, max_k, wg_begin, units, n_units, queue, xq, sx, rs);
}

template <int NT, bool B3>
void launch(bool norm, const GroupOp* ops, int n_ops, int M, const int* wg_begin,
            const GroupUnit* units, int n_units, int* queue, int G, int max_k, size_t lds,
            const int8_t* xq, const float* sx, const int* rs, hipStream_t s) {
#define BL_GROUP_LAUNCH(P, NM, MRV)                                                         \
  launch<NT, P, NM, MRV, B3>(ops, n_ops, M, wg_begin, units, n_units, queue, G, max_k, lds, \
                             xq, sx, rs, s)
  if (bl_group_prequantizes(M))
    BL_GROUP_LAUNCH(true, false, false);
  else if (norm)
    M > 1 ? BL_GROUP_LAUNCH(false, true, true) : BL_GROUP_LAUNCH(false, true, false);
  else
    M > 1 ? BL_GROUP_LAUNCH(false, false, true) : BL_GROUP_LAUNCH(false, false, false);
#undef BL_GROUP_LAUNCH
}

int blocks_per_cu(int threads, int M, bool norm, bool b3, size_t lds, int max_k) {
  int blocks = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &blocks, kernel_for(threads, M, norm, b3, max_k), threads, lds);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

}  // namespace

bool bl_group_prequantizes(int M) { return M > kGroupInlineQuantMaxM; }

hipError_t bl_launch_group_quant(const GroupOp* ops, int n_ops, int M, int max_k, bool norm,
                                 int8_t* xq, float* sx, int* rs, hipStream_t s) {
  const dim3 grid((unsigned)(n_ops * M)), block(256);
#define BL_GROUP_QUANT(KCH)                                                                  \
  if (norm)                                                                                  \
    hipLaunchKernelGGL((group_quant_kernel<KCH, true>), grid, block, 0, s, ops, M, xq, sx, rs); \
  else                                                                                       \
    hipLaunchKernelGGL((group_quant_kernel<KCH, false>), grid, block, 0, s, ops, M, xq, sx, rs)
  if (max_k <= 2048) {
    BL_GROUP_QUANT(1);
  } else if (max_k <= 4096) {
    BL_GROUP_QUANT(2);
  } else if (max_k <= 8192) {
    BL_GROUP_QUANT(4);
  } else if (max_k <= 12288) {
    BL_GROUP_QUANT(6);
  } else
    hipLaunchKernelGGL(group_quant_loop_kernel, grid, block, 0, s, ops, M, xq, sx, rs);
#undef BL_GROUP_QUANT
  return hipGetLastError();
}

size_t bl_group_lds_bytes(int M, int max_k) {
  return (size_t)M * (size_t)(max_k + 16) + (size_t)M * kSegTiles * kTileRows * sizeof(float);
}

hipError_t bl_group_plan(int M, int max_k, bool norm, bool b3, int* threads, int* per_cu) {
  const size_t lds = bl_group_lds_bytes(M, max_k);
  for (int nt : {256, 512}) {
    if (lds > 64 * 1024) {
      const hipError_t e =
          hipFuncSetAttribute(kernel_for(nt, M, norm, b3, max_k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
  }
  // Four-wave workgroups while at least two fit on a compute unit (more,
  // shorter weight streams); eight-wave ones when the activations take so
  // much LDS that only one does.  (Sixteen waves on pre-quantized rows, four
  // per SIMD instead of two, measured no faster at 16 tokens: 138.7 against
  // 140.4 us, within the spread of runs.)
  const int b256 = blocks_per_cu(256, M, norm, b3, lds, max_k);
  if (b256 >= 2) {
    *threads = 256;
    *per_cu = b256;
  } else {
    *threads = 512;
    *per_cu = blocks_per_cu(512, M, norm, b3, lds, max_k);
  }
  return hipSuccess;
}

hipError_t bl_launch_group(const GroupOp* ops, int n_ops, int M, const int* wg_begin,
                           const GroupUnit* units, int n_units, int* queue, int G, int max_k,
                           int threads, bool norm, bool b3, int8_t* xq, float* sx, int* rs,
                           hipStream_t s) {
  const size_t lds = bl_group_lds_bytes(M, max_k);
  const bool preq = bl_group_prequantizes(M);
  if (preq) {
    const hipError_t e = bl_launch_group_quant(ops, n_ops, M, max_k, norm, xq, sx, rs, s);
    if (e != hipSuccess) return e;
  }
  if (threads == 512 && b3)
    launch<512, true>(norm, ops, n_ops, M, wg_begin, units, n_units, queue, G, max_k, lds, xq,
                      sx, rs, s);
  else if (threads == 512)
    launch<512, false>(norm, ops, n_ops, M, wg_begin, units, n_units, queue, G, max_k, lds, xq,
                       sx, rs, s);
  else if (b3)
    launch<256, true>(norm, ops, n_ops, M, wg_begin, units, n_units, queue, G, max_k, lds, xq,
                      sx, rs, s);
  else
    launch<256, false>(norm, ops, n_ops, M, wg_begin, units, n_units, queue, G, max_k, lds, xq,
                       sx, rs, s);
  return hipGetLastError();
}
