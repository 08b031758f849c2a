// BitLinear forward from int8 activations on the CDNA4 int8 matrix cores,
// 32x32x32 form (v_mfma_i32_32x32x32_i8).  For larger M the ternary x int8
// product is a dense contraction (prefill): the 2-bit codes are unpacked in
// registers into MFMA B operands and multiplied against int8 activation
// tiles.  On gfx950 the 32x32x32 int8 instruction sustains about 1.7x the
// rate of the 16x16x64 one (measured: ~3.5 vs ~2.0 POP/s with random
// operands at 8 waves per CU), so the tiles are built around it.
//
// A workgroup of WM x WN waves computes a (32*TM*WM) x (32*TN*WN) output
// tile, walking K in steps of 128 columns (half of a packed 256-column
// block).  Each step's int8 activation rows (A) and packed weight half-tiles
// (B, still 2 bits per weight) are copied into LDS by direct-to-LDS buffer
// loads (no register staging) into a ring of S stages, up to S steps ahead of
// the multiply; each wave reads the fragments of the next half step (64
// columns) into registers while the MFMAs of the current one run.
//
// Operands of one MFMA (32 rows or columns, 32 k): lane l supplies row (or
// column) l % 32 and 16 k values, the lanes 0-31 one set and 32-63 another;
// any k order works as long as A and B use the same one.  For the 64-column
// group p of a step, lane half h takes packed words 2h and 2h+1 of its row's
// 16-byte chunk (one 8-byte LDS read) -- word w holds the codes of columns
// 16w .. 16w+15 of the group -- and MFMA u (0, 1) of the group uses word
// 2h+u with the matching 16 activation columns 64p + 32h + 16u .. +15.
// Codes are q+1 in {0,1,2}; the activation row sums turn sum(code*x) into
// sum(q*x) exactly in the epilogue.
//
// The load/unpack/multiply order follows the kernel outline of the "BitNet
// b1.58 2B4T Technical Report" card, section "Method Adaptation"; the tiling
// is this library's own, for gfx950.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "group.hpp"
#include "launch.hpp"

namespace {

using namespace bl;

typedef __attribute__((address_space(3))) void lds_void;
typedef int v16i __attribute__((ext_vector_type(16)));

// Raw buffer descriptor (gfx9 layout: 48-bit base, stride 0, byte range,
// raw-buffer format word) for the copies below.
__device__ __forceinline__ v4i rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// One wave-wide direct-to-LDS copy: lane j's 16 bytes at voff land at
// lds + 16*j (lds is wave-uniform).  Offsets at or past the range read zeros
// without touching memory.  Written as inline asm so that the compiler does
// not track these LDS writes itself: it can follow only one outstanding
// copy per LDS object and would otherwise wait for the next step's copies
// before reading the current step.  The kernel orders the copies with
// explicit vmcnt waits and barriers.  M0 holds the LDS base (read when the
// instruction issues; one wait state after writing it); no other code in the
// kernel uses M0.
__device__ __forceinline__ void copy16(v4i rs, uint32_t voff, void* lds) {
  const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(voff), "s"(la), "s"(rs) : "memory", "m0");
}

// The same copy with the non-temporal (streaming) policy: for weight tiles
// that no other workgroup will read.
__device__ __forceinline__ void copy16_nt(v4i rs, uint32_t voff, void* lds) {
  const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
               :: "v"(voff), "s"(la), "s"(rs) : "memory", "m0");
}

// The same copy with the sc1 cache policy (device-coherent: it does not
// hit data that another XCD's L2 may hold stale).
__device__ __forceinline__ void copy16_coherent(v4i rs, uint32_t voff, void* lds) {
  const uint32_t la = (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen sc1 lds"
               :: "v"(voff), "s"(la), "s"(rs) : "memory", "m0");
}

constexpr int kStepCols = 128;  // K columns per pipeline step

template <int WM, int WN, int TM, int TN, int S>
struct Tile {
  static constexpr int kStages = S;  // LDS ring depth (S-1 steps in flight)
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int BM = 32 * TM * WM;
  static constexpr int BN = 32 * TN * WN;
  static constexpr int kBTiles = BN / kTileRows;                // weight tiles per workgroup
  static constexpr int kABytes = BM * kStepCols;                // A bytes per step
  static constexpr int kAInstr = kABytes / 1024;                // 1 KiB per wave copy
  static constexpr int kBInstr = kBTiles / 2;                   // 2 half-tiles per copy
  static constexpr int kAPerWave = kAInstr / kWaves;
  static constexpr int kBPerWave = kBInstr / kWaves;
  static constexpr int kBBytes = kBInstr * 1024;                // B bytes per step
  static constexpr int kStageBytes = kABytes + kBBytes;
  static_assert(kAInstr % kWaves == 0 && kBInstr % kWaves == 0, "copies split evenly");
  static_assert(S >= 2 && S * kStageBytes <= 160 * 1024, "LDS ring must fit 160 KiB");
  static_assert((S - 1) * (kAPerWave + kBPerWave) < 64, "vmcnt range");
};

// vmcnt <= N and lgkmcnt == 0 (gfx9 s_waitcnt encoding): this wave's
// copies older than the last N have landed, and its LDS reads have returned
// -- the compiler may otherwise leave reads of the previous step in flight
// across the next barrier, after which other waves refill that slot.
template <int N>
__device__ __forceinline__ void wait_copies_and_reads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads() (which would
// wait for every outstanding copy).  The s_barrier intrinsic alone does not
// order memory accesses for the compiler, so empty asm statements with a
// memory clobber keep LDS reads and copies on their side of it; they emit
// no instructions.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The K loop of output tile (tm, tn) of one layer over pipeline steps
// [k0, k1) (128 columns each) into acc.  `ring` is the workgroup's LDS ring
// (S stages of kStageBytes).  Every wave leaves with its copies landed and
// its LDS reads returned; other waves may still be reading the ring.
// STREAM_B: copy the weight tiles with the non-temporal policy.
template <int WM, int WN, int TM, int TN, int S, bool LEVEL, bool STREAM_B = false>
__device__ __forceinline__ void tile_mainloop(int8_t* ring, const int8_t* __restrict__ Xq,
                                              int M, int K, int N,
                                              const uint8_t* __restrict__ packed, int tm,
                                              int tn, int k0, int k1, bool level,
                                              v16i (&acc)[TM][TN]) {
  using T = Tile<WM, WN, TM, TN, S>;
  constexpr int kStages = S;
  auto stage_ptr = [&](int slot) -> int8_t* { return ring + slot * T::kStageBytes; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = tm * T::BM;
  const int nt0 = tn * T::kBTiles;  // first 16-row weight tile
  const int ntiles = N / kTileRows;
  const int kblocks = K / kTileCols;

  // Buffer ranges: rows past M and weight tiles past N read as zero.
  const int rows_here = min(T::BM, M - m0);
  const v4i a_rsrc = rsrc_words(Xq + (int64_t)m0 * K, (uint32_t)rows_here * (uint32_t)K);
  const int tiles_here = min(T::kBTiles, ntiles - nt0);
  const v4i b_rsrc = rsrc_words(packed + (int64_t)nt0 * kblocks * kTileBytes,
                                (uint32_t)tiles_here * (uint32_t)kblocks * kTileBytes);

  // Copies of step kh into ring slot `slot`.  A: wave instruction q writes
  // rows 8q..8q+7 (128 bytes each); lane j fills row 8q + j/8, 16-byte slot
  // j%8, loading activation column group (j%8) ^ ((row / 2) & 7) -- the XOR
  // swizzle: the 16 rows that one A-fragment read touches at a time then
  // fall in 16 distinct 16-byte bank groups (a row is 128 bytes, so rows r
  // and r+8 would otherwise share banks).  B: instruction q writes weight tiles 2q, 2q+1 (their half for
  // this step, 512 bytes each).  Steps past the end are issued too, with
  // offsets moved out of the buffer range (so they read zeros without
  // touching memory): a branch around the copies would make the compiler
  // wait for all of them before LDS reads.
  auto dma = [&](int kh, int slot) {
    int8_t* base = stage_ptr(slot);
    const uint32_t past = kh < k1 ? 0u : 0x80000000u;
#pragma unroll
    for (int p = 0; p < T::kAPerWave; ++p) {
      const int q = wave + p * T::kWaves;
      const int r = 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const uint32_t voff =
          ((uint32_t)r * (uint32_t)K + (uint32_t)(kh * kStepCols + c * 16)) | past;
      copy16(a_rsrc, voff, base + q * 1024);
    }
#pragma unroll
    for (int p = 0; p < T::kBPerWave; ++p) {
      const int q = wave + p * T::kWaves;
      const int t = 2 * q + (lane >> 5);
      const uint32_t voff = (uint32_t)((t * kblocks + (kh >> 1)) * kTileBytes +
                                       (kh & 1) * (kTileBytes / 2) + (lane & 31) * 16) |
                            past;
      if constexpr (STREAM_B)
        copy16_nt(b_rsrc, voff, base + T::kABytes + q * 1024);
      else
        copy16(b_rsrc, voff, base + T::kABytes + q * 1024);
    }
  };
  // Copies this wave issues per step.
  constexpr int kMyDma = T::kAPerWave + T::kBPerWave;


#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Fragments of one half step (64-column group p of a step): for MFMA u,
  // A rows of 16 activation columns 64p + 32h + 16u .. +15, and per weight
  // column tile the two packed words of group p (one 8-byte read).
  struct Frag {
    v4i a[2][TM];
    uint2 b[TN];
  };
  const int r32 = lane & 31, h = lane >> 5;
  auto read_frags = [&](int slot, int p, Frag& f) {
    const int8_t* sa = stage_ptr(slot);
    const int8_t* sb = sa + T::kABytes;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = (wn * TN + j) * 32 + r32;  // column within the workgroup tile
      f.b[j] = *reinterpret_cast<const uint2*>(sb + (n >> 4) * (kTileBytes / 2) +
                                               (16 * p + (n & 15)) * 16 + h * 8);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = (wm * TM + i) * 32 + r32;
        const int c = (4 * p + 2 * h + u) ^ ((r >> 1) & 7);
        f.a[u][i] = *reinterpret_cast<const v4i*>(sa + r * kStepCols + c * 16);
      }
  };
  auto compute = [&](const Frag& f) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t w = u == 0 ? f.b[j].x : f.b[j].y;
        const v4i b =
            v4i{(int)codes(w, 0), (int)codes(w, 1), (int)codes(w, 2), (int)codes(w, 3)};
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f.a[u][i], b, acc[i][j], 0, 0, 0);
      }
  };

  // Prologue: copies of steps k0..k0+S-1 into every slot; first half of
  // step k0.
#pragma unroll
  for (int st = 0; st < kStages; ++st) dma(k0 + st, st);
  wait_copies_and_reads<(kStages - 1) * kMyDma>();
  lds_barrier();
  Frag f0, f1;
  read_frags(0, 0, f0);

  // Step kh (its first half in registers, cur): read its second half (nxt)
  // and run the first half's MFMAs.  Then wait until this wave's copies of
  // step kh+1 have landed (at most those of the S-2 later steps
  // outstanding) and its reads of step kh have returned; after the barrier
  // every wave's copies of kh+1 are visible and nobody reads step kh's slot
  // any more, so it takes the copies of step kh+S.  Read the first half of
  // step kh+1 (into cur) and run the second half's MFMAs while those reads
  // are in flight.  (Not __syncthreads(): its workgroup fence would wait for
  // every outstanding copy, emptying the pipeline.)
  //
  // The scheduling barriers keep each half step's fragment reads ahead of
  // the other half's MFMAs: left alone, the compiler moved them next to
  // their first use and waited on them there (2048 x 6912 -> 2560: 34.8-35.4
  // against 36.0-36.2 us; other shapes unchanged).
  auto step = [&](int kh, int slot) {
    read_frags(slot, 1, f1);
    __builtin_amdgcn_sched_barrier(0);
    compute(f0);
    wait_copies_and_reads<(kStages - 2) * kMyDma>();
    lds_barrier();
    dma(kh + kStages, slot);
    read_frags((slot + 1) % kStages, 0, f0);
    __builtin_amdgcn_sched_barrier(0);
    compute(f1);
  };
  // Unrolled so that slot indices are constants, and padded to whole rounds
  // instead of a remainder loop (a second loop makes the compiler shuffle
  // the accumulators every iteration).  Padding steps read zero activations
  // (their copies are out of range) and add nothing.
  //
  // LEVEL: issue is oldest-first, so of the workgroups resident on a CU the
  // first dispatched races ahead and the last one finishes alone, leaving
  // its SIMDs short of waves.  When nothing is queued behind them, each
  // wave steps its priority down 3 -> 0 over the quarters of its K range,
  // which keeps the resident workgroups level.
  const int nrounds = (k1 - k0 + kStages - 1) / kStages;
  if constexpr (LEVEL) if (level) __builtin_amdgcn_s_setprio(3);
  for (int rd = 0; rd < nrounds; ++rd) {
    if constexpr (LEVEL) if (level) {
      if (rd == nrounds / 4) __builtin_amdgcn_s_setprio(2);
      if (rd == nrounds / 2) __builtin_amdgcn_s_setprio(1);
      if (rd == 3 * nrounds / 4) __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int u = 0; u < kStages; ++u) step(k0 + rd * kStages + u, u);
  }
  // No copy of this wave may still be writing LDS when the ring is reused
  // or the workgroup exits.
  wait_copies_and_reads<0>();
  if constexpr (LEVEL) __builtin_amdgcn_s_setprio(0);
}

// Activation scale and row sum of one tile row: thread t < BM holds row
// m0 + t (rows past M, and threads past BM, read zeros through the buffer
// range).  Loaded before the K loop so that the loads' latency hides behind
// it; the epilogue hands them to the lanes that need them through LDS.
struct RowScale {
  float sx;
  int rs;
};

template <int WM, int WN, int TM, int TN, int S>
__device__ __forceinline__ RowScale load_row_scale(const float* __restrict__ x_scale,
                                                   const int32_t* __restrict__ x_rowsum, int M,
                                                   int tm) {
  using T = Tile<WM, WN, TM, TN, S>;
  static_assert(T::kThreads >= T::BM, "one thread per tile row");
  const int m0 = tm * T::BM;
  const uint32_t rows_here = (uint32_t)min(T::BM, M - m0);
  const uint32_t off = (uint32_t)min((int)threadIdx.x, T::BM) * 4u;
  RowScale r;
  r.sx = __uint_as_float(
      __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(x_scale + m0, rows_here * 4u), (int)off, 0, 0));
  r.rs = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(x_rowsum + m0, rows_here * 4u),
                                                   (int)off, 0, 0);
  return r;
}

// Epilogue of tile (tm, tn): Y = ((acc - rowsum) * s_x) * gamma, then the
// optional ReLU^2.  Called by every wave after its K loop.
template <int WM, int WN, int TM, int TN, int S, bool DEBUG, bool GLU>
__device__ __forceinline__ void tile_epilogue(int8_t* ring, const v16i (&acc)[TM][TN],
                                              RowScale own, float gamma, int M, int N,
                                              float* __restrict__ Y, int epi,
                                              int32_t* __restrict__ acc_out, int tm, int tn) {
  using T = Tile<WM, WN, TM, TN, S>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane & 31, h = lane >> 5;
  const int m0 = tm * T::BM;
  const int nt0 = tn * T::kBTiles;
  // Every wave is past its K loop (its copies landed, its ring reads
  // returned): the ring now passes the row scales and sums around.
  lds_barrier();
  float* s_sx = reinterpret_cast<float*>(ring);
  int* s_rs = reinterpret_cast<int*>(ring + T::BM * 4);
  if (tid < T::BM) {
    s_sx[tid] = own.sx;
    s_rs[tid] = own.rs;
  }
  __syncthreads();

  // D layout of a 32x32 int32 MFMA tile: lane holds column (lane % 32) and,
  // in register e, row 8*(e / 4) + 4*(lane / 32) + e % 4.  One store
  // instruction (fixed e) writes two 128-byte row segments.  Buffer stores
  // over the tile's rows drop what falls outside Y without a branch (rows
  // past M lie past the range; columns past N are moved past it): a branch
  // per store made each one cost a few hundred cycles.  No load follows a
  // store here, so the stores never wait for each other.  Y is written once
  // and not read back here: its stores use the non-temporal policy (NT, 2),
  // measured 1-7% faster over the prefill shapes.
  const uint32_t row_bytes = (uint32_t)N * 4u;
  const uint32_t rows_here = (uint32_t)min(T::BM, M - m0);
  // The gated epilogue (interleaved gate+up tiles) writes N/2 columns: lane
  // column c < 8 of each 16-column group holds a gate, its up is column c+8,
  // one DPP row rotation away (row_ror:8 within the 16-lane DPP row).
  const bool glu = GLU && epi == kEpiGlu;  // compiled out of the plain kernels
  const int64_t ny = glu ? N / 2 : N;
  const uint32_t yrow_bytes = (uint32_t)ny * 4u;
  const auto y_r = make_rsrc(Y + (int64_t)m0 * ny, rows_here * yrow_bytes);
  const auto a_r = make_rsrc(acc_out + (int64_t)m0 * N, DEBUG ? rows_here * row_bytes : 0u);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r = (wm * TM + i) * 32 + 8 * g + 4 * h;  // rows r .. r+3 of the tile
      const float4 sx4 = *reinterpret_cast<const float4*>(s_sx + r);
      const int4 rs4 = *reinterpret_cast<const int4*>(s_rs + r);
      const float sxv[4] = {sx4.x, sx4.y, sx4.z, sx4.w};
      const int rsv[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = nt0 * kTileRows + (wn * TN + j) * 32 + r32;
          const int v = acc[i][j][4 * g + q] - rsv[q];
          float y = rescale(v, sxv[q], gamma, epi == kEpiRelu2);
          uint32_t off;
          if (glu) {
            const float up = __int_as_float(dpp<0x128>(__float_as_int(y)));
            y = glu_relu2(y, up);
            const int f = (n >> 4) * 8 + (n & 7);
            off = n < N && (r32 & 8) == 0 ? (uint32_t)(r + q) * yrow_bytes + (uint32_t)f * 4u
                                          : 0x80000000u;
          } else {
            off = n < N ? (uint32_t)(r + q) * yrow_bytes + (uint32_t)n * 4u : 0x80000000u;
          }
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), y_r, (int)off, 0, 2);
          if constexpr (DEBUG) {
            const int64_t col = glu ? glu_source_row(n, N) : n;
            const uint32_t aoff =
                n < N ? (uint32_t)(r + q) * row_bytes + (uint32_t)col * 4u : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, a_r, (int)aoff, 0, 0);
          }
        }
      }
    }
  }
}

// One output tile, whole K: the K loop and the epilogue.
template <int WM, int WN, int TM, int TN, int S, bool DEBUG, bool LEVEL, bool GLU>
__device__ __forceinline__ void gemm_tile(
    int8_t* ring, const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_rowsum, int M, int K, int N,
    const uint8_t* __restrict__ packed, const float* __restrict__ gamma_p,
    float* __restrict__ Y, int epi, int32_t* __restrict__ acc_out, int tm, int tn) {
  const RowScale own = load_row_scale<WM, WN, TM, TN, S>(x_scale, x_rowsum, M, tm);
  const float gamma = *gamma_p;
  v16i acc[TM][TN];
  // Many layers up to 64 tokens (64-row tiles): one tile row per layer, so
  // each weight byte is read once and streams past the caches (7B step at
  // M = 64: 455-464 against 462-479 us, 2B step at M = 64 208-210 against
  // 216-219).  Taller tiles share weight tiles through L2 and keep the
  // default policy (non-temporal: 7B step at M = 512 +4.5%, prefill GEMMs
  // +20%), and so does the one-layer kernel (64 x 4096 -> 22016: 20.2
  // against 16.7 us).
  constexpr bool kStreamB = 32 * TM * WM <= 64;
  tile_mainloop<WM, WN, TM, TN, S, LEVEL, kStreamB>(ring, Xq, M, K, N, packed, tm, tn, 0,
                                                    K / kStepCols, true, acc);
  tile_epilogue<WM, WN, TM, TN, S, DEBUG, GLU>(ring, acc, own, gamma, M, N, Y, epi, acc_out, tm,
                                          tn);
}

// ---- Split tiles: the remainder round, cut along K ----
// When the output tiles do not divide evenly among the compute units, the
// tiles of the last, partial round are not given one workgroup each (most
// compute units would idle while a few run one more tile).  Instead each of
// those R tiles is cut along K into f pieces (f = compute units / R, at
// least two pipeline steps each), one workgroup per piece.  int32 sums are
// exact in any order, so the pieces of a tile combine bit for bit: every
// piece stores its partial sums in its workspace slot and counts itself in
// at the tile's counter; the last one to arrive adds the others' sums to its
// own and runs the epilogue.  Nobody waits for anybody, so the workgroups
// need not be resident together.
struct SkPlan {
  int tiles_dp;  // tiles with one workgroup each (the first tiles_dp tiles)
  int tiles_sk;  // R: the remaining tiles, after them
  int steps;     // S: pipeline steps per tile
  int pieces;    // f: pieces per remaining tile (R * f workgroups; 0: none)
};

constexpr int kSkMaxGroups = 256;      // at most this many pieces in all
constexpr int kSkCounterInts = 1024;   // one counter per remaining tile
constexpr int kSkSlotInts = 128 * 128; // partial sums of one 128x128 tile

// Pipeline steps [k0, k1) of piece `piece` of a tile.
__device__ __forceinline__ int sk_piece_begin(const SkPlan& p, int piece) {
  return piece * p.steps / p.pieces;
}

// Hands this workgroup's piece of remaining tile t over.  Returns true (for
// the whole workgroup) when it was the last piece to arrive; acc then holds
// the tile's whole sums.  Register e = 4q..4q+3 of block (i, j) of thread
// tid sits at int4 index ((i*TN + j)*4 + q)*threads + tid of the slot.  Slot
// stores and loads carry the sc1 cache policy (device-coherent: they do not
// stop at the per-XCD L2s, which are not coherent with each other).  The
// counter is raised only after every wave's stores have completed.  The
// last piece brings the other slots in through LDS (each wave its own 8 KiB
// of the ring), so that all of a slot's loads are in flight at once without
// holding registers.
constexpr int kCoherent = 16;  // cache policy of the slot stores: sc1

template <int WM, int WN, int TM, int TN, int S>
__device__ __forceinline__ bool sk_contribute(int8_t* ring, v16i (&acc)[TM][TN],
                                              const SkPlan& p, int* __restrict__ sk_ws,
                                              int t, int g) {
  using T = Tile<WM, WN, TM, TN, S>;
  static_assert(T::BM * T::BN <= kSkSlotInts, "slot holds one tile");
  constexpr int kChunks = TM * TN * 4;  // 16-byte stores per thread
  constexpr int kHalf = kChunks / 2;
  static_assert(T::kWaves * kHalf * 1024 + 64 <= S * T::kStageBytes, "ring holds the halves");
  int* counters = sk_ws;
  int* slots = sk_ws + kSkCounterInts;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const auto mine = make_rsrc(slots + (int64_t)g * kSkSlotInts, kSkSlotInts * 4u);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u v = {(uint32_t)acc[i][j][4 * q], (uint32_t)acc[i][j][4 * q + 1],
                       (uint32_t)acc[i][j][4 * q + 2], (uint32_t)acc[i][j][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(
            v, mine, ((((i * TN + j) * 4 + q) * T::kThreads) + tid) * 16, 0, kCoherent);
      }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave's stores have completed; the ring is free
  const int g_first = t * p.pieces;
  const int g_last = g_first + p.pieces - 1;
  // Past the waves' 8 KiB regions, so that no wave's copies overwrite it
  // while another wave still reads it.
  int* s_last = reinterpret_cast<int*>(ring + T::kWaves * kHalf * 1024);
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(counters + t, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == g_last - g_first ? 1 : 0;
    // Back to zero for the next launch (nobody else touches it in this one).
    if (last) __hip_atomic_store(counters + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = last;
  }
  __syncthreads();
  if (*s_last == 0) return false;
  int8_t* region = ring + wave * (kHalf * 1024);
  for (int o = g_first; o <= g_last; ++o) {
    if (o == g) continue;
    v4i src = rsrc_words(slots + (int64_t)o * kSkSlotInts, kSkSlotInts * 4u);
#pragma unroll
    for (int w = 0; w < 4; ++w) src[w] = __builtin_amdgcn_readfirstlane(src[w]);  // uniform
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int c = 0; c < kHalf; ++c) {
        const int ch = half * kHalf + c;
        copy16_coherent(src, (uint32_t)((ch * T::kThreads + wave * 64 + lane) * 16),
                        region + c * 1024);
      }
      wait_copies_and_reads<0>();
#pragma unroll
      for (int c = 0; c < kHalf; ++c) {
        const int ch = half * kHalf + c;
        const int blk = ch / 4, q = ch % 4, i = blk / TN, j = blk % TN;
        const v4i v = *reinterpret_cast<const v4i*>(region + c * 1024 + lane * 16);
        acc[i][j][4 * q] += v.x;
        acc[i][j][4 * q + 1] += v.y;
        acc[i][j][4 * q + 2] += v.z;
        acc[i][j][4 * q + 3] += v.w;
      }
      // This wave's reads of its region return before its next copies land
      // there (the adds above consume them; the copy asm is a memory fence
      // for the compiler).
    }
  }
  return true;
}

// Waves per SIMD a configuration is built for: four for 64x64 wave tiles
// in a 2-stage ring (at most 128 registers), two for wider ones (their
// accumulators alone take 128) and for 3-stage rings (60 KiB of LDS: two
// workgroups per CU).
template <int TM, int TN, int S>
constexpr int kWavesPerSimd = TM * TN > 4 || S > 2 ? 2 : 4;

// One layer.  Workgroups below plan.tiles_dp take one output tile each
// (whole K); the tiles_sk * pieces workgroups after them take one piece of
// a remaining tile each (sk_ws: counters, then one slot per piece).  Tiles
// larger than a slot are never cut (the host plans no pieces for them).
template <int WM, int WN, int TM, int TN, int S, bool DEBUG, bool LEVEL, bool GLU>
__global__ __launch_bounds__(64 * WM * WN, (kWavesPerSimd<TM, TN, S>)) void gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ x_rowsum, int M, int K, int N,
    const uint8_t* __restrict__ packed, const float* __restrict__ gamma_p,
    float* __restrict__ Y, int epi, int32_t* __restrict__ acc_out, int tiles_n,
    SkPlan plan, int* __restrict__ sk_ws) {
  using T = Tile<WM, WN, TM, TN, S>;
  __shared__ __align__(1024) int8_t ring[S * T::kStageBytes];
  const int b = blockIdx.x;
  const bool split = b >= plan.tiles_dp;
  int tile, k0 = 0, k1 = plan.steps, g = 0, t = 0;
  if (!split) {
    // Whole tiles: consecutive workgroup ids go to different XCDs; give each
    // XCD a contiguous run of tiles (row-major), so tiles that share
    // activation rows share that XCD's L2.
    const int n = plan.tiles_dp;
    tile = n % 8 == 0 ? (b % 8) * (n / 8) + b / 8 : b;
  } else {
    g = b - plan.tiles_dp;
    t = g / plan.pieces;
    const int piece = g - t * plan.pieces;
    tile = plan.tiles_dp + t;
    k0 = sk_piece_begin(plan, piece);
    k1 = sk_piece_begin(plan, piece + 1);
  }
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const RowScale own = load_row_scale<WM, WN, TM, TN, S>(x_scale, x_rowsum, M, tm);
  const float gamma = *gamma_p;
  v16i acc[TM][TN];
  // Leveled launches run the pieces first (top priority), so the hand-over
  // and epilogue of split tiles overlap the whole tiles' K loops.
  if constexpr (LEVEL) if (split) __builtin_amdgcn_s_setprio(3);
  tile_mainloop<WM, WN, TM, TN, S, LEVEL>(ring, Xq, M, K, N, packed, tm, tn, k0, k1, !split, acc);
  if constexpr (LEVEL) __builtin_amdgcn_s_setprio(0);
  bool whole = !split;
  if constexpr (T::BM * T::BN <= kSkSlotInts)
    if (split) whole = sk_contribute<WM, WN, TM, TN, S>(ring, acc, plan, sk_ws, t, g);
  if (whole)
    tile_epilogue<WM, WN, TM, TN, S, DEBUG, GLU>(ring, acc, own, gamma, M, N, Y, epi, acc_out, tm,
                                            tn);
}

// Many layers (a whole step): a persistent grid over the concatenation of
// every layer's output tiles (each layer row-major over its tm x tn tiles
// with tm fastest, starting at its item_begin), from activations quantized
// beforehand into xq / sx / rs.  Workgroup v takes items v, v + G, v + 2G,
// ...: at any time the grid works on a window of G consecutive items, so
// the tiles in flight share activation row blocks and weight tiles.  Each
// XCD takes a contiguous block of the window (consecutive workgroup ids go
// to different XCDs), so what they share stays in one L2.  Every layer's
// items spread evenly over the workgroups, which balances the cost.
template <int WM, int WN, int TM, int TN, int S, bool GLU>
__global__ __launch_bounds__(64 * WM * WN, (TM * TN > 4 ? 2 : 3)) void group_gemm_kernel(
    const GroupOp* __restrict__ ops, int n_ops, int M, int n_items,
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int* __restrict__ rs) {
  using T = Tile<WM, WN, TM, TN, S>;
  __shared__ __align__(1024) int8_t ring[S * T::kStageBytes];
  const int b = blockIdx.x, G = gridDim.x;
  const int v = G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
  const int tiles_m = (M + T::BM - 1) / T::BM;
  int op = 0;
  bool first = true;
  for (int item = v; item < n_items; item += G) {
    while (op + 1 < n_ops && ops[op + 1].item_begin <= item) ++op;
    const GroupOp o = ops[op];
    const int local = item - o.item_begin;
    const int tn = local / tiles_m, tm = local - tn * tiles_m;  // m fastest: weights reused
    if (!first) lds_barrier();  // every wave is past the previous tile's LDS reads
    first = false;
    gemm_tile<WM, WN, TM, TN, S, false, true, GLU>(ring, xq + o.xq_off, sx + op * M, rs + op * M, M,
                                              o.K, o.N, o.packed, o.gamma, o.Y, o.epi, nullptr,
                                              tm, tn);
  }
}

// Compute units of the current device (cached per device).  Callers on any
// thread may race to fill an entry: they compute the same value, and the
// atomics make the race well defined.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kSkMaxGroups;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      return kSkMaxGroups;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Workgroups of gemm_kernel<WM,WN,TM,TN,S> that fit on one CU at once
// (cached per configuration).
template <int WM, int WN, int TM, int TN, int S>
int resident_per_cu() {
  static std::atomic<int> cached{0};  // same idempotent race as device_cus
  int v = cached.load(std::memory_order_relaxed);
  if (v == 0) {
    int blocks = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &blocks, reinterpret_cast<const void*>(&gemm_kernel<WM, WN, TM, TN, S, false, false, false>),
        Tile<WM, WN, TM, TN, S>::kThreads, 0);
    v = (e == hipSuccess && blocks > 0) ? blocks : 4;
    cached.store(v, std::memory_order_relaxed);
  }
  return v;
}

// Output tiles of BM x BN for one layer, and which of them are cut along K
// (split: a workspace was given and a slot holds such a tile).
template <int BM, int BN>
SkPlan plan_tiles(int64_t M, int64_t K, int64_t N, bool split) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int total = tiles_m * tiles_n;
  SkPlan plan{total, 0, (int)(K / kStepCols), 0};
  if (split && BM * BN <= kSkSlotInts) {
    const int P = std::min(device_cus(), kSkMaxGroups);
    const int R = total % P;
    // Pieces per remaining tile: fill the compute units, at least two
    // steps a piece.
    const int f = R > 0 ? std::min(P / R, plan.steps / 2) : 0;
    if (f >= 2) {
      plan.tiles_dp = total - R;
      plan.tiles_sk = R;
      plan.pieces = f;
    }
  }
  return plan;
}

int plan_grid(const SkPlan& p) { return p.tiles_dp + p.tiles_sk * p.pieces; }

template <int WM, int WN, int TM, int TN, int S>
hipError_t launch_cfg(const int8_t* Xq, const float* sx, const int32_t* rs, int64_t M,
                      int64_t K, int64_t N, const uint8_t* packed, const float* gamma, float* Y,
                      int epi, int32_t* acc_out, int* sk_ws, hipStream_t s) {
  using T = Tile<WM, WN, TM, TN, S>;
  const int tiles_n = (int)((N + T::BN - 1) / T::BN);
  const SkPlan plan = plan_tiles<T::BM, T::BN>(M, K, N, sk_ws != nullptr);
  const int grid = plan_grid(plan);
  // Level the whole-tile workgroups (priority steps) when the whole grid is
  // resident at once: with rounds queued behind them, staggered finishes
  // overlap one workgroup's epilogue with the next one's start.  With split
  // pieces, only when at least two whole tiles per CU remain once the
  // pieces are done; with one (2048 x 6912 -> 2560: one tile and one piece
  // per CU) that tile would finish alone, and oldest-first issue measured
  // 8% faster.
  const int cus = device_cus();
  const bool level = grid <= cus * resident_per_cu<WM, WN, TM, TN, S>() &&
                     (plan.pieces == 0 || plan.tiles_dp >= 2 * cus);
  const bool glu = epi == kEpiGlu;
#define BL_GEMM_LAUNCH(DBG, LVL, GL)                                                          \
  hipLaunchKernelGGL((gemm_kernel<WM, WN, TM, TN, S, DBG, LVL, GL>), dim3(grid),             \
                     dim3(T::kThreads), 0, s, Xq, sx, rs, (int)M, (int)K, (int)N, packed,     \
                     gamma, Y, epi, acc_out, tiles_n, plan, sk_ws)
  if (acc_out) {
    if (glu) BL_GEMM_LAUNCH(true, false, true);
    else BL_GEMM_LAUNCH(true, false, false);
  } else if (level) {
    if (glu) BL_GEMM_LAUNCH(false, true, true);
    else BL_GEMM_LAUNCH(false, true, false);
  } else {
    if (glu) BL_GEMM_LAUNCH(false, false, true);
    else BL_GEMM_LAUNCH(false, false, false);
  }
#undef BL_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Tile choice, measured on MI355X (graph-timed launches, several runs each).
//
// One layer above 64 tokens: 128x128 tiles (4 waves of 64x64, four
// workgroups per CU), with the last partial round cut along K.  These beat
// 64x128 and 64x256 tiles, deeper rings with shorter steps, and two-wave
// workgroups.  The exception: when 128x256 tiles (4 waves of 64x128, two
// workgroups per CU) make one round that fills at least three quarters of
// the resident slots (so every CU joins and few finish early with one tile),
// they are used instead.  A 64x128 wave tile reads half the activation
// bytes from LDS per multiply, and the workgroup copies 24 KiB per step for
// 128 multiplies against 20 KiB for 64: 2048 x 2560 -> 6912 (432 tiles of
// 512 slots) 33.9-35.1 us against 36.9-38.9 us.  With fewer tiles the CUs
// left with one tile idle half the launch, and the 128x128 grid's finer
// balance wins: 324 tiles (1536 x 2560 -> 6912) 29.0-30.2 against
// 31.7-37.5 us, 344 (512 x 4096 -> 22016, 1024 x 4096 -> 11008) 42.5-46.6
// against 45.2-50.7 us; 264 (1024 x 2560 -> 8448) tied.  Fewer tiles than
// CUs (2048 x 6912 -> 2560): 46 against 38 us; 1.7 rounds
// (4096 x 2560 -> 6912): 69.6 against 67.1 us.
// They are never cut along K (a slot holds one 128x128 tile).  When the
// 128x128 grid (pieces included) needs no more than two workgroups per CU,
// a 3-stage ring (60 KiB, two steps of copies in flight) costs no
// residency and gains: 2048 x 6912 -> 2560 (256 tiles and 64 tiles in 4
// pieces) 36.9-37.2 against 38.0-38.4 us, 512 x 11008 -> 4096 28.9-29.3
// against 30.4-31.2 us; with rounds queued it loses (4096 x 2560 -> 6912:
// 73.6 against 66.3 us).
//
// One layer up to 64 tokens: 64-row tiles avoid multiplying 64 empty rows,
// 64x128 (4 waves of 32x64).
//
// Many layers (a persistent grid that has work for every slot): up to 64
// tokens, 64x256 tiles, which halve the activation bytes copied per multiply
// against 64x128 (7B step at M = 64: 547 against 611 us).  Their four waves
// sit side by side, 64x64 each, so every unpacked weight operand feeds two
// MFMAs (as 32x128 waves, one): 508-513 against 557-563 us, and the 2B step
// at M = 64 248 against 250 us.  (4 waves of 64x128 in 64x512 tiles: 538
// and 230 us.)  A 3-stage ring (48 KiB, three workgroups per CU) then
// gains: 519-524 against 534-550 us, 2B step 225 against 251 us.  Above 64
// tokens, the 128x256 tiles: 7B step at M = 512 3157-3195 against 3382 us
// with 128x128 tiles.
using WideCfg = Tile<2, 2, 2, 4, 2>;
using GroupSmallCfg = Tile<1, 4, 2, 2, 3>;
constexpr int kSmallM = 64;

int bl_group_gemm_tiles(int M, int N) {
  const int bm = M <= kSmallM ? GroupSmallCfg::BM : WideCfg::BM;
  const int bn = M <= kSmallM ? GroupSmallCfg::BN : WideCfg::BN;
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

int bl_group_gemm_blocks_per_cu(int M) {
  int blocks = 0;
  const void* k = M <= kSmallM
                      ? reinterpret_cast<const void*>(&group_gemm_kernel<1, 4, 2, 2, 3, false>)
                      : reinterpret_cast<const void*>(&group_gemm_kernel<2, 2, 2, 4, 2, false>);
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, 256, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

hipError_t bl_launch_group_gemm(const GroupOp* ops, int n_ops, int M, int n_items, int G,
                                const int8_t* xq, const float* sx, const int* rs, bool glu,
                                hipStream_t s) {
#define BL_GROUP_GEMM(WM, WN, TM, TN, S, GL)                                                  \
  hipLaunchKernelGGL((group_gemm_kernel<WM, WN, TM, TN, S, GL>), dim3(G), dim3(64 * WM * WN), \
                     0, s, ops, n_ops, M, n_items, xq, sx, rs)
  if (M <= kSmallM) {
    if (glu) BL_GROUP_GEMM(1, 4, 2, 2, 3, true);
    else BL_GROUP_GEMM(1, 4, 2, 2, 3, false);
  } else {
    if (glu) BL_GROUP_GEMM(2, 2, 2, 4, 2, true);
    else BL_GROUP_GEMM(2, 2, 2, 4, 2, false);
  }
#undef BL_GROUP_GEMM
  return hipGetLastError();
}

size_t bl_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  (void)M, (void)K, (void)N;
  return (size_t)(kSkCounterInts + (size_t)kSkMaxGroups * kSkSlotInts) * sizeof(int);
}

size_t bl_gemm_counter_bytes() { return kSkCounterInts * sizeof(int); }

hipError_t bl_launch_gemm_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, int epi, int32_t* acc_out,
                            void* gemm_ws, hipStream_t s) {
  if (M <= kSmallM)
    return launch_cfg<2, 2, 1, 2, 2>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y, epi,
                                     acc_out, static_cast<int*>(gemm_ws), s);
  const int64_t wide_tiles = ((M + WideCfg::BM - 1) / WideCfg::BM) *
                             ((N + WideCfg::BN - 1) / WideCfg::BN);
  const int cus = device_cus();
  const int64_t wide_slots = (int64_t)cus * resident_per_cu<2, 2, 2, 4, 2>();
  if (wide_tiles > cus && wide_tiles <= wide_slots && 4 * wide_tiles >= 3 * wide_slots)
    return launch_cfg<2, 2, 2, 4, 2>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y, epi,
                                     acc_out, static_cast<int*>(gemm_ws), s);
  if (plan_grid(plan_tiles<128, 128>(M, K, N, gemm_ws != nullptr)) <= 2 * cus)
    return launch_cfg<2, 2, 2, 2, 3>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y, epi,
                                     acc_out, static_cast<int*>(gemm_ws), s);
  return launch_cfg<2, 2, 2, 2, 2>(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y, epi,
                                   acc_out, static_cast<int*>(gemm_ws), s);
}
