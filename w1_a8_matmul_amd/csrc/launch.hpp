// Host-side declarations of the library's launchers and planning helpers,
// shared by the ABI layer and the .hip files that define them.  Kept apart
// from the device headers, so that the kernels' sources do not change when a
// launcher is added.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"
#include "group.hpp"

// Host-side launchers (defined in the .hip files).  All return hipError_t of
// the launch; shapes were validated by the ABI layer.
hipError_t bl_launch_absmean_rows(const float* W, int64_t N, int64_t K, double* row_sum,
                                  hipStream_t s);
hipError_t bl_launch_absmean_final(const double* row_sum, int64_t N, int64_t K,
                                   float* gamma, hipStream_t s);
hipError_t bl_launch_quant_pack(const float* W, int64_t N, int64_t K, const float* gamma,
                                uint8_t* packed, hipStream_t s,
                                bool glu = false);
hipError_t bl_launch_pack(const int8_t* Wq, int64_t N, int64_t K, uint8_t* packed,
                          hipStream_t s);
// The base-3 layout: K padded to a multiple of 320 (bl_b3_padded_k).
inline int64_t bl_b3_padded_k(int64_t K) { return (K + bl::kB3TileCols - 1) / bl::kB3TileCols * bl::kB3TileCols; }
hipError_t bl_launch_quant_pack_b3(const float* W, int64_t N, int64_t K, const float* gamma,
                                   uint8_t* packed, hipStream_t s, bool glu);
hipError_t bl_launch_pack_b3(const int8_t* Wq, int64_t N, int64_t K, uint8_t* packed,
                             hipStream_t s);
hipError_t bl_launch_unpack_b3(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wq,
                               hipStream_t s);
hipError_t bl_launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wq,
                            hipStream_t s);
// Per-token activation quantization; also zeroes n_zero ints at `zero`
// (may be null) for the launch that follows.  norm_gain (float [K], 16-byte
// aligned) selects subln first (RMSNorm with that gain and norm_eps).
hipError_t bl_launch_quant_acts(const void* X, int dtype, int64_t M, int64_t K, int8_t* Xq,
                                float* x_scale, int32_t* x_rowsum, int* zero, int n_zero,
                                hipStream_t s, const float* norm_gain = nullptr,
                                float norm_eps = 0.0f);
// Small-M fused forward (activation quantization inside the kernel).
bool bl_gemv_supports(int64_t M, int64_t K);
hipError_t bl_launch_gemv(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                          const uint8_t* packed, const float* gamma, float* Y, int epi,
                          int8_t* xq_out, float* xscale_out, int32_t* acc_out,
                          hipStream_t s, const float* norm_gain = nullptr,
                          float norm_eps = 0.0f);
// Lookup-table GEMV for one token (K % 256 == 0, K <= kLutMaxK): int16
// tables of column-pair sums in LDS indexed by 4-bit fields of the packed
// codes; same outputs as bl_launch_gemv at M = 1.
constexpr int64_t kLutMaxK = 8192;
size_t bl_lut_lds_bytes(int64_t K);
size_t bl_lut_max_lds_bytes();
hipError_t bl_launch_lut_gemv(const void* X, int dtype, int64_t K, int64_t N,
                              const uint8_t* packed, const float* gamma, float* Y, int epi,
                              int8_t* xq_out, float* xscale_out, int32_t* acc_out,
                              hipStream_t s);
// The small-M forward from pre-quantized int8 rows (M <= 4, K as
// bl_gemv_supports): the rows are copied into LDS instead of quantized.
hipError_t bl_launch_gemv_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, int epi, int32_t* acc_out,
                            hipStream_t s);
// The small-M forward of a fused gate+up matrix whose gated output h [M][N/2]
// also leaves quantized (hq, h_scale, h_rowsum) by the last workgroup;
// counter: one int, zero on entry, left zero.
hipError_t bl_launch_gemv_glu_quant(const void* X, int dtype, int64_t M, int64_t K, int64_t N,
                                    const uint8_t* packed, const float* gamma, float* H,
                                    int8_t* hq, float* h_scale, int32_t* h_rowsum,
                                    int* counter, hipStream_t s);
// Forward from quantized activations on the int8 MFMA units.  gemm_ws
// (bl_gemm_workspace_bytes, its first bl_gemm_counter_bytes zero on entry
// and left zero) lets the last, partial round of tiles be shared along K;
// null runs one workgroup per tile.
size_t bl_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);
size_t bl_gemm_counter_bytes();
hipError_t bl_launch_gemm_q(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum,
                            int64_t M, int64_t K, int64_t N, const uint8_t* packed,
                            const float* gamma, float* Y, int epi, int32_t* acc_out,
                            void* gemm_ws, hipStream_t s);

// The decode FFN (M <= 4) in one persistent launch: up projection with the
// squared ReLU (glu: the gated one of a fused gate+up matrix), h [M][F]
// (F = n_up, or n_up / 2 with glu), down projection [n_down][F] into Y.  ws
// holds bl_chain_workspace_bytes(n_up) bytes (counters and one flag per up
// tile), zero before its first use; its third int is an error flag, set if a
// wait gave up.  K and F are multiples of 256 up to 12288.
size_t bl_chain_workspace_bytes(int64_t n_up);
hipError_t bl_launch_ffn_chain(const void* X, int dtype, int64_t M, int64_t K, int64_t n_up,
                               const uint8_t* packed_up, const float* gamma_up, bool glu,
                               float* H, int64_t n_down, const uint8_t* packed_down,
                               const float* gamma_down, float* Y, void* ws, hipStream_t s);

// Grouped forward: the host's split of the work (constants the kernel does
// not see).
// A unit holds about kGroupUnitBlocks 1 KiB weight blocks (16 rows x 256
// columns each), at most one segment: 32 tiles at K = 2560, 12 at K = 6912,
// 20 at K = 4096.  Measured on MI355X over 80..640: smaller units cost more
// set-ups (a new layer's quantization, a pipeline restart), larger ones a
// longer tail (2B step at M = 1: 93 us at 320, 98 at 160, 100 at 80).
constexpr int kGroupUnitBlocks = 320;
// Share of the work (by bytes) in the static ranges, in percent, when the
// workgroups quantize activations themselves (a new layer costs a
// quantization) and when they copy pre-quantized rows (a new layer costs a
// copy of M rows); measured on MI355X over 2B and 7B decode steps.  From
// kGroupPreqWideM tokens on, the copies and output stores of a unit are long
// enough that a larger shared part balances better: 2B step at 8 tokens,
// 116.8-117.4 us at 85% against 121.8-123.4 at 95% (two runs each on one
// box; at 4 and 16 tokens the two were within the spread of runs).
constexpr int kGroupStaticPercentInline = 75;
constexpr int kGroupStaticPercentPreq = 95;
constexpr int kGroupStaticPercentPreqWide = 85;
constexpr int kGroupPreqWideM = 8;

// Whether the group needs the quantization launch and workspace.
bool bl_group_prequantizes(int M);

// The quantization launch of the grouped forward (one workgroup per layer
// and token) into xq / sx / rs at each layer's xq_off; max_k the largest K,
// norm whether some layer has a subln gain.
hipError_t bl_launch_group_quant(const GroupOp* ops, int n_ops, int M, int max_k, bool norm,
                                 int8_t* xq, float* sx, int* rs, hipStream_t s);

// Dynamic LDS bytes of the grouped kernel for M tokens and largest K.
size_t bl_group_lds_bytes(int M, int max_k);

// Chooses the workgroup size (256 or 512 threads) and reports how many
// workgroups fit on one compute unit; also allows the kernel the dynamic
// LDS it needs.  norm: some layer has a subln gain.
hipError_t bl_group_plan(int M, int max_k, bool norm, bool b3, int* threads, int* per_cu);

// Grouped forward (b3: every layer's weights in the base-3 layout, and max_k
// the largest padded K): G workgroups of `threads` threads; workgroup g first runs
// tiles wg_begin[g] .. wg_begin[g+1]-1, then takes the n_units units from the
// queue (two ints, zero on entry and left zero); max_k the largest K.  xq,
// sx, rs: the quantized activations, scales and row sums (used when
// bl_group_prequantizes(M)); norm as for bl_group_plan.
hipError_t bl_launch_group(const GroupOp* ops, int n_ops, int M, const int* wg_begin,
                           const GroupUnit* units, int n_units, int* queue, int G, int max_k,
                           int threads, bool norm, bool b3, int8_t* xq, float* sx, int* rs,
                           hipStream_t s);

// Above kGroupMaxM tokens a group runs as one persistent tiled int8 GEMM over
// the output tiles of all its layers (activations quantized beforehand).
// Output tiles of one layer at M tokens; workgroups per compute unit.
int bl_group_gemm_tiles(int M, int N);
int bl_group_gemm_blocks_per_cu(int M);
// n_items: output tiles over all layers; G workgroups take them strided.
hipError_t bl_launch_group_gemm(const GroupOp* ops, int n_ops, int M, int n_items, int G,
                                const int8_t* xq, const float* sx, const int* rs, bool glu,
                                hipStream_t s);
