// Device descriptor of one layer in a grouped decode forward (80 bytes),
// shared by the ABI layer (which fills the table) and the kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct GroupOp {
  const void* X;           // [M][K] activations (float or bf16)
  const uint8_t* packed;   // packed ternary weights, [N/16][K/256] tiles of 1 KiB
  const float* gamma;      // gamma_c (one float)
  float* Y;                // [M][N] output
  const float* norm_gain;  // subln gain [K] before the quantization, or null
  int64_t xq_off;          // byte offset of this layer's int8 [M][K] in the workspace
  int32_t K, N;
  int32_t dtype, epi;      // epi: kEpiNone, kEpiRelu2 or kEpiGlu (Y then [M][N/2])
  int32_t item_begin;      // index of this layer's first 16-row tile in the flat list
  float norm_eps;          // subln epsilon
  int32_t pad[2];
};
static_assert(sizeof(GroupOp) == 80, "GroupOp must stay 80 bytes");

// A unit of grouped work: tiles first..end-1 (indices into the concatenation
// of every layer's 16-row tiles) of layer op.
struct GroupUnit {
  int32_t first, end, op, pad;
};
// A unit holds about kGroupUnitBlocks 1 KiB weight blocks (16 rows x 256
// columns each), at most one segment: 32 tiles at K = 2560, 12 at K = 6912,
// 20 at K = 4096.  Measured on MI355X over 80..640: smaller units cost more
// set-ups (a new layer's quantization, a pipeline restart), larger ones a
// longer tail (2B step at M = 1: 93 us at 320, 98 at 160, 100 at 80).
constexpr int kGroupUnitBlocks = 320;
// Tiles whose outputs a workgroup holds in LDS at once (one segment).
constexpr int kGroupSegTiles = 32;
// Share of the work (by bytes) in the static ranges, in percent, when the
// workgroups quantize activations themselves (a new layer costs a
// quantization) and when they copy pre-quantized rows (a new layer costs a
// copy of M rows); measured on MI355X over 2B and 7B decode steps.
constexpr int kGroupStaticPercentInline = 75;
constexpr int kGroupStaticPercentPreq = 95;

// Largest K of a grouped layer and largest token count.  Up to
// kGroupInlineQuantMaxM tokens each workgroup quantizes the activations of
// the layer it starts on itself (one launch); above, a separate launch
// quantizes them once into the workspace.
constexpr int kGroupMaxK = 12288;
constexpr int kGroupMaxM = 16;
constexpr int kGroupInlineQuantMaxM = 4;

// Whether the group needs the quantization launch and workspace.
bool bl_group_prequantizes(int M);

// LDS available to one workgroup.
constexpr size_t kGroupMaxLds = 160 * 1024;

// Dynamic LDS bytes of the grouped kernel for M tokens and largest K.
size_t bl_group_lds_bytes(int M, int max_k);

// Chooses the workgroup size (256 or 512 threads) and reports how many
// workgroups fit on one compute unit; also allows the kernel the dynamic
// LDS it needs.  norm: some layer has a subln gain.
hipError_t bl_group_plan(int M, int max_k, bool norm, int* threads, int* per_cu);

// Grouped forward: G workgroups of `threads` threads; workgroup g first runs
// tiles wg_begin[g] .. wg_begin[g+1]-1, then takes the n_units units from the
// queue (two ints, zero on entry and left zero); max_k the largest K.  xq,
// sx, rs: the quantized activations, scales and row sums (used when
// bl_group_prequantizes(M)); norm as for bl_group_plan.
hipError_t bl_launch_group(const GroupOp* ops, int n_ops, int M, const int* wg_begin,
                           const GroupUnit* units, int n_units, int* queue, int G, int max_k,
                           int threads, bool norm, int8_t* xq, float* sx, int* rs,
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
// The quantization launch of the grouped forward (one workgroup per layer
// and token) into xq / sx / rs at each layer's xq_off; max_k the largest K.
hipError_t bl_launch_group_quant(const GroupOp* ops, int n_ops, int M, int max_k, int8_t* xq,
                                 float* sx, int* rs, hipStream_t s);
