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
  int32_t fmt;             // weight layout: 0 two-bit codes, 1 base-3 (kernels take it as a template)
  int32_t pad;
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
// quantizes them once into the workspace.  Measured on MI355X (2B step, one
// box, alternating runs): inline 102.8 against 107.2 us at two tokens,
// 107.6-110.5 against 110.3-111.3 at three, but 114.5-116.1 against
// 112.0-112.1 at four, where a new layer's four rows cost about three
// memory round trips inline and one copy after the quantization launch.
constexpr int kGroupMaxK = 12288;
constexpr int kGroupMaxM = 16;
constexpr int kGroupInlineQuantMaxM = 3;

// LDS available to one workgroup.
constexpr size_t kGroupMaxLds = 160 * 1024;
