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
// Tiles whose outputs a workgroup holds in LDS at once (one segment).
constexpr int kGroupSegTiles = 32;

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
