// Device descriptor of one layer in a grouped decode forward (64 bytes),
// shared by the ABI layer (which fills the table) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct GroupOp {
  const void* X;          // [M][K] activations (float or bf16)
  const uint8_t* packed;  // packed ternary weights, [N/16][K/256] tiles of 1 KiB
  const float* gamma;     // gamma_c (one float)
  float* Y;               // [M][N] output
  int64_t xq_off;         // byte offset of this layer's int8 [M][K] in the workspace
  int32_t K, N;
  int32_t dtype, relu2;
  int32_t item_begin;     // index of this layer's first 16-row tile in the flat list
  int32_t chunk;          // column blocks per streamed chunk (1..12)
};
static_assert(sizeof(GroupOp) == 64, "GroupOp must stay 64 bytes");

// Grouped forward: quantize every layer's activations, then stream all tiles.
// wg_begin[g]..wg_begin[g+1] is workgroup g's tile range; G workgroups.
hipError_t bl_launch_group(const GroupOp* ops, int n_ops, int M, const int* wg_begin, int G,
                           int max_k, int8_t* xq, float* sx, int32_t* rs, hipStream_t s);
