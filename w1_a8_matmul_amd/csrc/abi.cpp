// C ABI of the BitLinear library: argument checks, path choice by M, and
// error reporting.  Declared in include/bitlinear.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <new>
#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/bitlinear.h"
#include "common.hpp"
#include "group.hpp"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

bitlinear_status fail(bitlinear_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

bitlinear_status ok() {
  g_last_error[0] = '\0';
  return BITLINEAR_OK;
}

bitlinear_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// |acc| <= 127 * K must fit int32, and the prefill kernel's buffer ranges
// (128 rows of K bytes, with bit 31 of an offset meaning "past the end")
// must stay below 2^31: K <= 2^23.
constexpr int64_t kMaxK = 8388608;
// Largest N: 128 output rows of float32 stay addressable by one 32-bit buffer
// range (the GEMM epilogue's branch-free stores).
constexpr int64_t kMaxN = 4194304;

bitlinear_status check_nk(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return fail(BITLINEAR_ERR_SHAPE, "N=%lld K=%lld must be >= 1", (long long)N, (long long)K);
  if (N % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "N=%lld is not a multiple of 16", (long long)N);
  if (K % 256 != 0) return fail(BITLINEAR_ERR_SHAPE, "K=%lld is not a multiple of 256", (long long)K);
  if (K > kMaxK) return fail(BITLINEAR_ERR_SHAPE, "K=%lld exceeds %lld", (long long)K, (long long)kMaxK);
  if (N > kMaxN) return fail(BITLINEAR_ERR_SHAPE, "N=%lld exceeds %lld", (long long)N, (long long)kMaxN);
  return BITLINEAR_OK;
}

// Shapes of the base-3 layout: N % 16 == 0, K % 16 == 0 (K is padded to a
// multiple of 320 inside the layout).
bitlinear_status check_nk_b3(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return fail(BITLINEAR_ERR_SHAPE, "N=%lld K=%lld must be >= 1", (long long)N, (long long)K);
  if (N % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "N=%lld is not a multiple of 16", (long long)N);
  if (K % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "K=%lld is not a multiple of 16", (long long)K);
  if (K > kMaxK) return fail(BITLINEAR_ERR_SHAPE, "K=%lld exceeds %lld", (long long)K, (long long)kMaxK);
  if (N > kMaxN) return fail(BITLINEAR_ERR_SHAPE, "N=%lld exceeds %lld", (long long)N, (long long)kMaxN);
  return BITLINEAR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool is_b3(const bitlinear_group_op& o) { return o.format == BITLINEAR_FMT_B3; }

// 1 KiB weight blocks per 16-row tile of a layer (its cost unit), and the K
// its kernel holds activations for (padded to 320 for the base-3 layout).
int64_t op_kblocks(const bitlinear_group_op& o) {
  return is_b3(o) ? bl_b3_padded_k(o.K) / 320 : o.K / 256;
}
int64_t op_lds_k(const bitlinear_group_op& o) { return is_b3(o) ? bl_b3_padded_k(o.K) : o.K; }

// Workspace of the large-M path: int8 activations, scales, row sums.
// Forward workspace above the fused small-M path: quantized activations,
// scales and row sums, then the GEMM's own workspace.
size_t q_workspace(int64_t M, int64_t K) {
  return align256((size_t)M * (size_t)K) + 2 * align256((size_t)M * 4);
}
size_t forward_workspace(int64_t M, int64_t K, int64_t N) {
  return q_workspace(M, K) + align256(bl_gemm_workspace_bytes(M, K, N));
}

// Grouped forward: device workspace layout (layer table, work units and
// their queue for the skinny kernel, quantized activations).
constexpr int kGroupMaxWG = 2048;

struct GroupLayout {
  size_t table, wg_begin, units, queue, xq, sx, rs, total;
  int64_t split;    // first tile of the shared (queued) part
  int64_t n_units;  // units of the shared part
};

// The skinny kernel's split of the tiles (in layer order, a tile costing
// K/256 blocks) into the static part -- the first kGroupStaticPercent* of
// the cost -- and the shared part, cut into runs of about kGroupUnitBlocks
// weight blocks of one layer.  Calls f(op, first, end) for each unit.
template <typename F>
void group_split(const bitlinear_group_op* ops, int n_ops, int64_t M, int64_t* split,
                 int64_t* n_units, F f) {
  const int64_t pct = !bl_group_prequantizes((int)M) ? kGroupStaticPercentInline
                      : M >= kGroupPreqWideM            ? kGroupStaticPercentPreqWide
                                                        : kGroupStaticPercentPreq;
  int64_t total = 0;
  for (int i = 0; i < n_ops; ++i) total += (ops[i].N / 16) * op_kblocks(ops[i]);
  int64_t cost = 0, item = 0, s = -1, n = 0;
  for (int i = 0; i < n_ops; ++i) {
    const int64_t tiles = ops[i].N / 16, kb = op_kblocks(ops[i]);
    int64_t t = 0;
    if (s < 0) {
      // tiles of this layer still inside the static part
      while (t < tiles && (cost + kb) * 100 <= total * pct) {
        cost += kb;
        ++t;
      }
      if (t == tiles) {
        item += tiles;
        continue;
      }
      s = item + t;
    }
    const int64_t per_unit =
        std::min<int64_t>(kGroupSegTiles, std::max<int64_t>(1, (kGroupUnitBlocks + kb / 2) / kb));
    for (; t < tiles; t += per_unit, ++n) f(i, item + t, item + std::min(t + per_unit, tiles));
    item += tiles;
  }
  *split = s < 0 ? item : s;
  *n_units = n;
}

// The quantized activations, scales and row sums exist only for token
// counts whose activations are quantized by a launch of their own.
GroupLayout group_layout(const bitlinear_group_op* ops, int n_ops, int64_t M) {
  GroupLayout L;
  size_t off = 0;
  L.table = off;
  off += align256((size_t)n_ops * sizeof(GroupOp));
  L.wg_begin = off;
  off += align256((size_t)(kGroupMaxWG + 1) * sizeof(int));
  L.split = 0;
  L.n_units = 0;
  if (M <= kGroupMaxM)
    group_split(ops, n_ops, M, &L.split, &L.n_units, [](int, int64_t, int64_t) {});
  L.units = off;
  off += align256((size_t)L.n_units * sizeof(GroupUnit));
  L.queue = off;
  off += 256;
  L.xq = L.sx = L.rs = off;
  if (bl_group_prequantizes((int)M)) {
    for (int i = 0; i < n_ops; ++i) off += align256((size_t)M * (size_t)ops[i].K);
    L.sx = off;
    off += align256((size_t)n_ops * (size_t)M * sizeof(float));
    L.rs = off;
    off += align256((size_t)n_ops * (size_t)M * sizeof(int));
  }
  L.total = off;
  return L;
}

bool valid_epi(int epi) {
  return epi == BITLINEAR_EPI_NONE || epi == BITLINEAR_EPI_RELU2 || epi == BITLINEAR_EPI_RELU2_GLU;
}

// subln arguments: the gain is optional (NULL: none); when given it must be
// 16-byte aligned device memory and the epsilon finite and non-negative.
bitlinear_status check_norm(const float* norm_gain, float norm_eps) {
  if (!norm_gain) return BITLINEAR_OK;
  if (!aligned16(norm_gain)) return fail(BITLINEAR_ERR_ALIGN, "norm_gain must be 16-byte aligned");
  if (!(norm_eps >= 0.0f) || norm_eps > 3.0e38f)
    return fail(BITLINEAR_ERR_ARG, "norm_eps must be finite and >= 0");
  return BITLINEAR_OK;
}

bitlinear_status check_group(const bitlinear_group_op* ops, int n_ops, int64_t M) {
  if (!ops) return fail(BITLINEAR_ERR_NULL, "ops is required");
  if (n_ops < 1 || n_ops > 65536) return fail(BITLINEAR_ERR_ARG, "n_ops=%d out of range", n_ops);
  if (M < 1 || M > 65536)
    return fail(BITLINEAR_ERR_SHAPE, "grouped forward needs 1 <= M <= 65536, got %lld", (long long)M);
  const bool skinny = M <= kGroupMaxM;
  int64_t items = 0;
  for (int i = 0; i < n_ops; ++i) {
    const bitlinear_group_op& o = ops[i];
    if (o.dtype != BITLINEAR_F32 && o.dtype != BITLINEAR_BF16)
      return fail(BITLINEAR_ERR_DTYPE, "op %d: unknown dtype %d", i, (int)o.dtype);
    if (!valid_epi(o.epi))
      return fail(BITLINEAR_ERR_ARG, "op %d: unknown epilogue %d", i, (int)o.epi);
    if (o.format != BITLINEAR_FMT_2BIT && o.format != BITLINEAR_FMT_B3)
      return fail(BITLINEAR_ERR_ARG, "op %d: unknown weight format %d", i, (int)o.format);
    if (o.format != ops[0].format)
      return fail(BITLINEAR_ERR_ARG, "op %d: every layer of a group needs the same weight format",
                  i);
    if (is_b3(o) && !skinny)
      return fail(BITLINEAR_ERR_SHAPE, "op %d: base-3 weights need M <= %d, got %lld", i,
                  kGroupMaxM, (long long)M);
    bitlinear_status st = is_b3(o) ? check_nk_b3(o.N, o.K) : check_nk(o.N, o.K);
    if (st != BITLINEAR_OK) return st;
    if (skinny && op_lds_k(o) > kGroupMaxK)
      return fail(BITLINEAR_ERR_SHAPE, "op %d: K=%lld exceeds %d (M <= %d)", i, (long long)o.K,
                  kGroupMaxK, kGroupMaxM);
    if (!o.X || !o.packed || !o.gamma || !o.Y) return fail(BITLINEAR_ERR_NULL, "op %d: X, packed, gamma and Y are required", i);
    if (!aligned16(o.X) || !aligned16(o.packed) || !aligned16(o.gamma) || !aligned16(o.Y))
      return fail(BITLINEAR_ERR_ALIGN, "op %d: tensor pointers must be 16-byte aligned", i);
    st = check_norm(o.norm_gain, o.norm_eps);
    if (st != BITLINEAR_OK) return st;
    items += skinny ? o.N / 16 : bl_group_gemm_tiles((int)M, (int)o.N);
  }
  if (items > 0x7fffffff) return fail(BITLINEAR_ERR_SHAPE, "too many output tiles");
  if (!skinny) return BITLINEAR_OK;
  int64_t max_k = 0;
  for (int i = 0; i < n_ops; ++i) max_k = std::max(max_k, op_lds_k(ops[i]));
  if (bl_group_lds_bytes((int)M, (int)max_k) > kGroupMaxLds)
    return fail(BITLINEAR_ERR_SHAPE,
                "M=%lld tokens of K=%lld activations do not fit in LDS (M * (K + 16) + M * 2048 "
                "bytes must stay within %zu)", (long long)M, (long long)max_k, kGroupMaxLds);
  return BITLINEAR_OK;
}

}  // namespace

// ---- Scratch of the forward that allocates nothing ----
// One fixed device array (BITLINEAR_NOALLOC_SCRATCH_BYTES) per GPU, for
// callers that cannot allocate.  In host code `scratch` is only a host-side
// stand-in: its device address on each GPU comes from hipGetSymbolAddress,
// looked up once per device (with that device current) and kept here.
static __device__ __align__(256) unsigned char scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
bitlinear_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "bitlinear_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BITLINEAR_ERR_ARG, "device %d is beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "bitlinear_forward_noalloc: hipGetSymbolAddress");
    if (!ptr) return fail(BITLINEAR_ERR_HIP, "bitlinear_forward_noalloc: no scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BITLINEAR_OK;
}

}  // namespace

struct bitlinear_group {
  int n_ops;
  int M;
  int G;
  int max_k;
  int threads;
  bool norm;  // some layer has a subln gain
  bool glu;   // some layer has the gated epilogue
  bool b3;    // the layers' weights use the base-3 layout
  bool gemm;
  int n_items;  // items over all layers (output tiles in the GEMM mode)
  int n_units;  // shared work units of the skinny kernel
  GroupOp* ops;
  int* wg_begin;
  GroupUnit* units;
  int* queue;
  int8_t* xq;
  float* sx;
  int* rs;
};

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N % 16 != 0 || K % 256 != 0) return 0;
  return (size_t)N * (size_t)K / 4;
}

size_t bitlinear_weights_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N % 16 != 0 || K % 256 != 0) return 0;
  return align256((size_t)N * sizeof(double));
}

size_t bitlinear_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 1 || K < 1 || N % 16 != 0 || K % 256 != 0) return (size_t)-1;
  if (M == 0 || bl_gemv_supports(M, K)) return 0;
  return forward_workspace(M, K, N);
}

size_t bitlinear_forward_q_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 1 || K < 1 || N % 16 != 0 || K % 256 != 0) return (size_t)-1;
  if (M == 0) return 0;
  return bl_gemm_workspace_bytes(M, K, N);
}

static bitlinear_status quantize_weights_impl(const float* W, int64_t N, int64_t K,
                                              uint8_t* packed, float* gamma, void* ws,
                                              size_t ws_bytes, void* stream, bool glu,
                                              const char* name) {
  if (!W || !packed || !gamma) return fail(BITLINEAR_ERR_NULL, "W, packed and gamma are required");
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (!aligned16(W) || !aligned16(packed) || !aligned16(gamma))
    return fail(BITLINEAR_ERR_ALIGN, "W, packed and gamma must be 16-byte aligned");
  const size_t need = bitlinear_weights_workspace_bytes(N, K);
  if (!ws || ws_bytes < need)
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* row_sum = static_cast<double*>(ws);
  hipError_t e = bl_launch_absmean_rows(W, N, K, row_sum, s);
  if (e == hipSuccess) e = bl_launch_absmean_final(row_sum, N, K, gamma, s);
  if (e == hipSuccess) e = bl_launch_quant_pack(W, N, K, gamma, packed, s, glu);
  return from_hip(e, name);
}

bitlinear_status bitlinear_quantize_weights(const float* W, int64_t N, int64_t K,
                                            uint8_t* packed, float* gamma, void* ws,
                                            size_t ws_bytes, void* stream) {
  return quantize_weights_impl(W, N, K, packed, gamma, ws, ws_bytes, stream, false,
                               "bitlinear_quantize_weights");
}

bitlinear_status bitlinear_quantize_weights_glu(const float* W, int64_t N, int64_t K,
                                                uint8_t* packed, float* gamma, void* ws,
                                                size_t ws_bytes, void* stream) {
  return quantize_weights_impl(W, N, K, packed, gamma, ws, ws_bytes, stream, true,
                               "bitlinear_quantize_weights_glu");
}

bitlinear_status bitlinear_pack_ternary(const int8_t* Wq, int64_t N, int64_t K,
                                        uint8_t* packed, void* stream) {
  if (!Wq || !packed) return fail(BITLINEAR_ERR_NULL, "Wq and packed are required");
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (!aligned16(Wq) || !aligned16(packed))
    return fail(BITLINEAR_ERR_ALIGN, "Wq and packed must be 16-byte aligned");
  return from_hip(bl_launch_pack(Wq, N, K, packed, static_cast<hipStream_t>(stream)),
                  "bitlinear_pack_ternary");
}

bitlinear_status bitlinear_unpack_ternary(const uint8_t* packed, int64_t N, int64_t K,
                                          int8_t* Wq, void* stream) {
  if (!Wq || !packed) return fail(BITLINEAR_ERR_NULL, "packed and Wq are required");
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (!aligned16(Wq) || !aligned16(packed))
    return fail(BITLINEAR_ERR_ALIGN, "Wq and packed must be 16-byte aligned");
  return from_hip(bl_launch_unpack(packed, N, K, Wq, static_cast<hipStream_t>(stream)),
                  "bitlinear_unpack_ternary");
}

size_t bitlinear_packed_bytes_b3(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N % 16 != 0 || K % 16 != 0) return 0;
  return (size_t)N * (size_t)bl_b3_padded_k(K) / 5;
}

bitlinear_status bitlinear_quantize_weights_b3(const float* W, int64_t N, int64_t K,
                                               uint8_t* packed, float* gamma, void* ws,
                                               size_t ws_bytes, int glu, void* stream) {
  if (!W || !packed || !gamma) return fail(BITLINEAR_ERR_NULL, "W, packed and gamma are required");
  bitlinear_status st = check_nk_b3(N, K);
  if (st != BITLINEAR_OK) return st;
  if (glu && N % 32 != 0)
    return fail(BITLINEAR_ERR_SHAPE, "a fused gate+up matrix needs N %% 32 == 0, got %lld",
                (long long)N);
  if (!aligned16(W) || !aligned16(packed) || !aligned16(gamma))
    return fail(BITLINEAR_ERR_ALIGN, "W, packed and gamma must be 16-byte aligned");
  const size_t need = align256((size_t)N * sizeof(double));
  if (!ws || ws_bytes < need)
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* row_sum = static_cast<double*>(ws);
  hipError_t e = bl_launch_absmean_rows(W, N, K, row_sum, s);
  if (e == hipSuccess) e = bl_launch_absmean_final(row_sum, N, K, gamma, s);
  if (e == hipSuccess) e = bl_launch_quant_pack_b3(W, N, K, gamma, packed, s, glu != 0);
  return from_hip(e, "bitlinear_quantize_weights_b3");
}

bitlinear_status bitlinear_pack_ternary_b3(const int8_t* Wq, int64_t N, int64_t K,
                                           uint8_t* packed, void* stream) {
  if (!Wq || !packed) return fail(BITLINEAR_ERR_NULL, "Wq and packed are required");
  bitlinear_status st = check_nk_b3(N, K);
  if (st != BITLINEAR_OK) return st;
  if (!aligned16(Wq) || !aligned16(packed))
    return fail(BITLINEAR_ERR_ALIGN, "Wq and packed must be 16-byte aligned");
  return from_hip(bl_launch_pack_b3(Wq, N, K, packed, static_cast<hipStream_t>(stream)),
                  "bitlinear_pack_ternary_b3");
}

bitlinear_status bitlinear_unpack_ternary_b3(const uint8_t* packed, int64_t N, int64_t K,
                                             int8_t* Wq, void* stream) {
  if (!Wq || !packed) return fail(BITLINEAR_ERR_NULL, "packed and Wq are required");
  bitlinear_status st = check_nk_b3(N, K);
  if (st != BITLINEAR_OK) return st;
  if (!aligned16(Wq) || !aligned16(packed))
    return fail(BITLINEAR_ERR_ALIGN, "Wq and packed must be 16-byte aligned");
  return from_hip(bl_launch_unpack_b3(packed, N, K, Wq, static_cast<hipStream_t>(stream)),
                  "bitlinear_unpack_ternary_b3");
}

static bitlinear_status quantize_acts_impl(const void* X, bitlinear_dtype dtype, int64_t M,
                                           int64_t K, const float* norm_gain, float norm_eps,
                                           int8_t* Xq, float* x_scale, int32_t* x_rowsum,
                                           void* stream, const char* name) {
  if (dtype != BITLINEAR_F32 && dtype != BITLINEAR_BF16)
    return fail(BITLINEAR_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (M < 0 || K < 1 || K % 16 != 0 || K > kMaxK)
    return fail(BITLINEAR_ERR_SHAPE, "M=%lld K=%lld: need M >= 0, K >= 1, K %% 16 == 0",
                (long long)M, (long long)K);
  if (M > 0x7fffffff) return fail(BITLINEAR_ERR_SHAPE, "M=%lld too large", (long long)M);
  if (M == 0) return ok();
  if (!X || !Xq || !x_scale) return fail(BITLINEAR_ERR_NULL, "X, Xq and x_scale are required");
  if (!aligned16(X) || !aligned16(Xq) || !aligned16(x_scale) ||
      (x_rowsum && !aligned16(x_rowsum)))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const bitlinear_status st = check_norm(norm_gain, norm_eps);
  if (st != BITLINEAR_OK) return st;
  return from_hip(bl_launch_quant_acts(X, (int)dtype, M, K, Xq, x_scale, x_rowsum, nullptr, 0,
                                       static_cast<hipStream_t>(stream), norm_gain, norm_eps),
                  name);
}

bitlinear_status bitlinear_quantize_acts(const void* X, bitlinear_dtype dtype, int64_t M,
                                         int64_t K, int8_t* Xq, float* x_scale,
                                         int32_t* x_rowsum, void* stream) {
  return quantize_acts_impl(X, dtype, M, K, nullptr, 0.0f, Xq, x_scale, x_rowsum, stream,
                            "bitlinear_quantize_acts");
}

bitlinear_status bitlinear_quantize_acts_rmsnorm(const void* X, bitlinear_dtype dtype,
                                                 int64_t M, int64_t K, const float* norm_gain,
                                                 float norm_eps, int8_t* Xq, float* x_scale,
                                                 int32_t* x_rowsum, void* stream) {
  if (!norm_gain && M > 0) return fail(BITLINEAR_ERR_NULL, "norm_gain is required");
  return quantize_acts_impl(X, dtype, M, K, norm_gain, norm_eps, Xq, x_scale, x_rowsum, stream,
                            "bitlinear_quantize_acts_rmsnorm");
}


static bitlinear_status forward_impl(const void* X, bitlinear_dtype dtype, int64_t M,
                                     int64_t K, int64_t N, const float* norm_gain,
                                     float norm_eps, const uint8_t* packed, const float* gamma,
                                     float* Y, bitlinear_epilogue epi,
                                     const bitlinear_debug* dbg, void* ws, size_t ws_bytes,
                                     void* stream, const char* name) {
  if (dtype != BITLINEAR_F32 && dtype != BITLINEAR_BF16)
    return fail(BITLINEAR_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (!valid_epi(epi))
    return fail(BITLINEAR_ERR_ARG, "unknown epilogue %d", (int)epi);
  if (M < 0) return fail(BITLINEAR_ERR_SHAPE, "M=%lld is negative", (long long)M);
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (M > 0x7fffffff) return fail(BITLINEAR_ERR_SHAPE, "M=%lld too large", (long long)M);
  if (M == 0) return ok();
  if (!X || !packed || !gamma || !Y)
    return fail(BITLINEAR_ERR_NULL, "X, packed, gamma and Y are required");
  int8_t* xq_out = dbg ? dbg->xq_out : nullptr;
  float* xs_out = dbg ? dbg->xscale_out : nullptr;
  int32_t* acc_out = dbg ? dbg->acc_out : nullptr;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(gamma) || !aligned16(Y) ||
      (xq_out && !aligned16(xq_out)) || (xs_out && !aligned16(xs_out)) ||
      (acc_out && !aligned16(acc_out)))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  st = check_norm(norm_gain, norm_eps);
  if (st != BITLINEAR_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (bl_gemv_supports(M, K))
    return from_hip(bl_launch_gemv(X, (int)dtype, M, K, N, packed, gamma, Y, (int)epi, xq_out,
                                   xs_out, acc_out, s, norm_gain, norm_eps),
                    name);

  const size_t need = forward_workspace(M, K, N);
  if (!ws || ws_bytes < need)
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  char* base = static_cast<char*>(ws);
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* sx = reinterpret_cast<float*>(base + align256((size_t)M * (size_t)K));
  int32_t* rs = reinterpret_cast<int32_t*>(base + align256((size_t)M * (size_t)K) +
                                           align256((size_t)M * 4));
  int* gemm_ws = reinterpret_cast<int*>(base + q_workspace(M, K));
  // The quantization launch also clears the GEMM's counters, so the
  // workspace's contents on entry do not matter.
  hipError_t e = bl_launch_quant_acts(X, (int)dtype, M, K, xq, sx, rs, gemm_ws,
                                      (int)(bl_gemm_counter_bytes() / sizeof(int)), s,
                                      norm_gain, norm_eps);
  if (e == hipSuccess && xq_out)
    e = hipMemcpyAsync(xq_out, xq, (size_t)M * (size_t)K, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess && xs_out)
    e = hipMemcpyAsync(xs_out, sx, (size_t)M * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = bl_launch_gemm_q(xq, sx, rs, M, K, N, packed, gamma, Y, (int)epi, acc_out, gemm_ws,
                         s);
  return from_hip(e, name);
}

bitlinear_status bitlinear_forward(const void* X, bitlinear_dtype dtype, int64_t M, int64_t K,
                                   int64_t N, const uint8_t* packed, const float* gamma,
                                   float* Y, bitlinear_epilogue epi, const bitlinear_debug* dbg,
                                   void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(X, dtype, M, K, N, nullptr, 0.0f, packed, gamma, Y, epi, dbg, ws,
                      ws_bytes, stream, "bitlinear_forward");
}

bitlinear_status bitlinear_forward_rmsnorm(const void* X, bitlinear_dtype dtype, int64_t M,
                                           int64_t K, int64_t N, const float* norm_gain,
                                           float norm_eps, const uint8_t* packed,
                                           const float* gamma, float* Y,
                                           bitlinear_epilogue epi, const bitlinear_debug* dbg,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (!norm_gain && M > 0) return fail(BITLINEAR_ERR_NULL, "norm_gain is required");
  return forward_impl(X, dtype, M, K, N, norm_gain, norm_eps, packed, gamma, Y, epi, dbg, ws,
                      ws_bytes, stream, "bitlinear_forward_rmsnorm");
}


bitlinear_status bitlinear_forward_lut(const void* X, bitlinear_dtype dtype, int64_t K,
                                       int64_t N, const uint8_t* packed, const float* gamma,
                                       float* Y, bitlinear_epilogue epi,
                                       const bitlinear_debug* dbg, void* stream) {
  if (dtype != BITLINEAR_F32 && dtype != BITLINEAR_BF16)
    return fail(BITLINEAR_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (!valid_epi(epi)) return fail(BITLINEAR_ERR_ARG, "unknown epilogue %d", (int)epi);
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (K > kLutMaxK)
    return fail(BITLINEAR_ERR_SHAPE, "K=%lld exceeds %lld (the tables must fit in LDS)",
                (long long)K, (long long)kLutMaxK);
  if (!X || !packed || !gamma || !Y)
    return fail(BITLINEAR_ERR_NULL, "X, packed, gamma and Y are required");
  int8_t* xq_out = dbg ? dbg->xq_out : nullptr;
  float* xs_out = dbg ? dbg->xscale_out : nullptr;
  int32_t* acc_out = dbg ? dbg->acc_out : nullptr;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(gamma) || !aligned16(Y) ||
      (xq_out && !aligned16(xq_out)) || (xs_out && !aligned16(xs_out)) ||
      (acc_out && !aligned16(acc_out)))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  return from_hip(bl_launch_lut_gemv(X, (int)dtype, K, N, packed, gamma, Y, (int)epi, xq_out,
                                     xs_out, acc_out, static_cast<hipStream_t>(stream)),
                  "bitlinear_forward_lut");
}

size_t bitlinear_ffn_chain_workspace_bytes(int64_t N_up) {
  if (N_up < 16 || N_up % 16 != 0 || N_up > kMaxN) return 0;
  return align256(bl_chain_workspace_bytes(N_up));
}

bitlinear_status bitlinear_ffn_chain(const void* X, bitlinear_dtype dtype, int64_t M, int64_t K,
                                     int64_t N_up, const uint8_t* packed_up,
                                     const float* gamma_up, bitlinear_epilogue epi_up,
                                     int64_t N_down, const uint8_t* packed_down,
                                     const float* gamma_down, float* H, float* Y, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (dtype != BITLINEAR_F32 && dtype != BITLINEAR_BF16)
    return fail(BITLINEAR_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (epi_up != BITLINEAR_EPI_RELU2 && epi_up != BITLINEAR_EPI_RELU2_GLU)
    return fail(BITLINEAR_ERR_ARG, "epi_up must be BITLINEAR_EPI_RELU2 or _RELU2_GLU, got %d",
                (int)epi_up);
  const bool glu = epi_up == BITLINEAR_EPI_RELU2_GLU;
  bitlinear_status st = check_nk(N_up, K);
  if (st != BITLINEAR_OK) return st;
  if (glu && N_up % 32 != 0)
    return fail(BITLINEAR_ERR_SHAPE, "a fused gate+up matrix needs N %% 32 == 0, got %lld",
                (long long)N_up);
  const int64_t F = glu ? N_up / 2 : N_up;
  st = check_nk(N_down, F);
  if (st != BITLINEAR_OK) return st;
  if (M < 1 || M > 4 || K > 12288 || F > 12288)
    return fail(BITLINEAR_ERR_SHAPE,
                "M=%lld K=%lld F=%lld: the chained FFN needs 1 <= M <= 4 and K, F <= 12288",
                (long long)M, (long long)K, (long long)F);
  if (!X || !packed_up || !gamma_up || !packed_down || !gamma_down || !H || !Y)
    return fail(BITLINEAR_ERR_NULL, "X, both weights and gammas, H and Y are required");
  if (!aligned16(X) || !aligned16(packed_up) || !aligned16(gamma_up) ||
      !aligned16(packed_down) || !aligned16(gamma_down) || !aligned16(H) || !aligned16(Y))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!ws || ws_bytes < bitlinear_ffn_chain_workspace_bytes(N_up))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                bitlinear_ffn_chain_workspace_bytes(N_up), ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  return from_hip(bl_launch_ffn_chain(X, (int)dtype, M, K, N_up, packed_up, gamma_up, glu, H,
                                      N_down, packed_down, gamma_down, Y, ws,
                                      static_cast<hipStream_t>(stream)),
                  "bitlinear_ffn_chain");
}

bitlinear_status bitlinear_forward_noalloc(const void* X, bitlinear_dtype dtype, int64_t M,
                                           int64_t K, int64_t N, const uint8_t* packed,
                                           const float* gamma, float* Y,
                                           bitlinear_epilogue epi, const bitlinear_debug* dbg,
                                           void* stream) {
  // The workspace bitlinear_forward would need; (size_t)-1 on a bad shape,
  // which forward_impl then reports.
  const size_t need = bitlinear_workspace_bytes(M, K, N);
  void* ws = nullptr;
  if (need != (size_t)-1 && M > 0 && need > 0) {
    if (need > (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES)
      return fail(BITLINEAR_ERR_WORKSPACE,
                  "M=%lld K=%lld N=%lld needs %zu bytes of scratch; the no-allocation forward "
                  "has %zu (use bitlinear_forward with a workspace)",
                  (long long)M, (long long)K, (long long)N, need,
                  (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES);
    const bitlinear_status st = scratch_for_current_device(&ws);
    if (st != BITLINEAR_OK) return st;
  }
  // Same kernels as bitlinear_forward.  Its quantization launch clears the
  // GEMM's tile counters in the scratch itself, so the contents a previous
  // call left there do not matter.
  return forward_impl(X, dtype, M, K, N, nullptr, 0.0f, packed, gamma, Y, epi, dbg, ws,
                      ws ? (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES : 0, stream,
                      "bitlinear_forward_noalloc");
}

bitlinear_status bitlinear_forward_q(const int8_t* Xq, const float* x_scale,
                                     const int32_t* x_rowsum, int64_t M, int64_t K, int64_t N,
                                     const uint8_t* packed, const float* gamma, float* Y,
                                     bitlinear_epilogue epi, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!valid_epi(epi))
    return fail(BITLINEAR_ERR_ARG, "unknown epilogue %d", (int)epi);
  if (M < 0) return fail(BITLINEAR_ERR_SHAPE, "M=%lld is negative", (long long)M);
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (M > 0x7fffffff) return fail(BITLINEAR_ERR_SHAPE, "M=%lld too large", (long long)M);
  if (M == 0) return ok();
  if (!Xq || !x_scale || !x_rowsum || !packed || !gamma || !Y)
    return fail(BITLINEAR_ERR_NULL, "Xq, x_scale, x_rowsum, packed, gamma and Y are required");
  if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(x_rowsum) || !aligned16(packed) ||
      !aligned16(gamma) || !aligned16(Y))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ws) {
    const size_t need = bl_gemm_workspace_bytes(M, K, N);
    if (ws_bytes < need)
      return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  ws_bytes);
    if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  if (bl_gemv_supports(M, K))  // up to four tokens: the rows are copied, not re-quantized
    return from_hip(bl_launch_gemv_q(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y, (int)epi,
                                     nullptr, s),
                    "bitlinear_forward_q");
  return from_hip(bl_launch_gemm_q(Xq, x_scale, x_rowsum, M, K, N, packed, gamma, Y,
                                   (int)epi, nullptr, ws, s),
                  "bitlinear_forward_q");
}

size_t bitlinear_forward_glu_quant_workspace_bytes(void) { return 256; }

bitlinear_status bitlinear_forward_glu_quant(const void* X, bitlinear_dtype dtype, int64_t M,
                                             int64_t K, int64_t N, const uint8_t* packed,
                                             const float* gamma, float* H, int8_t* Hq,
                                             float* h_scale, int32_t* h_rowsum, void* ws,
                                             size_t ws_bytes, void* stream) {
  if (dtype != BITLINEAR_F32 && dtype != BITLINEAR_BF16)
    return fail(BITLINEAR_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  bitlinear_status st = check_nk(N, K);
  if (st != BITLINEAR_OK) return st;
  if (N % 32 != 0)
    return fail(BITLINEAR_ERR_SHAPE, "a fused gate+up matrix needs N %% 32 == 0, got %lld",
                (long long)N);
  if (M < 1 || !bl_gemv_supports(M, K))
    return fail(BITLINEAR_ERR_SHAPE,
                "M=%lld K=%lld: the quantized gated output needs 1 <= M <= 4 and K <= 12288",
                (long long)M, (long long)K);
  if (!X || !packed || !gamma || !H || !Hq || !h_scale || !h_rowsum)
    return fail(BITLINEAR_ERR_NULL, "X, packed, gamma, H, Hq, h_scale and h_rowsum are required");
  if (!aligned16(X) || !aligned16(packed) || !aligned16(gamma) || !aligned16(H) ||
      !aligned16(Hq) || !aligned16(h_scale) || !aligned16(h_rowsum))
    return fail(BITLINEAR_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!ws || ws_bytes < bitlinear_forward_glu_quant_workspace_bytes())
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                bitlinear_forward_glu_quant_workspace_bytes(), ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");
  return from_hip(bl_launch_gemv_glu_quant(X, (int)dtype, M, K, N, packed, gamma, H, Hq, h_scale,
                                           h_rowsum, static_cast<int*>(ws),
                                           static_cast<hipStream_t>(stream)),
                  "bitlinear_forward_glu_quant");
}

size_t bitlinear_group_workspace_bytes(const bitlinear_group_op* ops, int n_ops, int64_t M) {
  if (check_group(ops, n_ops, M) != BITLINEAR_OK) return 0;
  return group_layout(ops, n_ops, M).total;
}

bitlinear_status bitlinear_group_create(const bitlinear_group_op* ops, int n_ops, int64_t M,
                                        void* ws, size_t ws_bytes, bitlinear_group** out) {
  if (!out) return fail(BITLINEAR_ERR_NULL, "out is required");
  *out = nullptr;
  bitlinear_status st = check_group(ops, n_ops, M);
  if (st != BITLINEAR_OK) return st;
  const bool skinny = M <= kGroupMaxM;
  const GroupLayout L = group_layout(ops, n_ops, M);
  if (!ws || ws_bytes < L.total)
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BITLINEAR_ERR_ALIGN, "workspace must be 16-byte aligned");

  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return from_hip(e, "bitlinear_group_create");
  std::vector<GroupOp> table((size_t)n_ops);
  int64_t item = 0, xq_off = 0;
  int max_k = 0;
  bool norm = false, glu = false;
  for (int i = 0; i < n_ops; ++i) {
    const bitlinear_group_op& o = ops[i];
    GroupOp& t = table[(size_t)i];
    t = GroupOp{};
    t.X = o.X;
    t.packed = o.packed;
    t.gamma = o.gamma;
    t.Y = o.Y;
    t.K = (int32_t)o.K;
    t.N = (int32_t)o.N;
    t.dtype = (int32_t)o.dtype;
    t.epi = (int32_t)o.epi;
    if (o.epi == BITLINEAR_EPI_RELU2_GLU) glu = true;
    t.item_begin = (int32_t)item;
    t.norm_gain = o.norm_gain;
    t.norm_eps = o.norm_eps;
    t.fmt = (int32_t)o.format;
    if (o.norm_gain) norm = true;
    t.xq_off = xq_off;
    xq_off += (int64_t)align256((size_t)M * (size_t)o.K);
    // Work items: 16-row weight tiles (skinny) or output tiles of the GEMM;
    // either way an item's cost is proportional to K.
    const int64_t items = skinny ? o.N / 16 : bl_group_gemm_tiles((int)M, (int)o.N);
    item += items;
    if (op_lds_k(o) > max_k) max_k = (int)op_lds_k(o);
  }
  // As many workgroups as fit on the chip at once, at most four per compute
  // unit (skinny: each holds one layer's int8 activations in LDS and takes
  // work units from the queue; GEMM: output tiles strided).
  int threads = 256, per_cu = 1;
  if (skinny) {
    e = bl_group_plan((int)M, max_k, norm, is_b3(ops[0]), &threads, &per_cu);
    if (e != hipSuccess) return from_hip(e, "bitlinear_group_create");
  } else {
    per_cu = bl_group_gemm_blocks_per_cu((int)M);
  }
  if (per_cu > 4) per_cu = 4;
  int G = per_cu * (cus > 0 ? cus : 1);
  if (G > kGroupMaxWG) G = kGroupMaxWG;

  // Skinny kernel: cost-balanced contiguous static ranges over the tiles
  // before the split (workgroup g starts at the first tile whose preceding
  // cost reaches g/G of the static cost), then the shared units.  (The GEMM
  // mode takes output tiles strided instead.)
  std::vector<int> wg_begin((size_t)G + 1, 0);
  std::vector<GroupUnit> units;
  if (skinny) {
    int64_t split = 0, n_units = 0;
    group_split(ops, n_ops, M, &split, &n_units, [&](int op, int64_t first, int64_t end) {
      units.push_back(GroupUnit{(int32_t)first, (int32_t)end, op, 0});
    });
    int64_t static_cost = 0;
    {
      int64_t it = 0;
      for (int i = 0; i < n_ops && it < split; ++i) {
        const int64_t tiles = std::min<int64_t>(ops[i].N / 16, split - it);
        static_cost += tiles * op_kblocks(ops[i]);
        it += tiles;
      }
    }
    int g = 0;
    int64_t before = 0, it = 0;
    for (int i = 0; i < n_ops && it < split; ++i) {
      const int64_t kb = op_kblocks(ops[i]);
      const int64_t tiles = ops[i].N / 16;
      for (int64_t t = 0; t < tiles && it < split; ++t, ++it) {
        while (g <= G && before * G >= (int64_t)g * static_cost) wg_begin[(size_t)g++] = (int)it;
        before += kb;
      }
    }
    while (g <= G) wg_begin[(size_t)g++] = (int)split;
  }
  // The table, the schedule and the cleared queue go to the device on the
  // null stream; waiting for that stream alone (not the whole device) makes
  // them visible to launches on any stream afterwards.
  char* base = static_cast<char*>(ws);
  const int zeros[64] = {};
  e = hipMemcpyAsync(base + L.table, table.data(), table.size() * sizeof(GroupOp),
                     hipMemcpyHostToDevice, nullptr);
  if (e == hipSuccess)
    e = hipMemcpyAsync(base + L.wg_begin, wg_begin.data(), wg_begin.size() * sizeof(int),
                       hipMemcpyHostToDevice, nullptr);
  if (e == hipSuccess && !units.empty())
    e = hipMemcpyAsync(base + L.units, units.data(), units.size() * sizeof(GroupUnit),
                       hipMemcpyHostToDevice, nullptr);
  if (e == hipSuccess)  // the kernel leaves the queue zero again
    e = hipMemcpyAsync(base + L.queue, zeros, sizeof zeros, hipMemcpyHostToDevice, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) return from_hip(e, "bitlinear_group_create");
  bitlinear_group* g = new (std::nothrow) bitlinear_group;
  if (!g) return fail(BITLINEAR_ERR_ARG, "out of host memory");
  g->n_ops = n_ops;
  g->M = (int)M;
  g->G = G;
  g->max_k = max_k;
  g->threads = threads;
  g->norm = norm;
  g->glu = glu;
  g->b3 = is_b3(ops[0]);
  g->gemm = !skinny;
  g->n_items = (int)item;
  g->n_units = (int)L.n_units;
  g->ops = reinterpret_cast<GroupOp*>(base + L.table);
  g->wg_begin = reinterpret_cast<int*>(base + L.wg_begin);
  g->units = reinterpret_cast<GroupUnit*>(base + L.units);
  g->queue = reinterpret_cast<int*>(base + L.queue);
  g->xq = reinterpret_cast<int8_t*>(base + L.xq);
  g->sx = reinterpret_cast<float*>(base + L.sx);
  g->rs = reinterpret_cast<int*>(base + L.rs);
  *out = g;
  return ok();
}

bitlinear_status bitlinear_group_forward(const bitlinear_group* g, void* stream) {
  if (!g) return fail(BITLINEAR_ERR_NULL, "group handle is required");
  if (g->gemm) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e =
        bl_launch_group_quant(g->ops, g->n_ops, g->M, g->max_k, g->norm, g->xq, g->sx, g->rs, s);
    if (e == hipSuccess)
      e = bl_launch_group_gemm(g->ops, g->n_ops, g->M, g->n_items, g->G, g->xq, g->sx, g->rs,
                               g->glu, s);
    return from_hip(e, "bitlinear_group_forward");
  }
  return from_hip(bl_launch_group(g->ops, g->n_ops, g->M, g->wg_begin, g->units, g->n_units,
                                  g->queue, g->G, g->max_k, g->threads, g->norm, g->b3, g->xq, g->sx,
                                  g->rs,
                                  static_cast<hipStream_t>(stream)),
                  "bitlinear_group_forward");
}

void bitlinear_group_destroy(bitlinear_group* g) { delete g; }

const char* bitlinear_status_string(bitlinear_status s) {
  switch (s) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "null pointer";
    case BITLINEAR_ERR_SHAPE: return "bad shape";
    case BITLINEAR_ERR_ALIGN: return "misaligned pointer";
    case BITLINEAR_ERR_DTYPE: return "unknown dtype";
    case BITLINEAR_ERR_WORKSPACE: return "workspace too small";
    case BITLINEAR_ERR_HIP: return "HIP runtime error";
    case BITLINEAR_ERR_ARG: return "bad argument";
  }
  return "unknown status";
}

const char* bitlinear_last_error(void) { return g_last_error; }

}  // extern "C"
