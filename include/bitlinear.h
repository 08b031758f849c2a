/*
 * bitlinear.h -- C ABI of the W1.58A8 BitLinear forward for MI355X (gfx950).
 *
 * What is computed (sources: "BitNet b1.58 2B4T Technical Report" paper card,
 * ai-papers.xuzou.cn, sections "Method Adaptation" and "Compute Setup";
 * fishai news digest on BitNet b1.58 2B4T, news.fishai.com.cn/news/3455510,
 * the BitLinear items; dignews.cc article on BitNet b1.58 2B4T, section 2):
 * a BitLinear layer stands in for a dense linear layer y = x W^T without
 * bias.  Its weights are mapped to {-1, 0, +1} by an absmean scale and
 * stored four to a byte in HBM; its input is mapped per token to 8-bit
 * integers by an absmax scale; the product runs on integers and is scaled
 * back.  The pages give no formulas; the readings this library implements:
 *
 *   gamma    = mean |W| over the whole [N][K] matrix, summed in double (each
 *              row in column order, then the rows in row order) and rounded
 *              once to float; gamma_c = max(gamma, 1e-5f).
 *   q_w      = clamp(rint(W / gamma_c), -1, 1) (float division, ties to even).
 *   per token m: a = max_k |x[m,k]|, a_c = max(a, 1e-5f), qs = 127.0f / a_c,
 *              q_x = clamp(rint(x * qs), -127, 127), s_x[m] = a_c / 127.0f.
 *   acc      = sum_k q_x[m,k] * q_w[n,k], exact in int32.
 *   y[m,n]   = ((float)acc * s_x[m]) * gamma_c, two float roundings in that
 *              order (no fused multiply-add).
 *   ReLU^2   (optional epilogue) y <- max(y, 0)^2.
 *
 * All of it is reproducible bit for bit: integer work is exact and the float
 * steps are single IEEE operations in a fixed order.
 *
 * Layouts.  Row-major, contiguous.  W and q_w are [N][K] (like a linear
 * layer's weight), X is [M][K], Y is [M][N].  Packed weights: the matrix is
 * cut into tiles of 16 rows x 256 columns; each tile is 1024 bytes; tiles
 * are stored row-tile major, then by column block.  Inside a tile, the
 * 16-byte chunk c (0..63) holds row (c mod 16) of the tile and its columns
 * 64*(c div 16) .. 64*(c div 16)+63 of the block; inside a chunk, the
 * column offset t (0..63) is stored in little-endian 32-bit word (t div 16),
 * byte (t mod 4), bits 2f..2f+1 with f = (t mod 16) div 4, as the code
 * q_w + 1 (0, 1 or 2; 3 never occurs).  So one 32-bit word shifted right by
 * 2f and masked with 0x03030303 gives the codes of four consecutive columns,
 * one per byte, and 64 lanes that each load 16 bytes read one whole tile.
 *
 * Conventions for every call below.
 *   - Tensor pointers are device pointers (hipMalloc'ed or torch CUDA/HIP
 *     tensors) owned by the caller; the library allocates no device memory
 *     and keeps no pointer after a call returns.
 *   - Every tensor pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return; no call synchronizes.  Results are ready when
 *     the stream reaches them.
 *   - Arguments are checked before anything is enqueued; a failed check
 *     returns an error code and enqueues nothing.  A launch failure returns
 *     BITLINEAR_ERR_HIP.  Device faults surface at the caller's next
 *     synchronization.  bitlinear_last_error() gives a thread-local message
 *     for the last failing call on that thread.
 *   - Inputs must be finite; NaN or Inf input gives unspecified (but memory
 *     safe) results.
 *   - Shapes: N % 16 == 0 and K % 256 == 0 (the packed tile); M >= 0 and
 *     M == 0 is a no-op that returns BITLINEAR_OK; N, K >= 1 otherwise.
 *     K <= 8,388,608 (checked; |acc| <= 127*K then fits int32 with room)
 *     and N <= 4,194,304 (checked).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 7

typedef enum {
  BITLINEAR_OK = 0,
  BITLINEAR_ERR_NULL = 1,      /* a required pointer is NULL */
  BITLINEAR_ERR_SHAPE = 2,     /* a size is negative or breaks N%16, K%256 */
  BITLINEAR_ERR_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
  BITLINEAR_ERR_DTYPE = 4,     /* unknown bitlinear_dtype */
  BITLINEAR_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required */
  BITLINEAR_ERR_HIP = 6,       /* the HIP runtime reported an error */
  BITLINEAR_ERR_ARG = 7        /* another bad argument (e.g. epilogue) */
} bitlinear_status;

typedef enum {
  BITLINEAR_F32 = 0,  /* float32 activations */
  BITLINEAR_BF16 = 1  /* bfloat16 activations, widened exactly to float */
} bitlinear_dtype;

typedef enum {
  BITLINEAR_EPI_NONE = 0,  /* Y = y */
  BITLINEAR_EPI_RELU2 = 1, /* Y = max(y, 0)^2 (the squared-ReLU FFN
                              activation, "BitNet b1.58 2B4T Technical
                              Report" card, Method Adaptation) */
  BITLINEAR_EPI_RELU2_GLU = 2
  /* Gated squared ReLU of a fused gate+up matrix packed by
     bitlinear_quantize_weights_glu: with y = [gate | up] (N columns),
     Y [M][N/2] = max(gate, 0)^2 * up, left to right, no fused multiply-add.
     The pages give ReLU^2 as the FFN activation (same card) and no gating
     formula; the gate+up shape of the decode workload is read as gate rows
     then up rows.  Only valid with weights packed that way; dbg->acc_out
     then stays [M][N] in the unpermuted row order. */
} bitlinear_epilogue;

/* Layouts of packed weights.  BITLINEAR_FMT_2BIT is the layout described
 * above (four codes per byte), used by every call.  BITLINEAR_FMT_B3 is the
 * denser base-3 layout (five codes per byte, 1.6 bits per weight; a ternary
 * weight carries log2(3) bits, wikiprompt.org "1.58-bit large language
 * model", introduction; the technical-report card, Evidence, gives the 2B
 * model's weights as 0.4 GB, which is that density): K is padded up to Kp, a
 * multiple of 320, with code 0; the matrix is cut into tiles of 16 rows x
 * 320 columns (1024 bytes) ordered row-tile major, then by column block;
 * 16-byte chunk c of a tile holds row (c mod 16) and the columns
 * 80*(c div 16) .. +79 of its block; byte b of little-endian 32-bit word j
 * of a chunk holds the codes c_i of columns 20j + 4i + b (i = 0..4) as the
 * number c_0 + 3 c_1 + 9 c_2 + 27 c_3 + 81 c_4 (0..242).  Only the grouped
 * forward (up to 16 tokens) runs on it. */
typedef enum {
  BITLINEAR_FMT_2BIT = 0,
  BITLINEAR_FMT_B3 = 1
} bitlinear_weight_format;

/* Optional extra outputs of bitlinear_forward, for checking the integer
 * intermediates.  Each pointer may be NULL.  xq_out: int8 [M][K];
 * xscale_out: float [M]; acc_out: int32 [M][N] (the exact sum_k q_x*q_w). */
typedef struct {
  int8_t* xq_out;
  float* xscale_out;
  int32_t* acc_out;
} bitlinear_debug;

/* Version of this ABI (BITLINEAR_ABI_VERSION). */
int bitlinear_abi_version(void);

/* Bytes of the packed form of an [N][K] ternary matrix: N*K/4.  Returns 0
 * when N or K is negative or breaks N%16 / K%256. */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Workspace bytes bitlinear_quantize_weights needs for an [N][K] matrix
 * (per-row double sums).  0 on a bad shape. */
size_t bitlinear_weights_workspace_bytes(int64_t N, int64_t K);

/* Workspace bytes bitlinear_forward needs for M tokens x K -> N (may be 0):
 * when the large-M path runs, the quantized activations, scales and row
 * sums, then bitlinear_forward_q's workspace.  Returns (size_t)-1 on a bad
 * shape.  Needs no GPU. */
size_t bitlinear_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* Workspace bytes bitlinear_forward_q can use for M x K -> N (about 16 MiB:
 * counters, then partial int32 sums of output tiles cut along K).
 * Returns (size_t)-1 on a bad shape.  Needs no GPU. */
size_t bitlinear_forward_q_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* Absmean ternary quantization and packing of float W [N][K] ("BitNet b1.58
 * 2B4T Technical Report" card, Method Adaptation: absmean to {-1,0,+1}, four
 * ternary weights per int8 in HBM).  Writes `packed`
 * (bitlinear_packed_bytes(N,K) bytes) and gamma_c into `gamma` (one float,
 * device memory).  `ws` holds at least bitlinear_weights_workspace_bytes(N,K)
 * bytes; its contents on entry do not matter. */
bitlinear_status bitlinear_quantize_weights(const float* W, int64_t N, int64_t K,
                                            uint8_t* packed, float* gamma, void* ws,
                                            size_t ws_bytes, void* stream);

/* The same for a fused gate+up matrix W [N][K] (gate rows 0..N/2-1, then
 * the up rows; one gamma over the whole matrix), packed with its halves
 * interleaved: 16-row tile t holds gate rows 8t..8t+7, then up rows
 * N/2+8t..N/2+8t+7, so that every kernel finds a gate row and its up row in
 * one tile.  Use with BITLINEAR_EPI_RELU2_GLU. */
bitlinear_status bitlinear_quantize_weights_glu(const float* W, int64_t N, int64_t K,
                                                uint8_t* packed, float* gamma, void* ws,
                                                size_t ws_bytes, void* stream);

/* Packs already-ternary int8 q_w [N][K] into the layout above: four 2-bit
 * codes per byte ("BitNet b1.58 2B4T Technical Report" card, Method
 * Adaptation: four ternary weights are stored in one int8; dignews.cc
 * article, section 2).  `packed` receives bitlinear_packed_bytes(N,K) bytes.
 * Values should be in {-1,0,1}; any other value is clamped into that range
 * before it is stored.  Errors: NULL pointers, bad shapes or misaligned
 * pointers are rejected before anything is enqueued. */
bitlinear_status bitlinear_pack_ternary(const int8_t* Wq, int64_t N, int64_t K,
                                        uint8_t* packed, void* stream);

/* Inverse of the packing (same passages as bitlinear_pack_ternary): int8
 * q_w [N][K], caller-allocated, from bitlinear_packed_bytes(N,K) packed
 * bytes.  A code 3 (never written by this library) unpacks as 0.  Errors as
 * bitlinear_pack_ternary. */
bitlinear_status bitlinear_unpack_ternary(const uint8_t* packed, int64_t N, int64_t K,
                                          int8_t* Wq, void* stream);

/* Bytes of an [N][K] matrix in the base-3 layout: N * Kp / 5 with Kp = K
 * rounded up to a multiple of 320.  0 when N or K is below 1 or breaks
 * N % 16 / K % 16. */
size_t bitlinear_packed_bytes_b3(int64_t N, int64_t K);

/* Absmean ternary quantization of float W [N][K], as
 * bitlinear_quantize_weights (the same gamma and codes), packed in the
 * base-3 layout: `packed` receives bitlinear_packed_bytes_b3(N, K) bytes.
 * glu != 0 packs a fused gate+up matrix with its halves interleaved per
 * 16-row tile, as bitlinear_quantize_weights_glu (then N % 32 == 0).  K needs
 * only K % 16 == 0.  `ws` as bitlinear_quantize_weights. */
bitlinear_status bitlinear_quantize_weights_b3(const float* W, int64_t N, int64_t K,
                                               uint8_t* packed, float* gamma, void* ws,
                                               size_t ws_bytes, int glu, void* stream);

/* Packs int8 q_w [N][K] (values clamped into {-1, 0, 1}) in the base-3
 * layout, and unpacks it (padding columns are skipped).  Shapes as
 * bitlinear_packed_bytes_b3; errors as bitlinear_pack_ternary. */
bitlinear_status bitlinear_pack_ternary_b3(const int8_t* Wq, int64_t N, int64_t K,
                                           uint8_t* packed, void* stream);
bitlinear_status bitlinear_unpack_ternary_b3(const uint8_t* packed, int64_t N, int64_t K,
                                             int8_t* Wq, void* stream);

/* Per-token absmax int8 quantization of X [M][K] (fishai digest, activation
 * quantization item; technical-report card, Method Adaptation).  Writes Xq
 * [M][K], x_scale [M] (= s_x) and, if x_rowsum is not NULL, the int32 row
 * sums of Xq [M].  Here K needs only K >= 1 and K % 16 == 0. */
bitlinear_status bitlinear_quantize_acts(const void* X, bitlinear_dtype dtype, int64_t M,
                                         int64_t K, int8_t* Xq, float* x_scale,
                                         int32_t* x_rowsum, void* stream);

/* The same quantization after subln, the normalization a BitLinear layer
 * contains (fishai digest, list of BitLinear parts: normalization;
 * technical-report card, Method Adaptation), read as an RMSNorm of each
 * token with a per-feature gain: x_hat = x * r * g with
 * r = 1 / sqrt(mean_k x^2 + norm_eps).  Absmax quantization cannot see the
 * row's positive factor r, so Xq and x_rowsum are the codes of x * g (float
 * products) and x_scale = (max|x * g| / 127) * r: the codes do not depend on
 * the order of the sum of squares (taken in double).  norm_gain: float [K],
 * device, 16-byte aligned, required; norm_eps finite and >= 0 (1e-5 is the
 * usual value).  Other arguments and errors as bitlinear_quantize_acts. */
bitlinear_status bitlinear_quantize_acts_rmsnorm(const void* X, bitlinear_dtype dtype,
                                                 int64_t M, int64_t K, const float* norm_gain,
                                                 float norm_eps, int8_t* Xq, float* x_scale,
                                                 int32_t* x_rowsum, void* stream);

/* The BitLinear forward ("BitNet b1.58 2B4T Technical Report" card, Method
 * Adaptation and Compute Setup: the packed weights are loaded, unpacked just
 * before the product and multiplied with per-token int8 activations; fishai
 * digest, the BitLinear items): Y [M][N] (float) from X [M][K] (dtype), the
 * packed ternary weights and gamma_c (device float, as written by
 * bitlinear_quantize_weights).  Quantizes X per token, contracts in int32,
 * rescales, then applies `epi`.  `dbg` may be NULL.  `ws` holds at least
 * bitlinear_workspace_bytes(M, K, N) bytes (NULL allowed when that is 0).
 * Kernels by token count (both give the same bits): M <= 4 one fused launch
 * (quantization and v_dot4 contraction); larger M a quantization launch and
 * the tiled int8 MFMA GEMM of bitlinear_forward_q, with its workspace (which
 * the quantization launch clears, so `ws` needs no initial contents).  For
 * steps with several layers, the grouped forward below runs all of them
 * together. */
bitlinear_status bitlinear_forward(const void* X, bitlinear_dtype dtype, int64_t M,
                                   int64_t K, int64_t N, const uint8_t* packed,
                                   const float* gamma, float* Y, bitlinear_epilogue epi,
                                   const bitlinear_debug* dbg, void* ws, size_t ws_bytes,
                                   void* stream);

/* bitlinear_forward with subln first, fused into the quantization (as in
 * bitlinear_quantize_acts_rmsnorm): norm_gain float [K] (device, 16-byte
 * aligned, required), norm_eps finite and >= 0.  Same kernels, workspace and
 * errors as bitlinear_forward; xscale_out in `dbg` receives the scale with
 * the RMS factor. */
bitlinear_status bitlinear_forward_rmsnorm(const void* X, bitlinear_dtype dtype, int64_t M,
                                           int64_t K, int64_t N, const float* norm_gain,
                                           float norm_eps, const uint8_t* packed,
                                           const float* gamma, float* Y,
                                           bitlinear_epilogue epi, const bitlinear_debug* dbg,
                                           void* ws, size_t ws_bytes, void* stream);

/* ---- Forward that allocates nothing -------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * bitlinear_forward without the workspace argument: where the forward needs
 * a workspace (M > 4), it uses a fixed scratch array of
 * BITLINEAR_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every
 * GPU it runs on until the process ends.  It calls no allocating routine.
 * A forward whose workspace (bitlinear_workspace_bytes) exceeds that size
 * returns BITLINEAR_ERR_WORKSPACE before anything is enqueued; the shapes of
 * the 2B and 7B workloads fit (the largest, 2048 tokens of 6912 -> 2560,
 * needs 29.5 MiB).  Every call on one GPU shares that GPU's array and leaves
 * its contents behind: calls that overlap on one GPU (on different streams,
 * or from different threads without ordering) race and give undefined
 * results.  The first call on a device looks up the array's device address
 * (a host-side query, no allocation).  Results are bit-identical to
 * bitlinear_forward; arguments and other errors as there. */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (32u << 20)
bitlinear_status bitlinear_forward_noalloc(const void* X, bitlinear_dtype dtype, int64_t M,
                                           int64_t K, int64_t N, const uint8_t* packed,
                                           const float* gamma, float* Y,
                                           bitlinear_epilogue epi, const bitlinear_debug* dbg,
                                           void* stream);

/* The same forward from activations already quantized by
 * bitlinear_quantize_acts (the int8 matmul and rescale of the same card,
 * Method Adaptation): Xq [M][K], x_scale [M], x_rowsum [M] (all three
 * required).  The output tiles (128 x 128; 64 x 128 up to 64 tokens) are
 * spread over the compute units one workgroup each; when they do not divide
 * evenly, each tile of the last, partial round is instead cut along K into
 * pieces, one workgroup each, whose exact int32 partial sums meet in `ws`
 * (same bits either way).  `ws` (device, 16-byte aligned, at least
 * bitlinear_forward_q_workspace_bytes) enables that; NULL runs one workgroup
 * per tile.  Above 64 tokens, when 128 x 256 tiles outnumber the compute
 * units, fit on them at once (two per unit) and fill at least three
 * quarters of those places, those run instead, never cut along K.  Every choice gives the same bits.  Up to four tokens (K <=
 * 12288) the one-launch decode kernel runs instead, with the rows copied
 * rather than quantized, and `ws` is not used.  Its first 4 KiB (counters) must be zero the first time a
 * workspace is used, and every call leaves them zero again; the rest needs
 * no initial contents.  Calls that share a workspace must not overlap. */
bitlinear_status bitlinear_forward_q(const int8_t* Xq, const float* x_scale,
                                     const int32_t* x_rowsum, int64_t M, int64_t K,
                                     int64_t N, const uint8_t* packed, const float* gamma,
                                     float* Y, bitlinear_epilogue epi, void* ws,
                                     size_t ws_bytes, void* stream);

/* The front half of the gated FFN (the technical-report card, Method
 * Adaptation: squared ReLU as the FFN activation) with the down projection's input
 * quantization fused in: from a fused gate+up matrix packed with
 * bitlinear_quantize_weights_glu, h = max(gate, 0)^2 * up as the
 * BITLINEAR_EPI_RELU2_GLU forward computes it, written to H [M][N/2]
 * (float) and, in the same launch, quantized per token exactly as
 * bitlinear_quantize_acts would quantize H: Hq [M][N/2] int8, h_scale [M],
 * h_rowsum [M], ready for bitlinear_forward_q of the down projection.  The
 * last workgroup to finish quantizes (no workgroup waits for another).
 * 1 <= M <= 4, K % 256 == 0 and K <= 12288, N % 32 == 0.  `ws`: at least
 * bitlinear_forward_glu_quant_workspace_bytes() bytes, 16-byte aligned,
 * zero before its first use and left zero by every call (a counter); calls
 * sharing it must not overlap.  Errors as bitlinear_forward. */
size_t bitlinear_forward_glu_quant_workspace_bytes(void);
bitlinear_status bitlinear_forward_glu_quant(const void* X, bitlinear_dtype dtype, int64_t M,
                                             int64_t K, int64_t N, const uint8_t* packed,
                                             const float* gamma, float* H, int8_t* Hq,
                                             float* h_scale, int32_t* h_rowsum, void* ws,
                                             size_t ws_bytes, void* stream);

/* The decode FFN ("BitNet b1.58 2B4T Technical Report" card, Method
 * Adaptation: squared ReLU as the FFN activation) in one persistent launch:
 * h = relu(X W_up^T)^2 -- or, with epi_up BITLINEAR_EPI_RELU2_GLU and W_up a
 * fused gate+up matrix from bitlinear_quantize_weights_glu, the gated
 * max(gate, 0)^2 * up -- written to H [M][F] (F = N_up, or N_up / 2 gated),
 * then Y [M][N_down] = the BitLinear forward of h with W_down [N_down][F].
 * H and Y are the same bits as two bitlinear_forward calls.  The up tiles'
 * workgroups come first in the grid; a down tile's workgroup waits until
 * every up tile is done (a bounded wait: workgroups start in index order, so
 * the up tiles are running).  1 <= M <= 4; K % 256 == 0 and F %
 * 256 == 0, both <= 12288; dtype as bitlinear_forward.  `ws`: at least
 * bitlinear_ffn_chain_workspace_bytes(N_up) bytes (0 for a bad N_up),
 * 16-byte aligned, zero before its first use; it holds a counter, a
 * generation count and one flag per up tile, which every call leaves ready
 * for the next (its third int is set to 1 and stays set if a wait ever gave
 * up, which only a failing device can cause).  Calls sharing it must not
 * overlap.  Errors as bitlinear_forward. */
size_t bitlinear_ffn_chain_workspace_bytes(int64_t N_up);
bitlinear_status bitlinear_ffn_chain(const void* X, bitlinear_dtype dtype, int64_t M, int64_t K,
                                     int64_t N_up, const uint8_t* packed_up,
                                     const float* gamma_up, bitlinear_epilogue epi_up,
                                     int64_t N_down, const uint8_t* packed_down,
                                     const float* gamma_down, float* H, float* Y, void* ws,
                                     size_t ws_bytes, void* stream);

/* The forward of one token (M = 1) by table lookup instead of multiplies,
 * the method bitnet.cpp's ternary kernels take from T-MAC (dignews.cc
 * article on BitNet b1.58 2B4T, section 3).  X [1][K] is quantized as in
 * bitlinear_forward; then, for every pair of columns, a table of the 16 sums
 * its two 2-bit codes can select is built in LDS, and each 4-bit field of
 * the packed weights reads one entry.  The int32 sums, and so Y, are the same
 * bits as bitlinear_forward's; `dbg` as there.  Needs K % 256 == 0 and
 * K <= 8192 (16.5 bytes of table per column must fit in LDS); N as
 * bitlinear_forward; no workspace.  Errors as bitlinear_forward. */
bitlinear_status bitlinear_forward_lut(const void* X, bitlinear_dtype dtype, int64_t K,
                                       int64_t N, const uint8_t* packed, const float* gamma,
                                       float* Y, bitlinear_epilogue epi,
                                       const bitlinear_debug* dbg, void* stream);


/* ---- Grouped decode forward ------------------------------------------------
 * Many independent BitLinear layers that share the token count M
 * (1..65536), run by persistent launches over the output tiles of all
 * layers.  Up to 16 tokens one launch streams the packed weights of all
 * layers back to back with skinny int8 MFMA contraction; up to 3 tokens
 * each workgroup quantizes the activations of the layers it works on itself,
 * above one more launch quantizes them first into the workspace.  Above 16
 * tokens the quantization launch is followed by one tiled int8 MFMA GEMM
 * launch whose work items are the 128x128 output tiles of all layers.  Each
 * layer's result is bit-identical to bitlinear_forward on the same
 * arguments.  Intended for decode and short prefill, where one launch per
 * layer of a few megabytes is dominated by the launch's start-up and
 * drain. */
typedef struct {
  const void* X;          /* [M][K] activations, device, 16-byte aligned */
  bitlinear_dtype dtype;  /* BITLINEAR_F32 or BITLINEAR_BF16 */
  bitlinear_epilogue epi; /* any epilogue; RELU2_GLU writes Y [M][N/2] */
  int64_t K, N;           /* N % 16 == 0, K % 256 == 0, K <= 8388608,
                             N <= 4194304; for M <= 16 also K <= 12288
                             and M * (max K + 16) + M * 2048 <= 160 KiB */
  const uint8_t* packed;  /* packed weights of this layer */
  const float* gamma;     /* gamma_c of this layer (device float) */
  float* Y;               /* [M][N] output; must not overlap any layer's input */
  const float* norm_gain; /* NULL, or subln's gain [K] (device, 16-byte aligned):
                             the layer then quantizes as
                             bitlinear_quantize_acts_rmsnorm does */
  float norm_eps;         /* subln epsilon (finite, >= 0) when norm_gain is set */
  bitlinear_weight_format format; /* layout of `packed`; 0 (2-bit) when zeroed.
                             Every layer of a group uses the same one; the
                             base-3 layout needs M <= 16 and K % 16 == 0
                             (instead of K % 256), its padded K <= 12288 */
} bitlinear_group_op;

/* Opaque host-side handle of a planned group (host memory only). */
typedef struct bitlinear_group bitlinear_group;

/* Device workspace bytes for a group of n_ops layers at M tokens (the layer
 * table, the tile schedule and, for M > 4, the quantized activations,
 * their scales and row sums).
 * Returns 0 on a bad argument; needs no GPU. */
size_t bitlinear_group_workspace_bytes(const bitlinear_group_op* ops, int n_ops, int64_t M);

/* Checks every layer, plans the tile schedule for the current device and
 * writes the layer table into `ws` with a synchronous copy (so call it
 * outside stream capture).  `ws` must hold bitlinear_group_workspace_bytes
 * bytes and must stay allocated, and the layers' buffers valid, for as long
 * as the group is used.  *out receives a handle to free with
 * bitlinear_group_destroy. */
bitlinear_status bitlinear_group_create(const bitlinear_group_op* ops, int n_ops, int64_t M,
                                        void* ws, size_t ws_bytes, bitlinear_group** out);

/* Runs every layer of the group on `stream` (one launch for M <= 3, two
 * above; capturable in a HIP graph).  Calls that overlap on one group
 * race. */
bitlinear_status bitlinear_group_forward(const bitlinear_group* g, void* stream);

/* Frees the handle (not the workspace).  NULL is allowed. */
void bitlinear_group_destroy(bitlinear_group* g);

/* Static text for a status code. */
const char* bitlinear_status_string(bitlinear_status s);

/* Thread-local detail for the last non-OK return on the calling thread
 * ("" if none).  Valid until the next library call on that thread. */
const char* bitlinear_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
