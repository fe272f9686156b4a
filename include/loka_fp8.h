/*
 * loka_fp8.h -- C ABI of liblokafp8.so: the FP8 "small GEMM followed by
 * normalization" block on AMD Instinct MI355X (gfx950).
 *
 * The block (sources, by page title and section):
 *   - "LoKA: Low-precision Kernel Applications for Recommendation Models At
 *     Scale", section I and section III-B: recommendation models are
 *     dominated by small GEMMs followed immediately by a normalization, and
 *     the LayerNorm must run in higher precision after dequantization;
 *     section III-B2 (Block-wise Normalization, Case 1): with a large batch
 *     and a small output dimension the whole output row fits in one block
 *     of the GEMM, so the normalization is fused into its epilogue;
 *     section III-B1 (No Bias): a missing bias is a first-class mode;
 *     section III-C (Dispatch): the FP8 linear is a drop-in for a standard
 *     Linear, with tensorwise / rowwise / blockwise recipes and separate
 *     forward and backward routing; unsupported sites stay in high
 *     precision.
 *   - "GEM Training: How Meta Doubled the Efficiency of Its LLM-Scale Ads
 *     Foundation Model", "Low Precision Flash Attention" and "Mixed
 *     Ultra-Low-Precision Training": MXFP8 block scales along each GEMM's K
 *     dimension, E8M0 scales derived by bit manipulation from a max-abs
 *     reduction; weights quantized once per step, separately from the
 *     activations.
 *
 * Conventions for every entry point:
 *   - All tensors are row-major and dense unless an `ld` says otherwise.
 *     bf16 tensors are passed as raw 16-bit patterns (void*).  FP8 codes are
 *     OCP e4m3 ("e4m3fn", max 448) or e5m2 (max 57344) bytes.
 *   - Every pointer is a DEVICE pointer except `loka_grouped_args::groups`
 *     (host array).  The caller allocates and owns every buffer, including
 *     the workspace; the library never allocates or frees memory and keeps
 *     no global state, so calls are thread-safe.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Nothing synchronizes the host.
 *   - Arguments are validated before anything is enqueued.  On any error
 *     nothing is enqueued and outputs are untouched.  LOKA_ERR_UNSUPPORTED
 *     marks a shape or mode combination this library does not run (the
 *     caller's cue to fall back to bf16).  A HIP launch failure returns
 *     LOKA_ERR_HIP; loka_last_error() then holds the HIP error text
 *     (thread-local).
 *   - Base pointers must be 16-byte aligned (LOKA_ERR_ALIGNMENT otherwise).
 *
 * Quantization arithmetic (identical in every entry point):
 *   tensor / row / column scaling: amax = max |x| over the group; the
 *   stored dequantization scale is s = RN32(amax / FMAX), the multiplier
 *   r = RN32(FMAX / amax) (saturating at the largest fp32), amax == 0 gives
 *   s = r = 1; code = satRNE_fp8(RN32(x * r)): round to nearest even, values
 *   past +-FMAX clamp to the +-FMAX code, -0 encodes as 0x80.
 *   MX32: one E8M0 scale per 32 consecutive elements,
 *   e = clamp(floor(log2 amax) - emax_elem, -127, 127) with emax_elem 8
 *   (e4m3) / 15 (e5m2), stored as e + 127 (amax == 0 -> 0);
 *   code = satRNE_fp8(x * 2^-e).
 *   Non-finite inputs are outside the contract (results unspecified).
 */
#ifndef LOKA_FP8_H
#define LOKA_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOKA_ABI_VERSION 3

typedef enum {
  LOKA_OK = 0,
  LOKA_ERR_INVALID_ARG = 1, /* null required pointer, negative size, bad enum */
  LOKA_ERR_UNSUPPORTED = 2, /* valid request this library does not run      */
  LOKA_ERR_ALIGNMENT = 3,   /* a base pointer is not 16-byte aligned        */
  LOKA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required   */
  LOKA_ERR_HIP = 5          /* a HIP call failed; see loka_last_error()     */
} loka_status;

typedef enum { LOKA_E4M3 = 0, LOKA_E5M2 = 1 } loka_fp8_fmt;

typedef enum {
  LOKA_SCALE_TENSOR = 0,  /* one fp32 scale for the whole array                 */
  LOKA_SCALE_ROW = 1,     /* one fp32 scale per row (amax along the row)        */
  LOKA_SCALE_COL = 2,     /* one fp32 scale per column (amax down the column)   */
  LOKA_SCALE_MX32_ROW = 3,/* one E8M0 per 32 consecutive elements along a row   */
  LOKA_SCALE_MX32_COL = 4,/* one E8M0 per 32 consecutive elements down a column */
  LOKA_SCALE_MX32_SQ = 5  /* one E8M0 per 32 x 32 block (rows and columns)      */
} loka_scaling;

typedef enum { LOKA_DTYPE_BF16 = 0, LOKA_DTYPE_F32 = 1 } loka_dtype;

/* ------------------------------------------------------------------------
 * loka_quant_fp8: amax -> scale -> saturating RNE cast of a 2-D array.
 *
 * Source: LoKA section II-C (quantization overhead is a first-order cost
 * of the FP8 linear) and section III-C (tensorwise / rowwise / blockwise
 * recipes); GEM "Low Precision Flash Attention" (MX block scales along K,
 * E8M0 by bit manipulation) and "Mixed Ultra-Low-Precision Training"
 * (weights quantized separately from activations).
 *
 *   src      [rows, cols] with row stride `ld` elements (ld >= cols),
 *            bf16 or fp32 (src_dtype).
 *   codes    transpose_out == 0: [rows, cols] (row stride cols);
 *            transpose_out == 1: [cols, rows] (row stride rows): the
 *            codes of src^T, with `rows` contiguous -- the MFMA operand
 *            layout when `rows` is the caller's contraction dimension (a
 *            weight W[K, N] for the forward, X or dZ for the wgrad);
 *            transpose_out == 2: the codes of src^T in the fragment-
 *            interleaved ("packed") layout, cols * ceil(rows/128)*128
 *            bytes: for every 16 consecutive columns j0..j0+15 of src and
 *            every 128-row chunk c (rows past `rows` are zero codes) one
 *            2 KiB block at ((j0/16) * ceil(rows/128) + c) * 2048, whose
 *            byte 256 p + 16 i + b is src^T[j0 + i][128 c + 16 p + b]
 *            (p = 0..7, i = 0..15, b = 0..15).  Lane l = i + 16 g of a
 *            64-wide MFMA fragment load then reads bytes 16 l of each
 *            1 KiB half: the weight layout loka_gemm_fp8_ln and the
 *            grouped launch read with LOKA_FWD_W_PACKED;
 *            transpose_out == 3: the codes of src itself (not transposed)
 *            in the same layout, rows * ceil(cols/128)*128 bytes: for
 *            every 16 consecutive rows i0..i0+15 and 128-column chunk c
 *            (columns past `cols` are zero codes) one 2 KiB block at
 *            ((i0/16) * ceil(cols/128) + c) * 2048, whose byte
 *            256 p + 16 i + b is src[i0 + i][128 c + 16 p + b] -- the dgrad
 *            weight layout loka_gemm_fp8_bwd reads with LOKA_BWD_W_PACKED.
 *   scales   TENSOR: float[1]; ROW: float[rows]; COL: float[cols];
 *            MX32_ROW: uint8[rows][cols/32]; MX32_COL: uint8[cols][rows/32];
 *            MX32_SQ: uint8[rows/32][cols/32], the block (i, j) covering
 *            rows 32i..32i+31 and columns 32j..32j+31 (GEM "Low Precision
 *            Flash Attention", Block-wise Quantization: the square block is
 *            transpose-invariant, so one quantization serves a tensor and its
 *            transpose; the codes of src^T are transpose_out's bytes and
 *            the scales of src^T are the transposed grid).
 *            (The scale layout does not depend on transpose_out.)
 *   amax     optional float out, same count as the fp32 scales
 *            (TENSOR/ROW/COL only; must be NULL for MX).
 *   workspace device scratch of loka_quant_workspace_size() bytes
 *            (may be NULL when that size is 0).
 * Requirements: rows, cols >= 0; cols % 16 == 0; MX32_ROW: cols % 32 == 0;
 * MX32_COL: rows % 32 == 0; MX32_SQ: rows % 32 == 0 and cols % 32 == 0;
 * transpose_out 1, 2 and 3 require rows % 16 == 0.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t rows, cols, ld;
  int32_t src_dtype;     /* loka_dtype   */
  int32_t fmt;           /* loka_fp8_fmt */
  int32_t mode;          /* loka_scaling */
  int32_t transpose_out; /* 0, 1, 2 or 3 */
  const void* src;
  uint8_t* codes;
  void* scales;
  float* amax;
  void* workspace;
  size_t workspace_bytes;
} loka_quant_args;

size_t loka_quant_workspace_size(const loka_quant_args* args);
loka_status loka_quant_fp8(const loka_quant_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_gemm_fp8_ln: Y = LayerNorm(dequant(q(X) . q(W)) + bias), fused.
 *
 * Source: LoKA section III-B2 (normalization fused into the GEMM epilogue
 * while the output tile is on chip; Case 1, the whole row in one block),
 * section III-B (dequantize before the LayerNorm, which runs in high
 * precision), section III-B1 (No Bias); GEM "Mixed Ultra-Low-Precision
 * Training" (activation quantization fused into the neighbouring kernel
 * instead of a separate pass).
 *
 *   X       bf16 [M, K]; quantized inside the kernel per x_mode, e4m3.
 *   qw, sw  the weight, quantized beforehand with loka_quant_fp8 on
 *           W [K, N] with transpose_out = 1 (codes [N, K], e4m3), or with
 *           transpose_out = 2 (the packed layout) and flags
 *           LOKA_FWD_W_PACKED:
 *             x_mode TENSOR   -> W mode TENSOR,  sw float[1]
 *             x_mode ROW      -> W mode COL,     sw float[N]
 *             x_mode MX32_ROW -> W mode MX32_COL, sw uint8[N][K/32]
 *             x_mode MX32_SQ  -> W mode MX32_SQ,  sw uint8[K/32][N/32]
 *   x_mode MX32_SQ (GEM "Low Precision Flash Attention", Block-wise
 *           Quantization, with activation quantization fused into the
 *           producer, GEM "Mixed Ultra-Low-Precision Training"): X arrives
 *           quantized -- x holds its e4m3 codes [M, K] and x_scales its
 *           E8M0 scales uint8[M/32][K/32], as loka_quant_fp8 (MX32_SQ,
 *           transpose_out 0) writes them -- and the same codes serve the
 *           backward.  Needs M % 32 == 0, the weight-resident shapes and
 *           qx_out = sx_out = NULL; x_scales must be NULL in other modes.
 *   y_codes, y_scales (optional, together; LayerNorm epilogue, any x_mode):
 *           Y also leaves quantized in 32 x 32 blocks -- the next layer's
 *           MX32_SQ input, with the activation quantization fused into the
 *           normalization that produces it (GEM "Handling Quantization
 *           Overhead", PreNorm fusion).  The codes and scales equal
 *           loka_quant_fp8(Y, e4m3, MX32_SQ) of the bf16 Y.  Needs N = 256 or
 *           512, the weight-resident shapes and M % 32 == 0.
 *   bias, gamma, beta  bf16 [N] or NULL (NULL = 0, 1, 0; NULL bias is the
 *           No-Bias mode).
 *   Z[m,n]  = acc[m,n] * s_x[m] * s_w[n] + bias[n]   (MX: the E8M0 scales
 *           multiply each 32-wide K block inside the MFMA), acc the fp32
 *           FP8 MFMA sum.
 *   Y       = gamma * (Z - mean_n Z) / sqrt(var_n Z + eps) + beta, bf16 RNE
 *           (population variance, two-pass, fp32).
 *   Optional outputs (NULL to skip): z fp32 [M, N]; mean, rstd fp32 [M];
 *   qx_out e4m3 [M, K] and sx_out (float[1] | float[M] | uint8[M][K/32]):
 *   the quantized X, bit-identical to loka_quant_fp8's, for the backward.
 *   workspace: loka_gemm_fp8_ln_workspace_size() bytes: the TENSOR amax
 *   partials and, for a row-major qw on the weight-resident shapes (N <=
 *   512, K <= 1024 / 640 / 512 for N <= 256 / 384 / 512), the weight
 *   rearranged into the packed layout (one extra pass over qw per call;
 *   LOKA_FWD_W_PACKED avoids it).  0 when neither applies.
 *   flags: LOKA_FWD_W_PACKED (qw in the packed layout; only on the
 *   weight-resident shapes or with BlockNorm, LOKA_ERR_UNSUPPORTED
 *   otherwise) and/or LOKA_FWD_BLOCKNORM_HSWISH (below), or 0.
 * Requirements: M >= 0; N % 64 == 0 and 64 <= N <= 1024 (else
 * UNSUPPORTED: the row must fit one workgroup); K % 16 == 0 (MX: % 32),
 * 16 <= K <= 2048.
 * ---------------------------------------------------------------------- */
#define LOKA_FWD_W_PACKED 1 /* qw is in loka_quant_fp8's transpose_out = 2 layout */
/* BlockNorm + Hard Swish epilogue instead of LayerNorm: LoKA section III-B2
 * (Block-wise Normalization, Fig. 7d) and III-B3 (Hard Swish):
 *   Y = h(Z / sqrt(mean_b Z^2 + eps)) over blocks b of 256 consecutive
 *   columns, h(t) = t * min(max(t + 3, 0), 6) / 6, Z as above (bias
 *   optional), no affine parameters, bf16 RNE.
 * Requirements: x_mode ROW; gamma, beta, mean and rstd NULL; N % 256 == 0,
 * 256 <= N <= 8192; 16 <= K <= 1024, K % 16 == 0.  The row does not have to
 * fit one workgroup: N is processed as independent slabs of 512 columns
 * (N % 512 == 0 and K <= 512) or else 256 columns.  Optional z, qx_out and
 * sx_out as for LayerNorm. */
#define LOKA_FWD_BLOCKNORM_HSWISH 2
typedef struct {
  int64_t M, N, K;
  int32_t x_mode; /* LOKA_SCALE_TENSOR, LOKA_SCALE_ROW, LOKA_SCALE_MX32_ROW or LOKA_SCALE_MX32_SQ */
  int32_t flags;  /* LOKA_FWD_W_PACKED | LOKA_FWD_BLOCKNORM_HSWISH, or 0 */
  float eps;
  const void* x;
  const uint8_t* qw;
  const void* sw;
  const void* bias;
  const void* gamma;
  const void* beta;
  void* y;
  float* z;
  float* mean;
  float* rstd;
  uint8_t* qx_out;
  void* sx_out;
  void* workspace;
  size_t workspace_bytes;
  const uint8_t* x_scales; /* MX32_SQ only: X's E8M0 scales [M/32][K/32] */
  uint8_t* y_codes;        /* optional (with y_scales): Y in 32 x 32 blocks, e4m3 [M, N] */
  uint8_t* y_scales;       /* optional (with y_codes): their E8M0 scales [M/32][N/32] */
} loka_fwd_args;

size_t loka_gemm_fp8_ln_workspace_size(const loka_fwd_args* args);
loka_status loka_gemm_fp8_ln(const loka_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_gemm_fp8_ln_noalloc: loka_gemm_fp8_ln for callers that cannot
 * allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same arguments and results
 * (the same kernels, bit-identical outputs), except that `workspace` and
 * `workspace_bytes` are ignored: the workspace lives in a fixed device
 * array of LOKA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends.  Neither the call nor the library allocates
 * or frees device memory.
 *   - A call whose loka_gemm_fp8_ln_workspace_size() exceeds
 *     LOKA_NOALLOC_SCRATCH_BYTES returns LOKA_ERR_UNSUPPORTED (every
 *     LayerNorm-epilogue shape fits; a row-major weight for BlockNorm with
 *     N * K above about 1 MiB does not -- pass LOKA_FWD_W_PACKED).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other host threads) race and must be
 *     serialized by the caller.  No state carries from one call to the next.
 *   - The first call on a device looks the array's device address up
 *     (hipGetSymbolAddress) with that device current; make it before any
 *     graph capture.  `stream` must belong to the current device
 *     (LOKA_ERR_HIP otherwise).
 * ---------------------------------------------------------------------- */
#define LOKA_NOALLOC_SCRATCH_BYTES (1u << 20)
loka_status loka_gemm_fp8_ln_noalloc(const loka_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_gemm_fp8_bwd: the backward of loka_gemm_fp8_ln (x_mode ROW).
 *
 * Source: LoKA section III-C (Trainer Integration: a custom autograd
 * function routes forward and backward separately; rowwise recipes, with
 * Table VI's RW recipe for the gradients); GEM "Mixed Ultra-Low-Precision
 * Training" (gradients in the e5m2 range, scales along each GEMM's own
 * contraction dimension).
 *
 * dY is the gradient at Y.  Per row, with yhat = (Z - mean) * rstd and
 * g = dY * gamma:
 *   dZ     = rstd * (g - mean_n g - yhat * mean_n(g * yhat))   (fp32)
 *   dgamma = sum_m dY * yhat,  dbeta = sum_m dY,  dbias = sum_m dZ
 *   dgrad: dX = dequant(q_row(dZ, e5m2) . q_row(W, e4m3)^T)   bf16 [M, K]
 *          (W's rows are its k index: scales per k, amax over n)
 *   wgrad: dW = dequant(q_col(X, e4m3)^T . q_col(dZ, e5m2))   fp32 [K, N]
 *          (scales per column of X and of dZ, amax over the M rows)
 * With flags & LOKA_BWD_NO_LN, dY already is dZ (no LayerNorm); mean,
 * rstd, gamma, qx, sx, qw, sw, bias are then unused and may be NULL, and
 * dgamma/dbeta must be NULL.
 *
 *   ctx from the forward: qx e4m3 [M, K] + sx float[M] (its qx_out/sx_out),
 *     mean, rstd float[M], qw [N, K] + sw float[N] (its weight), bias and
 *     gamma bf16 [N] or NULL.  Z is recomputed from qx, qw in the kernel.
 *   x       bf16 [M, K] (column-quantized here for wgrad).
 *   qw_row, sw_row: W [K, N] quantized with loka_quant_fp8 mode ROW, e4m3,
 *     transpose_out 0 (codes [K, N], scales float[K]).
 *   Outputs: dx bf16 [M, K]; dw fp32 [K, N]; dgamma, dbeta, dbias fp32 [N]
 *     or NULL; optional dz fp32 [M, N]; optional dz_codes e5m2 [M, N] and
 *     dz_scales float[M] (the dgrad operand, for parity checks).
 *   All reductions over M are deterministic (fixed-order two-stage sums).
 * Requirements: as loka_gemm_fp8_ln with x_mode ROW, plus K % 64 == 0,
 *   K <= 1024 and M % 16 == 0.
 *
 * With flags & LOKA_BWD_MX32_SQ, the backward of the square-block forward
 * (x_mode MX32_SQ; GEM "Low Precision Flash Attention", Block-wise
 * Quantization: 32 x 32 blocks are transpose-invariant, so each tensor is
 * quantized once and serves every GEMM that reads it):
 *   qx, sx   X's codes [M, K] and E8M0 scales uint8[M/32][K/32] (the
 *            forward's input, read transposed by the wgrad);
 *   qw, sw   W's codes [N, K] (transpose_out 1) and scales uint8[K/32][N/32]
 *            (read as they are for Z, transposed for the dgrad);
 *   dZ is quantized once, e5m2 in 32 x 32 blocks:
 *     dX = dequant(q(dZ)) . dequant(q(W))^T,  dW = dequant(q(X))^T . dequant(q(dZ));
 *   x, qw_row and sw_row are unused (may be NULL); dz_scales, if given,
 *   receives dZ's scales uint8[M/32][N/32].  Needs M % 32 == 0, N <= 512
 *   and K <= 512; mean and rstd unless LOKA_BWD_NO_LN.
 *
 * With flags & LOKA_BWD_W_PACKED both weights arrive in the
 * fragment-interleaved layout instead of row-major, so no rearrangement
 * runs inside the call: qw as loka_quant_fp8 (COL, transpose_out 2) writes
 * it for W [K, N] (the forward's packed weight, N * ceil(K/128)*128
 * bytes), qw_row as loka_quant_fp8 (ROW, transpose_out 3) writes it
 * (K * ceil(N/128)*128 bytes).  With LOKA_BWD_MX32_SQ the same two layouts
 * come from MX32_SQ quantizations of W (transpose_out 2 for qw, 3 for
 * qw_row, which is then required); sw stays the [K/32][N/32] block grid,
 * and sw_row is unused.  The results are bit-identical to the row-major
 * call.
 *
 * Optional outputs of the ROW recipe (each may be NULL; must be NULL with
 * LOKA_BWD_MX32_SQ): the wgrad's two operands, exactly as
 * loka_quant_fp8 (COL, transpose_out 2) would write them --
 *   xc_codes   e4m3 codes of X quantized per column (amax over the M rows),
 *              packed layout of X^T, K * ceil(M/128)*128 bytes;
 *   xc_scales  float[K];
 *   dzc_codes  e5m2 codes of the fp32 dZ quantized per column, packed
 *              layout of dZ^T, N * ceil(M/128)*128 bytes;
 *   dzc_scales float[N].
 * ---------------------------------------------------------------------- */
#define LOKA_BWD_NO_LN 1
#define LOKA_BWD_MX32_SQ 2
#define LOKA_BWD_W_PACKED 4

typedef struct {
  int64_t M, N, K;
  int32_t flags;
  int32_t reserved;
  const void* dy;
  const uint8_t* qx;
  const void* sx; /* float[M] (ROW) or uint8[M/32][K/32] (MX32_SQ) */
  const float* mean;
  const float* rstd;
  const uint8_t* qw;
  const void* sw; /* float[N] (ROW) or uint8[K/32][N/32] (MX32_SQ) */
  const void* bias;
  const void* gamma;
  const void* x;
  const uint8_t* qw_row;
  const float* sw_row;
  void* dx;
  float* dw;
  float* dgamma;
  float* dbeta;
  float* dbias;
  float* dz;
  uint8_t* dz_codes;
  void* dz_scales; /* float[M] (ROW) or uint8[M/32][N/32] (MX32_SQ) */
  void* workspace;
  size_t workspace_bytes;
  uint8_t* xc_codes;
  float* xc_scales;
  uint8_t* dzc_codes;
  float* dzc_scales;
} loka_bwd_args;

size_t loka_gemm_fp8_bwd_workspace_size(const loka_bwd_args* args);
loka_status loka_gemm_fp8_bwd(const loka_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_grouped_gemm_fp8_ln: many independent loka_gemm_fp8_ln problems
 * (x_mode ROW) in one call: one persistent launch when every group has
 * N <= 384 and K <= 512 and a guarded shape, else one per register shape
 * class of the groups (column tiles per wavefront, ceil(N/128), and K depth).
 *
 * Source: LoKA section I (wide ensembles of small layers); GEM
 * "Generalized Dot-Product Attention" (tile lists precomputed on the CPU,
 * empty tiles skipped) and "Expert Parallelism" (one expert per rank).
 *
 *   groups  HOST array of num_groups descriptors; each is one forward with
 *           the same meaning and requirements as loka_fwd_args (x_mode
 *           ROW): x bf16 [M,K], qw [N,K] + sw float[N] from
 *           loka_quant_fp8(COL, transpose_out=1) (or every group's qw in
 *           the packed layout of transpose_out=2, with flags
 *           LOKA_FWD_W_PACKED), bias/gamma/beta bf16 [N] or NULL, y bf16
 *           [M,N], optional z fp32 [M,N].
 *   workspace device memory of loka_grouped_workspace_size() bytes: the
 *           library copies the descriptors and the tile table into it with
 *           an asynchronous host-to-device copy on `stream`, so it must not
 *           be reused until the launch has completed.
 *   The workspace also receives the launch plan (each group's first tile
 *   and each workgroup's share) when it is computed on the device from the
 *   copied descriptors, and without LOKA_FWD_W_PACKED every group's weight
 *   rearranged into the packed layout (at a fixed stride: the largest
 *   group's N * ceil(K/128) * 128 bytes).  For graph capture the host array must stay valid and
 *   unchanged for every replay.
 * Each group's output is bit-identical to a single loka_gemm_fp8_ln call
 * with the same inputs.  Requirements: as loka_gemm_fp8_ln, with
 * num_groups <= 2048 and every group's weight small enough to stay in
 * registers: N <= 512 and K <= 1024 (N <= 256), 640 (N <= 384) or 512
 * (N <= 512); LOKA_ERR_UNSUPPORTED otherwise (run such groups as single
 * calls).
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t M, N, K;
  const void* x;
  const uint8_t* qw;
  const float* sw;
  const void* bias;
  const void* gamma;
  const void* beta;
  void* y;
  float* z;
} loka_group_desc;

typedef struct {
  int32_t num_groups;
  int32_t x_mode; /* LOKA_SCALE_ROW */
  float eps;
  int32_t flags;  /* 0 or LOKA_FWD_W_PACKED */
  const loka_group_desc* groups;
  void* workspace;
  size_t workspace_bytes;
} loka_grouped_args;

size_t loka_grouped_workspace_size(const loka_grouped_args* args);
loka_status loka_grouped_gemm_fp8_ln(const loka_grouped_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_mere_z: the error of a candidate recipe's linear-layer output against
 * the high-precision reference, on sampled rows.
 *
 * Source: LoKA section II-C ("Error Analysis": the mean element-wise
 * relative error, MERE, of a low-precision linear layer against a higher
 * precision) and section III-C ("Library and Recipe Selection": Dispatch
 * filters candidates by MERE).
 *
 *   x     bf16 [M, K], w bf16 [K, N] (the unquantized operands), bias bf16
 *         [N] or NULL;
 *   z     the candidate's output Z = dequant(q(X) q(W)) + bias, fp32 [M, N]
 *         (loka_gemm_fp8_ln's optional z output);
 *   rows  DEVICE int64 [S]: the sampled row indices;
 *   out   DEVICE double[3]: MERE = mean over the sampled rows' entries with
 *         z_ref != 0 of |z - z_ref| / |z_ref|; the count of those entries;
 *         the count of row indices outside [0, M) (those rows contribute
 *         nothing: a caller checks out[2] == 0).
 * z_ref = X W + b is computed here in fp32 (exact bf16 products, summed in
 * k order).  Sums are in a fixed order: the result is deterministic.
 * workspace: loka_mere_workspace_size() bytes (24 S).
 * Requirements: M, N, K >= 1, K <= 2048, N <= 8192, S >= 1.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t M, N, K, S;
  const void* x;
  const void* w;
  const void* bias;
  const float* z;
  const int64_t* rows;
  double* out;
  void* workspace;
  size_t workspace_bytes;
} loka_mere_args;

size_t loka_mere_workspace_size(const loka_mere_args* args);
loka_status loka_mere_z(const loka_mere_args* args, void* stream);

/* ------------------------------------------------------------------------
 * loka_dispatch_select: the Dispatch runtime's choice among measured
 * candidate recipes for one operation (host only; no GPU work).
 *
 * Source: LoKA section III-C ("Library and Recipe Selection"): candidates
 * are filtered by accuracy (MERE below a conservative threshold, typically
 * 0.2) and by speed (speedup above a minimum factor, typically 1.05x), and
 * the one with the highest measured throughput is chosen.
 *
 *   cands        HOST array of n {time in us, MERE} (n >= 0);
 *   baseline_us  the high-precision path's time (> 0): speedup = baseline_us / us;
 *   mere_max, min_speedup  the thresholds (> 0); both tests are strict;
 *   choice       out: the index of the shortest time among the candidates
 *                that pass both filters (the earlier one on equal times),
 *                or -1 when none does (keep the high-precision path).
 * Candidates with a non-finite MERE or time, or a time <= 0, never pass.
 * ---------------------------------------------------------------------- */
typedef struct {
  double us;
  double mere;
} loka_dispatch_candidate;

loka_status loka_dispatch_select(const loka_dispatch_candidate* cands, int32_t n, double baseline_us,
                                 double mere_max, double min_speedup, int32_t* choice);

/* ------------------------------------------------------------------------
 * The Probe's statistics (LoKA section III-A1, "Online Distribution
 * Learning" and "Sampling learned distributions"), on the device.  fp32
 * throughout; every reduction runs in a fixed order (deterministic).
 * Shapes: 1 <= K, R, C <= 2048; B >= 1.  All pointers are device pointers
 * unless marked HOST; workspace as returned by the _workspace_size call.
 *
 * loka_probe_input_update: merge a batch T bf16 [B, K] of a layer's input
 *   into (n_old, mu fp32 [K], S fp32 [K, K]) in place, S the unnormalized
 *   scatter (Chan, Golub and LeVeque's pairwise update, as the pages give it):
 *     n' = n_old + B, d = mean(T) - mu, mu += (B / n') d,
 *     S += (T - mean T)^T (T - mean T) + (n_old B / n') d d^T.
 *   The caller keeps n (add B after the call); the covariance is S / (n - 1).
 *
 * loka_probe_weight_update: the matrix-normal Kronecker flip-flop with an
 *   EMA of momentum m for W bf16 [R, C] ~ MN(M, U, V), state M fp32 [R, C],
 *   U fp32 [R, R], V fp32 [C, C] in place.  first != 0 initializes
 *   (M = W, U = I, V = I).  Otherwise, with eps = 1e-6 trace(A) / dim(A):
 *     M <- m M + (1 - m) W, Wc = W - M,
 *     L_V L_V^T = V + eps I, Wt = Wc L_V^-T, U1 = Wt Wt^T / C,
 *     L_U L_U^T = U + eps I, Wu = L_U^-1 Wc, V1 = Wu^T Wu / R
 *     (both factors from the state before the update; linear solves, no
 *     inverses), U'' = m U + (1 - m) U1, V'' = m V + (1 - m) V1,
 *     U <- (U'' + U''^T) / 2 + eps'' I, V <- (V'' + V''^T) / 2 + eps'' I
 *     (eps'' = 1e-6 trace(U'') / R, resp. 1e-6 trace(V'') / C),
 *     s = trace(U) / R, U <- U / s, V <- s V.
 *   info: device int[2], the Cholesky status of V and U (0, or the 1-based
 *   column of a non-positive pivot, after which the state is not valid).
 *
 * loka_probe_sample_input: T' = 1 mu^T + Z L^T, L L^T = S / (n - 1) + eps I,
 *   out bf16 [B, K]; info int[1].
 * loka_probe_sample_weight: W' = M + L_U Z L_V^T, out bf16 [R, C]; info int[2].
 *   Z is standard normal: Philox4x64-10 (Salmon et al., SC'11) block i with
 *   counter (i, 0, 0, 0) and key (seed, 0); each 64-bit output w gives the
 *   uniform (w >> 11) 2^-53, pairs (u1, u2) the Box-Muller normals
 *   sqrt(-2 ln(1 - u1)) (cos 2 pi u2, sin 2 pi u2), in row-major order.
 * ---------------------------------------------------------------------- */
typedef struct {
  int64_t B, K, n_old;
  const void* T;
  float* mu;
  float* S;
  void* workspace;
  size_t workspace_bytes;
} loka_probe_input_args;

typedef struct {
  int64_t R, C;
  float m;
  int32_t first;
  const void* W;
  float* M;
  float* U;
  float* V;
  int32_t* info;
  void* workspace;
  size_t workspace_bytes;
} loka_probe_weight_args;

typedef struct {
  int64_t B, K, n;
  const float* mu;
  const float* S;
  uint64_t seed;
  void* out;
  int32_t* info;
  void* workspace;
  size_t workspace_bytes;
} loka_probe_sample_input_args;

typedef struct {
  int64_t R, C;
  const float* M;
  const float* U;
  const float* V;
  uint64_t seed;
  void* out;
  int32_t* info;
  void* workspace;
  size_t workspace_bytes;
} loka_probe_sample_weight_args;

size_t loka_probe_input_workspace_size(const loka_probe_input_args* args);
loka_status loka_probe_input_update(const loka_probe_input_args* args, void* stream);
size_t loka_probe_weight_workspace_size(const loka_probe_weight_args* args);
loka_status loka_probe_weight_update(const loka_probe_weight_args* args, void* stream);
size_t loka_probe_sample_input_workspace_size(const loka_probe_sample_input_args* args);
loka_status loka_probe_sample_input(const loka_probe_sample_input_args* args, void* stream);
size_t loka_probe_sample_weight_workspace_size(const loka_probe_sample_weight_args* args);
loka_status loka_probe_sample_weight(const loka_probe_sample_weight_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Helpers.
 * ---------------------------------------------------------------------- */
const char* loka_status_string(loka_status s); /* static text, never NULL */
const char* loka_last_error(void);            /* thread-local detail of the last failing call */
int loka_abi_version(void);                   /* LOKA_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* LOKA_FP8_H */
