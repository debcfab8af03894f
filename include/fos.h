/*
 * fos.h -- C ABI of the Four Over Six (4/6) NVFP4 library for AMD MI355X (gfx950).
 *
 * Method (Four Over Six documentation page, Hugging Face transformers docs,
 * section "Four Over Six"): every NVFP4 block is scaled adaptively so that its
 * largest magnitude maps either to 6 or to 4, whichever gives the lower quantization
 * error; the options listed there are a random Hadamard transform, 2D block scaling,
 * transposed inputs and stochastic rounding.  Format (Ultralytics glossary "FP4",
 * section "How FP4 works"): 16 E2M1 values share one FP8 E4M3 scale, and the tensor
 * carries a second FP32 scale.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or keeps a pointer after returning.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: the status reports argument validation and
 *     launch errors only; faults in the kernels surface at the caller's next sync.
 *   - Validation runs before any HIP call; a non-FOS_OK status means nothing was
 *     launched and no output was touched.
 *   - Tensors are row-major and contiguous.  Element (r, c) of a [rows, cols] bf16
 *     tensor is at byte offset 2*(r*cols + c).
 *   - Inputs must be finite; NaN or Inf inputs give unspecified outputs.
 *   - Calls are thread-safe; calls that may run concurrently (different streams)
 *     must not share a workspace.
 *
 * NVFP4 record layout (one orientation):
 *   data   [R][C/2] bytes: byte k of a row holds element 2k in its low nibble and
 *          element 2k+1 in its high nibble; a nibble is sign<<3 | magnitude code,
 *          codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6 (E2M1, exponent bias 1).
 *   scales [R][C/16] bytes: OCP E4M3 ("FN", bias 7, max 448) block scales.
 *   t      one fp32 per tensor, decode direction: value = E2M1 * (E4M3 * t).
 * Row-wise output: R = rows, C = cols (16-blocks along a row).
 * Column-wise output ("transposed inputs"): the quantization of X^T: R = cols,
 * C = rows (16-blocks of 16 consecutive rows of one column of X).
 */
#ifndef FOS_H
#define FOS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FOS_ABI_VERSION 2

typedef enum {
  FOS_OK = 0,
  FOS_E_NULL = 1,      /* a required pointer is NULL                                */
  FOS_E_SHAPE = 2,     /* negative size, a size that must be a multiple of 16 (or
                          of 32, 64, 256 where stated) is not, a dimension of 2^31
                          or more, more than 2^40 elements in one tensor, or a
                          shape whose launch would need more than 2^32 - 1
                          work-items (e.g. 2D blocks on a [2^29, 16] tensor)       */
  FOS_E_ALIGN = 3,     /* bf16 input not 16-byte aligned, packed data not 8-byte
                          aligned, or an output buffer misaligned                   */
  FOS_E_FLAGS = 4,     /* unknown enum value, wrong struct_size, or an unsupported
                          option combination (e.g. Hadamard with 2D blocks)         */
  FOS_E_WORKSPACE = 5, /* workspace NULL, not 16-byte aligned, or smaller than
                          fos_workspace_bytes() (fos_qlinear_fwd_act: not 256-byte
                          aligned, or smaller than
                          fos_qlinear_act_workspace_bytes(M, K))                   */
  FOS_E_HIP = 6        /* a HIP launch failed                                        */
} fos_status;

/* Block-scale rule.  FOS_RULE_4OVER6: per block, keep the candidate (block max ->
 * 6, or block max -> 4) with the lower squared error; ties go to 6.
 * FOS_RULE_6ONLY: standard NVFP4, block max -> 6 (Ultralytics glossary "FP4",
 * "How FP4 works"). */
enum { FOS_RULE_4OVER6 = 0, FOS_RULE_6ONLY = 1 };
/* E2M1 rounding: nearest-even, or stochastic (one Philox4x32-10 draw per block,
 * 8 random bits per element; the pages list stochastic rounding as an option and
 * the FP4 glossary's training section uses it for gradients).  With 8-bit draws a
 * value at fractional position p between its two grid neighbours rounds up with
 * chance n/256, n = number of draw bytes k with (k + 0.5)/256 < p (p taken to 22
 * fractional bits): p <= 1/512 never rounds up, p > 511/512 always does, and the
 * expected result is off by at most 2^-9 of the grid step (plus 2^-22). */
enum { FOS_ROUND_RNE = 0, FOS_ROUND_STOCHASTIC = 1, FOS_ROUND_STOCHASTIC_FULL = 2 };
/* FOS_ROUND_STOCHASTIC_FULL: stochastic rounding with a whole 32-bit Philox4x32-10
 * word per element (four calls per block; element i of block b takes word i % 4 of
 * the call with counter (b_lo, b_hi, i / 4, stream)): with u = word >> 10 and P = p's
 * first 22 fractional bits as an integer, the value rounds up iff P + u >= 2^22, a
 * chance of p to within 2^-22 and no dead zone near the grid points. */
/* 1D: 16 consecutive values share a scale.  2D: a 16x16 tile shares one scale and
 * one 4-vs-6 decision; its byte is written into all 16 row-block slots of the tile
 * (the 1D scale layout is kept). */
enum { FOS_BLOCK_1D = 0, FOS_BLOCK_2D = 1 };
/* Output orientations (bitmask; at least one). */
enum { FOS_OUT_ROWWISE = 1, FOS_OUT_COLWISE = 2 };
/* Dequantize output element type. */
enum { FOS_OUT_F32 = 0, FOS_OUT_BF16 = 1 };

typedef struct {
  uint32_t struct_size;   /* must equal sizeof(fos_quant_config)                    */
  uint32_t rule;          /* FOS_RULE_*                                             */
  uint32_t rounding;      /* FOS_ROUND_*                                            */
  uint32_t block;         /* FOS_BLOCK_*                                            */
  uint32_t outputs;       /* FOS_OUT_ROWWISE | FOS_OUT_COLWISE                      */
  uint32_t hadamard;      /* 0, or 1 = random-sign 16-point Hadamard transform of
                             every 1D block before quantization (one orientation
                             only; not with 2D)                                      */
  uint64_t hadamard_seed; /* Philox key for the 16 signs                            */
  uint64_t sr_seed;       /* Philox key for stochastic rounding                     */
} fos_quant_config;       /* host struct, read only during the call                 */

/* ABI version of the loaded library (FOS_ABI_VERSION). */
int fos_abi_version(void);

/* Human-readable name of a status (static string, never NULL). */
const char* fos_status_string(fos_status status);

/* Bytes of device workspace that fos_tensor_scale / fos_quantize need (scratch for
 * the per-workgroup partial maxima of the tensor-scale pass, 16-byte aligned; its
 * contents on entry are ignored, and it must stay untouched until the call's
 * kernels have run).  The per-tensor FP32 scale that the pass computes is the
 * second-level scale of NVFP4 (Ultralytics glossary "FP4", "How FP4 works").
 * The size does not depend on the tensor: 4096 bytes. */
size_t fos_quantize_workspace_bytes(void);

/* The same value as fos_quantize_workspace_bytes (earlier name, kept). */
size_t fos_workspace_bytes(void);

/* Per-tensor scale.  Writes t = RN_fp32(A / 2688) to *tensor_scale (device fp32),
 * where A = max |x| over the tensor -- over the transformed values when
 * cfg->hadamard is set, in the orientation of the single requested output -- and
 * 2688 = 448 * 6 (largest E4M3 value times largest E2M1 value).  The pages give
 * only "a second per-tensor FP32 scale" (Ultralytics glossary "FP4", "How FP4
 * works"); the constant is this library's reading.
 *   x: bf16 [rows][cols], 16-byte aligned.  rows, cols >= 0; cols % 16 == 0;
 *      rows % 16 == 0 when cfg requests a column-wise Hadamard transform.
 *   An empty tensor gives t = 0.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_WORKSPACE,
 * FOS_E_HIP. */
fos_status fos_tensor_scale(const fos_quant_config* cfg, const void* x, int64_t rows,
                            int64_t cols, float* tensor_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/* 4/6 quantization given the tensor scale (device fp32, e.g. from
 * fos_tensor_scale, or the all-reduced maximum of per-shard scales).
 * Per 16-value block (Four Over Six documentation page, "Four Over Six"): the
 * block's E4M3 scale maps its largest magnitude to 6 or to 4, the candidate with
 * the lower squared error of the dequantized block is kept (ties go to 6;
 * FOS_RULE_6ONLY keeps 6), and the values are rounded onto the E2M1 grid under it.
 * The record is NVFP4's (Ultralytics glossary "FP4", "How FP4 works": 16 E2M1 values
 * per E4M3 scale, one FP32 scale per tensor); the options (2D blocks, transposed
 * output, Hadamard transform, stochastic rounding) are the page's list.
 *   row_data [rows][cols/2], row_scales [rows][cols/16]: required iff
 *     cfg->outputs has FOS_OUT_ROWWISE, else ignored.  row_data 8-byte aligned.
 *   col_data [cols][rows/2], col_scales [cols][rows/16]: required iff
 *     FOS_OUT_COLWISE, else ignored.  col_data 8-byte aligned.
 *   cols % 16 == 0; rows % 16 == 0 for column-wise output or 2D blocks.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_HIP. */
fos_status fos_quantize_scaled(const fos_quant_config* cfg, const void* x, int64_t rows,
                               int64_t cols, const float* tensor_scale,
                               uint8_t* row_data, uint8_t* row_scales,
                               uint8_t* col_data, uint8_t* col_scales, void* stream);

/* Four Over Six quantization of a bf16 tensor into an NVFP4 record (Four Over Six
 * documentation page, "Four Over Six": per block, max -> 6 or max -> 4, whichever
 * gives the lower error; Ultralytics glossary "FP4", "How FP4 works": 16 E2M1 values
 * per E4M3 scale plus one FP32 tensor scale).
 * fos_tensor_scale followed by fos_quantize_scaled on the same stream, with the same
 * results; the tensor scale is written to *tensor_scale.  (The partial maxima of the
 * scale pass are reduced inside the quantize kernel, which saves one launch.)
 *   workspace: device scratch of at least fos_quantize_workspace_bytes() bytes,
 *   16-byte aligned, owned by the caller; calls that may overlap need their own.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_WORKSPACE,
 * FOS_E_HIP. */
fos_status fos_quantize(const fos_quant_config* cfg, const void* x, int64_t rows,
                        int64_t cols, uint8_t* row_data, uint8_t* row_scales,
                        uint8_t* col_data, uint8_t* col_scales, float* tensor_scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/* fos_quantize for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same results.  The
 * tensor-scale pass keeps its partial maxima in a 4096-byte device array that the
 * library holds on each GPU it runs on until the process ends (1024 fp32 partial
 * maxima; the pass never needs more, for any shape the other checks accept, and a
 * pass that would is refused with FOS_E_WORKSPACE).  The call allocates nothing
 * and frees nothing; its first call on a device looks the array's address up.
 * Every call on one GPU shares that array: calls that may overlap on one GPU
 * (different streams, or other threads) race and must be ordered by the caller.
 * Nothing in the array needs clearing between calls (every partial is written
 * before it is read).
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_WORKSPACE,
 * FOS_E_HIP. */
fos_status fos_quantize_noalloc(const fos_quant_config* cfg, const void* x, int64_t rows,
                                int64_t cols, uint8_t* row_data, uint8_t* row_scales,
                                uint8_t* col_data, uint8_t* col_scales, float* tensor_scale,
                                void* stream);

/* Self-test of the hardware E4M3 conversion that the quantize kernels use for the
 * block scales (gfx950's packed fp32 -> OCP E4M3 conversion, nearest-even): adds to
 * *mismatches (device uint64, 8-byte aligned; the caller zeroes it) the number of
 * fp32 values r in [0, 448] -- every bit pattern, 1,138,753,537 of them -- whose
 * hardware code differs from the bit-level rule (E4M3 "FN" round-to-nearest-even,
 * subnormals kept; Ultralytics glossary "FP4", "How FP4 works", for the E4M3 block
 * scale).  A correct device gives 0.  Takes a few milliseconds.
 * Errors: FOS_E_NULL, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_selftest_e4m3(unsigned long long* mismatches, void* stream);

/* Self-test of the hardware E2M1 conversion that the quantize kernels use for the
 * element codes (gfx950's fp32 -> FP4 conversion with scale 1): adds to *mismatches
 * (device uint64, 8-byte aligned; the caller zeroes it) the number of finite fp32
 * values v -- every bit pattern except NaN and Inf -- whose hardware code differs from
 * the rounding rule: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (Ultralytics glossary
 * "FP4", opening section), ties to the even code, saturating at 6, with the sign of v
 * (a value that rounds to 0 keeps it).  A correct device gives 0.  Takes a few tens
 * of milliseconds.
 * Errors: FOS_E_NULL, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_selftest_e2m1(unsigned long long* mismatches, void* stream);

/* Self-test of the hardware stochastic rounding to E2M1 that the quantize kernels use
 * with FOS_ROUND_SR (gfx950's fp32 -> FP4 conversion with a 32-bit rounding operand,
 * scale 1), driven exactly as the kernels drive it (the operand built from the draw
 * byte): for every finite fp32 value v and every draw byte k in 0..255, the code must
 * be the draw rule's -- with lo and hi the E2M1 values around min(|v|, 6),
 * p = (|v| - lo) / (hi - lo) and p22 = p truncated to 22 fractional bits, hi iff
 * (k + 0.5) / 256 < p22, with the sign of v (the stochastic rounding of the Four Over
 * Six page, section "Four Over Six", under the draws this library takes), at both
 * positions of a pair.
 * Adds to *mismatches (device uint64, 8-byte aligned; the caller zeroes it) the number
 * of disagreements over those 2 x 256 x (2^32 - 2^24) cases.  A correct device gives
 * 0.  Takes about a second.
 * Errors: FOS_E_NULL, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_selftest_e2m1_sr(unsigned long long* mismatches, void* stream);

/* Self-test of the hardware stochastic rounding to E2M1 as FOS_ROUND_STOCHASTIC_FULL
 * drives it (operand = the draw word at the first position of a pair, the word
 * shifted right by one at the second): for every finite fp32 value v and both
 * positions, the draw words on either side of the rounding boundary -- u = 2^22 - P
 * (rounds up, when P > 0) and u = 2^22 - P - 1 (stays down), u = word >> 10, P = the
 * first 22 fractional bits of v's position between its grid neighbours -- must give
 * the rule's codes (6 and above: 6 for any draw), with the word's low 10 bits set to
 * an arbitrary pattern.  Since the rounding is monotone in u, this fixes it for every
 * draw.  Adds the number of disagreements to *mismatches (device uint64, 8-byte
 * aligned; the caller zeroes it); a correct device gives 0.
 * Errors: FOS_E_NULL, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_selftest_e2m1_sr_full(unsigned long long* mismatches, void* stream);

/* Dequantize one NVFP4 record (Ultralytics glossary "FP4", "How FP4 works": a value
 * is its E2M1 code times its block's E4M3 scale times the tensor's FP32 scale):
 *   out[r][c] = RN_fp32(E2M1(q) * RN_fp32(E4M3(s) * t))
 * with the nibble's sign (-0 for code 8); FOS_OUT_BF16 rounds that fp32 value to
 * bf16 (nearest-even).  Works for row-wise, column-wise (giving X^T) and 2D records.
 *   data [rows][cols/2] (8-byte aligned), scales [rows][cols/16], tensor_scale: one
 *   device fp32; out [rows][cols] (16-byte aligned).  cols % 16 == 0.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_HIP. */
fos_status fos_dequantize(const uint8_t* data, const uint8_t* scales,
                          const float* tensor_scale, int64_t rows, int64_t cols,
                          int out_dtype, void* out, void* stream);

/* Dequantize a record made with the random Hadamard transform (cfg->hadamard with
 * seed `hadamard_seed`) back to the original basis: fos_dequantize's fp32 values,
 * then for every 16-value block of the record's rows the inverse transform, in fp32
 * and in this order: multiply by 1/4, the 16-point Walsh-Hadamard butterflies
 * (strides 1, 2, 4, 8), then the tensor's signs (the transform is orthogonal, so
 * its inverse is its transpose).  FOS_OUT_BF16 rounds the result to nearest-even.
 * The Four Over Six documentation page lists the transform among the quantization
 * options; the Ultralytics glossary "FP4" (FP4 for inference and training) notes
 * that such transforms spread outliers.  For a column-wise record the result is
 * X^T.  Arguments, layout and errors as for fos_dequantize. */
fos_status fos_dequantize_hadamard(const uint8_t* data, const uint8_t* scales,
                                   const float* tensor_scale, int64_t rows, int64_t cols,
                                   uint64_t hadamard_seed, int out_dtype, void* out,
                                   void* stream);

/* Simulated quantized linear forward (Four Over Six documentation page, "Four Over
 * Six": without native FP4 matmuls the layer is simulated with a higher-precision
 * matrix multiplication of the dequantized operands):
 *   Y[m][n] = bf16( (t_x * t_w) * sum_k (E*D)_x[m][k] * (E*D)_w[n][k] )
 * Operands are NVFP4 records blocked along K: Xq [M][K] (x_data [M][K/2],
 * x_scales [M][K/16]) and Wq [N][K] (the [out][in] Linear layout); any records
 * blocked along their shared dimension work (e.g. column-wise records, which are
 * the records of the transposes, or 2D records).
 * E*D products are formed exactly in fp16, multiplied on the matrix cores with fp32
 * accumulation; the tensor scales are applied in fp32 before the bf16 rounding.
 *   M, N >= 1; K >= 64 and K % 64 == 0; (M + 256) * K / 2 and (N + 256) * K / 2
 *   below 2^32 (each packed operand is one buffer resource).  x_data, w_data
 *   16-byte aligned, x_scales, w_scales 4-byte aligned, y_bf16 [M][N] 2-byte
 *   aligned.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_qlinear_fwd(const uint8_t* x_data, const uint8_t* x_scales,
                           const float* x_tensor_scale, const uint8_t* w_data,
                           const uint8_t* w_scales, const float* w_tensor_scale,
                           int64_t M, int64_t N, int64_t K, void* y_bf16, void* stream);

/* Backward pass of the simulated quantized linear layer (Four Over Six documentation
 * page, "Training": the quantized linear layer implements a backward pass).  For
 * Y = X W^T with X [M][K], W [N][K] and the output gradient dY [M][N]:
 *   dX [M][K] = bf16( deq(dY) . deq(W^T)^T )      inner dimension N
 *   dW [N][K] = bf16( deq(dY^T) . deq(X^T)^T )    inner dimension M
 * computed by the same kernel as fos_qlinear_fwd, from records blocked along each
 * product's inner dimension:
 *   dy_*  : row-wise record of dY   [M][N]   (blocked along N)
 *   dyt_* : column-wise record of dY = record of dY^T [N][M]   (blocked along M)
 *   xt_*  : column-wise record of X  = record of X^T  [K][M]   (blocked along M)
 *   wt_*  : column-wise record of W  = record of W^T  [K][N]   (blocked along N)
 * A random Hadamard transform on the two operands of one product with the same seed
 * (e.g. dY^T and X^T along M) cancels in the product, since the transform is
 * orthogonal.  dx_bf16 or dw_bf16 may be NULL to skip that product (not both);
 * the operands of a skipped product are not read.  Shapes and alignment as for
 * fos_qlinear_fwd, with each product's inner dimension in the role of K.  All
 * arguments are validated before either product is launched.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_qlinear_bwd(const uint8_t* dy_data, const uint8_t* dy_scales,
                           const float* dy_tensor_scale, const uint8_t* dyt_data,
                           const uint8_t* dyt_scales, const float* dyt_tensor_scale,
                           const uint8_t* xt_data, const uint8_t* xt_scales,
                           const float* xt_tensor_scale, const uint8_t* wt_data,
                           const uint8_t* wt_scales, const float* wt_tensor_scale,
                           int64_t M, int64_t N, int64_t K, void* dx_bf16, void* dw_bf16,
                           void* stream);

/* Workspace bytes that fos_qlinear_fwd_act needs for an activation X [M][K]; 0 when
 * M or K is negative or the size does not fit in size_t.  Layout of the workspace
 * after a call (offsets from its start; P = round_up(M*K/2, 256),
 * Q = round_up(P + M*K/16, 256)):
 *   [0, M*K/2)                 nibbles of X's row-wise record  [M][K/2]
 *   [P, P + M*K/16)            its E4M3 block scales           [M][K/16]
 *   [Q, Q + fos_workspace_bytes())  scratch of the tensor-scale pass */
size_t fos_qlinear_act_workspace_bytes(int64_t M, int64_t K);

/* Quantized linear forward from a bf16 activation: the inference path of a linear
 * layer whose weight was quantized ahead of time (Four Over Six documentation page,
 * "Four Over Six": the quantized layer is simulated with a higher-precision matmul
 * of the dequantized operands).  X [M][K] is quantized with cfg into the workspace
 * (its row-wise record, blocked along K), then multiplied with Wq as in
 * fos_qlinear_fwd, on the same stream:
 *   Y = fos_qlinear_fwd(record of X, Wq)
 * with results identical to fos_quantize (or fos_quantize_scaled) followed by
 * fos_qlinear_fwd.  The record stays in the workspace (layout above) until the
 * workspace is reused.
 *   x_tensor_scale: device fp32.  x_scale_given == 0: the call runs the tensor-scale
 *     pass and writes t_x there.  x_scale_given != 0: the call reads a t_x that the
 *     caller computed beforehand (delayed scaling, or fos_tensor_scale issued ahead
 *     of time, e.g. on a second stream while the previous layer runs), and X is
 *     read once.
 *   cfg: outputs must be FOS_OUT_ROWWISE.  Any rule and rounding; 2D blocks need
 *     M % 16 == 0; with the Hadamard transform W must carry the same transform
 *     along K, so that it cancels in the product.
 *   x_bf16 [M][K] 16-byte aligned; workspace 256-byte aligned, at least
 *     fos_qlinear_act_workspace_bytes(M, K) bytes; Wq, y_bf16, M, N, K as for
 *     fos_qlinear_fwd (K % 64 == 0).
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_WORKSPACE,
 * FOS_E_HIP. */
fos_status fos_qlinear_fwd_act(const fos_quant_config* cfg, const void* x_bf16,
                               float* x_tensor_scale, int x_scale_given,
                               const uint8_t* w_data, const uint8_t* w_scales,
                               const float* w_tensor_scale, int64_t M, int64_t N, int64_t K,
                               void* y_bf16, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- MXFP4 -------------------------------------------------------------------
 * Ultralytics glossary "FP4", "How FP4 works": MXFP4 (OCP Microscaling) groups 32
 * E2M1 values under one power-of-two E8M0 scale; "FP4 for inference and training":
 * MI350-class accelerators multiply it natively.  No per-tensor scale.
 * Record layout: data [R][C/2] nibbles as for NVFP4; scales [R][C/32] E8M0 bytes
 * (value 2^(byte - 127)).
 * Scale rule (the OCP MX specification's; the page names the specification but not
 * the rule): e = floor(log2(max |x| of the block)) - 2, clamped to [-127, 127], -127
 * for a block of zeros; elements are E2M1 round-to-nearest-even of x / 2^e,
 * saturating at 6, zeros keeping the sign of x. */

/* MXFP4 quantization of bf16 x [rows][cols] (16-byte aligned), cols % 32 == 0;
 * data 16-byte aligned.  Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_mx_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* data,
                           uint8_t* scales, void* stream);

/* out[r][c] = E2M1(q) * 2^(scale - 127) (exact in fp32; FOS_OUT_BF16 rounds it to
 * nearest-even).  data 4-byte aligned, out 16-byte aligned, cols % 32 == 0.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_FLAGS, FOS_E_HIP. */
fos_status fos_mx_dequantize(const uint8_t* data, const uint8_t* scales, int64_t rows,
                             int64_t cols, int out_dtype, void* out, void* stream);

/* Native FP4 linear: Y[m][n] = bf16( sum_k deq(A)[m][k] * deq(B)[n][k] ) for MXFP4
 * records A [M][K] and B [N][K] blocked along K, on the scaled FP4 matrix cores
 * (E2M1 x E2M1 products with the two E8M0 block scales, fp32 accumulation).
 *   M, N >= 1; K >= 256 and K % 256 == 0; (M + 256) * K / 2 and (N + 256) * K / 2
 *   below 2^32.  a_data, b_data 16-byte aligned; a_scales, b_scales 4-byte
 *   aligned; y_bf16 [M][N] 2-byte aligned.
 * Errors: FOS_E_NULL, FOS_E_SHAPE, FOS_E_ALIGN, FOS_E_HIP. */
fos_status fos_mx_qlinear_fwd(const uint8_t* a_data, const uint8_t* a_scales,
                              const uint8_t* b_data, const uint8_t* b_scales, int64_t M,
                              int64_t N, int64_t K, void* y_bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FOS_H */
