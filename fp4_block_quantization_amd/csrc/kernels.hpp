// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fos {

struct QuantArgs {
  const uint16_t* x;        // bf16 [rows][cols]
  int64_t rows, cols;
  const float* tscale;      // device fp32 t (read when `partials` is null)
  const float* partials;    // tensor-scale partial maxima: when set, every workgroup
  int npartials;            //   reduces them to t itself and workgroup 0 writes t to
  float* tscale_out;        //   *tscale_out (fused finish of the tensor-scale pass)
  uint8_t* row_data;        // [rows][cols/2]   (may be null when not requested)
  uint8_t* row_scales;      // [rows][cols/16]
  uint8_t* col_data;        // [cols][rows/2]
  uint8_t* col_scales;      // [cols][rows/16]
  uint32_t rht_mask;        // bit k set -> sign k of the Hadamard transform is -1
  uint32_t sr_k0, sr_k1;    // Philox key for stochastic rounding
  bool four_over_six;
  uint8_t sr;               // 0: nearest-even, 1: 8-bit draws, 2: full-resolution draws
  bool two_d;
  bool rows_out, cols_out;
  bool hadamard;
};

// Number of partial maxima the tensor-scale pass writes for this shape (a multiple
// of 4, at least 4 and at most kMaxPartials).
int tensor_scale_partials(int64_t rows, int64_t cols, bool hadamard, bool hadamard_cols);

// Tensor-scale pass: one partial max|x| per workgroup into `partials` (16-byte
// aligned; the count, a multiple of 4 and at most kMaxPartials, goes to *npartials).
// With `finalize`, a one-workgroup kernel then writes t = max / 2688 to *tscale;
// without it the quantize kernel finishes the reduction (QuantArgs::partials).
hipError_t launch_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, bool hadamard,
                               bool hadamard_cols, uint32_t rht_mask, float* partials,
                               bool finalize, float* tscale, int* npartials,
                               hipStream_t stream);

// One dispatch covers at most 2^32 - 1 work-items along a grid dimension, so a launch
// of 256-thread workgroups may use at most this many workgroups.  The C ABI checks
// the grid of every launch below against it before launching anything.
constexpr int64_t kMaxGrid = (((int64_t)1 << 32) - 1) / 256;

// Workgroups of the quantize launch for these arguments (0 for an empty tensor).
int64_t quantize_grid(const QuantArgs& a);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);

// Adds to *mismatches the number of disagreements between the hardware E4M3
// conversion the quantize kernels use and the bit-level definition (e4m3_encode),
// over every fp32 value in [0, 448].
hipError_t launch_selftest_e4m3(unsigned long long* mismatches, hipStream_t stream);

// Adds to *mismatches the number of disagreements between the hardware E2M1
// conversion the quantize kernels use and the rounding rule, over every finite fp32.
hipError_t launch_selftest_e2m1(unsigned long long* mismatches, hipStream_t stream);

// Adds to *mismatches the number of disagreements between the hardware stochastic
// rounding to E2M1 under the operands the quantize kernels build from their draws and
// the draw rule, over every finite fp32 and every draw byte, at both pair positions.
hipError_t launch_selftest_e2m1_sr(unsigned long long* mismatches, hipStream_t stream);

// Adds to *mismatches the number of disagreements at the rounding boundary of the
// full-resolution stochastic rounding (operands straight from the draw words), over
// every finite fp32 at both pair positions.
hipError_t launch_selftest_e2m1_sr_full(unsigned long long* mismatches, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* data, const uint8_t* scales, const float* tscale,
                             int64_t rows, int64_t cols, bool bf16_out, void* out,
                             hipStream_t stream);

// Dequantize a record made with the random Hadamard transform (sign mask `rht_mask`)
// and apply the inverse transform to every 16-value block.
hipError_t launch_dequantize_hadamard(const uint8_t* data, const uint8_t* scales,
                                      const float* tscale, int64_t rows, int64_t cols,
                                      uint32_t rht_mask, bool bf16_out, void* out,
                                      hipStream_t stream);

// MXFP4 (32 E2M1 values per E8M0 scale): quantize bf16 [rows][cols] (cols % 32 == 0),
// dequantize, and the native FP4 GEMM Y = deq(A) deq(B)^T (K % 256 == 0).
int64_t mx_quantize_grid(int64_t rows, int64_t cols);
int64_t mx_gemm_grid(int64_t M, int64_t N);
hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* data,
                              uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_dequantize(const uint8_t* data, const uint8_t* scales, int64_t rows,
                                int64_t cols, bool bf16_out, void* out, hipStream_t stream);
hipError_t launch_mx_gemm(const uint8_t* ad, const uint8_t* as, const uint8_t* bd,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          hipStream_t stream);

// Workgroups of the qlinear launch for an [M][N] output.
int64_t qlinear_grid(int64_t M, int64_t N);

hipError_t launch_qlinear(const uint8_t* xd, const uint8_t* xs, const float* xt,
                          const uint8_t* wd, const uint8_t* ws, const float* wt, int64_t M,
                          int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

}  // namespace fos
