// NVFP4 dequantization: value = E2M1(nibble) * (E4M3(scale) * t), each product
// rounded once to fp32 (Ultralytics glossary "FP4", section "How FP4 works": the
// dequantized value is the grid value times its sign times the block scale; the
// NVFP4 block scale is itself an E4M3 number under a per-tensor FP32 scale).
// One lane per 16-value block: an 8-byte nibble load, one scale byte, hardware
// E2M1->fp32 conversion, and 64 (fp32) or 32 (bf16) output bytes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint2* __restrict__ data,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tscale,
                                                           int64_t nblk, void* __restrict__ out) {
  const float t = tscale[0];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    const uint2 q = data[b];
    const float d = e4m3_decode(scales[b]) * t;
    f32x2 e[8];
    e[0] = cvt_pk_f32_fp4<0>(q.x); e[1] = cvt_pk_f32_fp4<1>(q.x);
    e[2] = cvt_pk_f32_fp4<2>(q.x); e[3] = cvt_pk_f32_fp4<3>(q.x);
    e[4] = cvt_pk_f32_fp4<0>(q.y); e[5] = cvt_pk_f32_fp4<1>(q.y);
    e[6] = cvt_pk_f32_fp4<2>(q.y); e[7] = cvt_pk_f32_fp4<3>(q.y);
    float y[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      y[2 * j] = e[j].x * d;
      y[2 * j + 1] = e[j].y * d;
    }
    if (kBF16) {
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j] = f32_to_bf16_rne(y[2 * j]) | (f32_to_bf16_rne(y[2 * j + 1]) << 16);
      uint4* o = reinterpret_cast<uint4*>(out) + 2 * b;
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float4* o = reinterpret_cast<float4*>(out) + 4 * b;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* data, const uint8_t* scales, const float* tscale,
                             int64_t rows, int64_t cols, bool bf16_out, void* out,
                             hipStream_t s) {
  const int64_t nblk = rows * cols / 16;
  if (nblk == 0) return hipSuccess;
  int64_t grid = (nblk + kThreads - 1) / kThreads;
  if (grid > (int64_t)1 << 30) grid = (int64_t)1 << 30;
  if (bf16_out)
    dequant_kernel<true><<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint2*>(data), scales,
                                                   tscale, nblk, out);
  else
    dequant_kernel<false><<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint2*>(data), scales,
                                                    tscale, nblk, out);
  return hipGetLastError();
}

}  // namespace fos
