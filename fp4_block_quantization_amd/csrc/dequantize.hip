// NVFP4 dequantization: value = E2M1(nibble) * (E4M3(scale) * t), each product
// rounded once to fp32 (Ultralytics glossary "FP4", section "How FP4 works": the
// dequantized value is the grid value times its sign times the block scale; the
// NVFP4 block scale is itself an E4M3 number under a per-tensor FP32 scale).
//
// Output-major: lane g writes the g-th 16-byte chunk of the output (4 fp32 or 8 bf16
// values), so every store instruction of a wave covers 1 KB of contiguous memory; it
// reads the 2 or 4 nibble bytes of its chunk (contiguous across lanes) and the block's
// scale byte (shared by the 4 or 2 lanes of a block).  Hardware E2M1 -> fp32
// conversion; bf16 output rounds the fp32 value to nearest-even.  The inverse-Hadamard
// variant needs whole blocks per lane and stages its outputs through LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

// The output-major kernel's outputs are written once, 1 KB contiguous per wave
// instruction: non-temporal 16-byte stores (measured faster than cached ones).
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 4;

template <bool kBF16>
__device__ __forceinline__ void dequant_chunk(const uint8_t* __restrict__ data,
                                              const uint8_t* __restrict__ scales, float t,
                                              int64_t g, void* __restrict__ out) {
  if (kBF16) {
    // 8 values = one 4-byte word of nibbles; block g/2
    const uint32_t q = reinterpret_cast<const uint32_t*>(data)[g];
    const float d = e4m3_decode(scales[g >> 1]) * t;
    const f32x2 e0 = cvt_pk_f32_fp4<0>(q), e1 = cvt_pk_f32_fp4<1>(q);
    const f32x2 e2 = cvt_pk_f32_fp4<2>(q), e3 = cvt_pk_f32_fp4<3>(q);
    uint4 o;
    o.x = pack_bf16x2(e0.x * d, e0.y * d);
    o.y = pack_bf16x2(e1.x * d, e1.y * d);
    o.z = pack_bf16x2(e2.x * d, e2.y * d);
    o.w = pack_bf16x2(e3.x * d, e3.y * d);
    __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(out) + g);
  } else {
    // 4 values = one 2-byte half-word of nibbles; block g/4
    const uint32_t q = reinterpret_cast<const uint16_t*>(data)[g];
    const float d = e4m3_decode(scales[g >> 2]) * t;
    const f32x2 e0 = cvt_pk_f32_fp4<0>(q), e1 = cvt_pk_f32_fp4<1>(q);
    __builtin_nontemporal_store(v4f{e0.x * d, e0.y * d, e1.x * d, e1.y * d},
                                reinterpret_cast<v4f*>(out) + g);
  }
}

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ data,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tscale,
                                                           int64_t nchunk, void* __restrict__ out) {
  const float t = tscale[0];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; g + (kUnroll - 1) * stride < nchunk; g += kUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dequant_chunk<kBF16>(data, scales, t, g + u * stride, out);
  }
  for (; g < nchunk; g += stride) dequant_chunk<kBF16>(data, scales, t, g, out);
}

// Dequantize one 16-value block (8 nibble bytes + its scale byte) into v.
__device__ __forceinline__ void dequant_block(uint2 q, uint32_t s, float t, float (&v)[16]) {
  const float d = e4m3_decode(s) * t;
  const f32x2 e[8] = {cvt_pk_f32_fp4<0>(q.x), cvt_pk_f32_fp4<1>(q.x), cvt_pk_f32_fp4<2>(q.x),
                      cvt_pk_f32_fp4<3>(q.x), cvt_pk_f32_fp4<0>(q.y), cvt_pk_f32_fp4<1>(q.y),
                      cvt_pk_f32_fp4<2>(q.y), cvt_pk_f32_fp4<3>(q.y)};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[2 * j] = e[j].x * d;
    v[2 * j + 1] = e[j].y * d;
  }
}

// Records made with the random Hadamard transform, returned to the original basis:
// lane = one 16-value block (8 nibble bytes + 1 scale byte in, 32 or 64 bytes out);
// values are dequantized exactly as above, then inverse-transformed in registers.
// A workgroup's 256 blocks are contiguous in the output, so their values go through
// LDS and out as 16-byte chunks that are contiguous across lanes: every store
// instruction of a wave writes 1 KB of whole lines (non-temporal, as in the
// output-major kernel).  Stored from the lanes that computed them, each instruction
// wrote 16 bytes at a 32- or 64-byte stride.
template <bool kBF16>
__global__ __launch_bounds__(kThreads) void dequant_rht_kernel(const uint2* __restrict__ data,
                                                               const uint8_t* __restrict__ scales,
                                                               const float* __restrict__ tscale,
                                                               int64_t nblk, uint32_t mask,
                                                               void* __restrict__ out) {
  constexpr int kChunks = kBF16 ? 2 : 4;      // 16-byte output chunks per block
  __shared__ uint4 stage[kThreads * kChunks];
  const float t = tscale[0];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint4* __restrict__ o = reinterpret_cast<uint4*>(out);
  for (int64_t b0 = (int64_t)blockIdx.x * kThreads; b0 < nblk; b0 += stride) {  // uniform
    const int64_t b = b0 + threadIdx.x;
    if (b < nblk) {
      float v[16];
      dequant_block(data[b], scales[b], t, v);
      irht16(v, mask);
      uint4* st = stage + threadIdx.x * kChunks;
      if (kBF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          st[h] = make_uint4(pack_bf16x2(v[8 * h + 0], v[8 * h + 1]),
                             pack_bf16x2(v[8 * h + 2], v[8 * h + 3]),
                             pack_bf16x2(v[8 * h + 4], v[8 * h + 5]),
                             pack_bf16x2(v[8 * h + 6], v[8 * h + 7]));
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          st[h] = make_uint4(__float_as_uint(v[4 * h]), __float_as_uint(v[4 * h + 1]),
                             __float_as_uint(v[4 * h + 2]), __float_as_uint(v[4 * h + 3]));
      }
    }
    __syncthreads();
    const int64_t nchunk = min((int64_t)kThreads, nblk - b0) * kChunks;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = threadIdx.x + kThreads * j;
      if (c < nchunk) {
        const uint4 w = stage[c];
        __builtin_nontemporal_store(v4u{w.x, w.y, w.z, w.w},
                                    reinterpret_cast<v4u*>(o + b0 * kChunks + c));
      }
    }
    __syncthreads();   // the next iteration overwrites the stage
  }
}

}  // namespace

hipError_t launch_dequantize_hadamard(const uint8_t* data, const uint8_t* scales,
                                      const float* tscale, int64_t rows, int64_t cols,
                                      uint32_t rht_mask, bool bf16_out, void* out,
                                      hipStream_t s) {
  const int64_t nblk = rows * cols / 16;
  if (nblk == 0) return hipSuccess;
  int64_t grid = (nblk + kThreads - 1) / kThreads;
  if (grid > 8192) grid = 8192;
  if (bf16_out)
    dequant_rht_kernel<true><<<grid, kThreads, 0, s>>>((const uint2*)data, scales, tscale, nblk,
                                                       rht_mask, out);
  else
    dequant_rht_kernel<false><<<grid, kThreads, 0, s>>>((const uint2*)data, scales, tscale, nblk,
                                                        rht_mask, out);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* data, const uint8_t* scales, const float* tscale,
                             int64_t rows, int64_t cols, bool bf16_out, void* out,
                             hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const int64_t nchunk = bf16_out ? n / 8 : n / 4;
  int64_t grid = (nchunk + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  if (bf16_out)
    dequant_kernel<true><<<grid, kThreads, 0, s>>>(data, scales, tscale, nchunk, out);
  else
    dequant_kernel<false><<<grid, kThreads, 0, s>>>(data, scales, tscale, nchunk, out);
  return hipGetLastError();
}

}  // namespace fos
