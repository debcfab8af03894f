// Per-tensor scale: t = max|x| / 2688 (one FP32 scale per tensor, Ultralytics
// glossary "FP4", section "How FP4 works"; 2688 = 448 * 6).
//
// One pass over the tensor.  Each thread folds |x| into a running maximum (integer
// max of bf16 bit patterns with the sign cleared: for non-negative floats the bit
// order is the value order), the wave reduces with lane shuffles, the workgroup
// through LDS, and one u32 atomic max per workgroup merges into the workspace cell.
// The last workgroup to finish (counted with a second atomic) turns the maximum
// into t and clears both workspace words for the next call.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_abs(uint32_t m, uint32_t w) {
  u16x2 a = __builtin_bit_cast(u16x2, m);
  u16x2 b = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t pk_max_abs4(uint32_t m, const uint4& w) {
  m = pk_max_abs(m, w.x);
  m = pk_max_abs(m, w.y);
  m = pk_max_abs(m, w.z);
  return pk_max_abs(m, w.w);
}

// Block-wide max of `bits` (fp32 patterns of non-negative values), atomic merge into
// ws[0], and last-block finalisation of t.
__device__ __forceinline__ void reduce_and_finalize(uint32_t bits, uint32_t* ws, float* tscale) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bits = max(bits, (uint32_t)__shfl_xor((int)bits, off));
  __shared__ uint32_t part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = bits;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = max(m, part[w]);
    atomicMax(&ws[0], m);
    __threadfence();
    const uint32_t prev = atomicAdd(&ws[1], 1u);
    if (prev == gridDim.x - 1) {
      __threadfence();
      const uint32_t a = atomicOr(&ws[0], 0u);
      tscale[0] = __uint_as_float(a) / kScaleDenom;
      atomicExch(&ws[0], 0u);
      atomicExch(&ws[1], 0u);
    }
  }
}

// No transform: flat pass over 16-byte chunks (8 bf16).
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const uint4* __restrict__ x,
                                                             int64_t n16, uint32_t* ws,
                                                             float* tscale) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 w0 = x[i], w1 = x[i + stride], w2 = x[i + 2 * stride], w3 = x[i + 3 * stride];
    m = pk_max_abs4(m, w0);
    m = pk_max_abs4(m, w1);
    m = pk_max_abs4(m, w2);
    m = pk_max_abs4(m, w3);
  }
  for (; i < n16; i += stride) m = pk_max_abs4(m, x[i]);
  const uint32_t bits = max(m & 0xffffu, m >> 16) << 16;
  reduce_and_finalize(bits, ws, tscale);
}

// Hadamard along rows: every 16-value block (two 16-byte chunks) is transformed.
__global__ __launch_bounds__(kThreads) void amax_rht_rows_kernel(const uint4* __restrict__ x,
                                                                 int64_t nblk, uint32_t mask,
                                                                 uint32_t* ws, float* tscale) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    const uint4 w0 = x[2 * b], w1 = x[2 * b + 1];
    float v[16];
    unpack16(w0, w1, v);
    rht16(v, mask);
    m = fmaxf(m, amax16(v));
  }
  reduce_and_finalize(__float_as_uint(m), ws, tscale);
}

// Hadamard along columns: a thread owns a patch of 16 rows x 8 columns and
// transforms each of its 8 column blocks.
__global__ __launch_bounds__(kThreads) void amax_rht_cols_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows, int64_t cols,
                                                                 uint32_t mask, uint32_t* ws,
                                                                 float* tscale) {
  const int64_t ncg = cols / 8;
  const int64_t npatch = (rows / 16) * ncg;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < npatch; p += stride) {
    const int64_t r0 = (p / ncg) * 16, c0 = (p % ncg) * 8;
    uint4 w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = *(const uint4*)(x + (r0 + i) * cols + c0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t d = (c >> 1) == 0 ? w[i].x : (c >> 1) == 1 ? w[i].y : (c >> 1) == 2 ? w[i].z : w[i].w;
        v[i] = (c & 1) ? bf16_hi(d) : bf16_lo(d);
      }
      rht16(v, mask);
      m = fmaxf(m, amax16(v));
    }
  }
  reduce_and_finalize(__float_as_uint(m), ws, tscale);
}

int grid_for(int64_t work_items, int per_thread) {
  int64_t g = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  return (int)g;
}

}  // namespace

hipError_t launch_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, bool hadamard,
                               bool hadamard_cols, uint32_t rht_mask, uint32_t* ws,
                               float* tscale, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (!hadamard) {
    const int64_t n16 = n / 8;
    amax_flat_kernel<<<grid_for(n16, 4), kThreads, 0, stream>>>((const uint4*)x, n16, ws, tscale);
  } else if (!hadamard_cols) {
    const int64_t nblk = n / 16;
    amax_rht_rows_kernel<<<grid_for(nblk, 2), kThreads, 0, stream>>>((const uint4*)x, nblk,
                                                                     rht_mask, ws, tscale);
  } else {
    const int64_t npatch = (rows / 16) * (cols / 8);
    amax_rht_cols_kernel<<<grid_for(npatch, 1), kThreads, 0, stream>>>(x, rows, cols, rht_mask,
                                                                       ws, tscale);
  }
  return hipGetLastError();
}

}  // namespace fos
