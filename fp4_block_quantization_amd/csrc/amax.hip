// Per-tensor scale: t = max|x| / 2688 (one FP32 scale per tensor, Ultralytics
// glossary "FP4", section "How FP4 works"; 2688 = 448 * 6).
//
// One streaming pass writes one partial maximum per workgroup into the caller's
// workspace (plain stores: no atomics, no fences, nothing to clear between calls);
// a one-workgroup kernel then reduces the partials and writes t.  Each thread folds
// |x| into a running maximum (integer max of bf16 bit patterns with the sign cleared:
// for non-negative floats the bit order is the value order); the wave reduces with
// lane shuffles and the workgroup through LDS.
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

// Block-wide max of `bits` (fp32 patterns of non-negative values) -> partials[block].
__device__ __forceinline__ void write_partial(uint32_t bits, float* partials) {
  bits = block_max_u32(bits);
  if (threadIdx.x == 0) partials[blockIdx.x] = __uint_as_float(bits);
}

// No transform: each workgroup reduces one contiguous slab of 16-byte chunks (8
// bf16), a multiple of 1024 chunks long; every lane issues four independent 16-byte
// loads per iteration before consuming any.
constexpr int kUnroll = 4;
constexpr int64_t kSlabQuantum = (int64_t)kThreads * kUnroll;
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const uint4* __restrict__ x,
                                                             int64_t n16, int64_t per,
                                                             float* partials) {
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = min(beg + per, n16);
  uint32_t m = 0;
  for (int64_t i = beg + threadIdx.x; i < end; i += kSlabQuantum) {
    uint4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + u * kThreads;
      w[u] = j < end ? x[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) m = pk_max_abs4(m, w[u]);
  }
  const uint32_t bits = max(m & 0xffffu, m >> 16) << 16;
  write_partial(bits, partials);
}

// Hadamard along rows: every 16-value block (two 16-byte chunks) is transformed.
__global__ __launch_bounds__(kThreads) void amax_rht_rows_kernel(const uint4* __restrict__ x,
                                                                 int64_t nblk, uint32_t mask,
                                                                 float* partials) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    const uint4 w0 = x[2 * b], w1 = x[2 * b + 1];
    float v[16];
    unpack16(w0, w1, v);
    rht16(v, mask);
    m = fmaxf(m, amax16(v));
  }
  write_partial(__float_as_uint(m), partials);
}

// Hadamard along columns: a thread owns a patch of 16 rows x 8 columns and
// transforms each of its 8 column blocks.
__global__ __launch_bounds__(kThreads) void amax_rht_cols_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t rows, int64_t cols,
                                                                 uint32_t mask, float* partials) {
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
  write_partial(__float_as_uint(m), partials);
}

// Reduce the partials of the tensor-scale pass and write t.  Every thread issues its
// loads (n <= 4096 = 16 per thread; indices past n re-read the last partial, which
// leaves the maximum unchanged) before reducing, so the pass costs one memory latency.
__global__ __launch_bounds__(kThreads) void scale_finalize_kernel(const float* __restrict__ partials,
                                                                  int n, float* tscale) {
  constexpr int kPer = kMaxPartials / kThreads;
  uint32_t v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    v[k] = __float_as_uint(partials[min((int)threadIdx.x + k * kThreads, n - 1)]);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) m = max(m, v[k]);
  const float a = __uint_as_float(block_max_u32(m));
  if (threadIdx.x == 0) tscale[0] = a / kScaleDenom;
}

int grid_for(int64_t work_items, int per_thread) {
  int64_t g = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (g < 1) g = 1;
  if (g > kMaxPartials) g = kMaxPartials;
  return (int)g;
}

}  // namespace

hipError_t launch_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, bool hadamard,
                               bool hadamard_cols, uint32_t rht_mask, float* partials,
                               float* tscale, hipStream_t stream) {
  const int64_t n = rows * cols;
  int g;
  if (!hadamard) {
    const int64_t n16 = n / 8;
    int64_t per = (n16 + kMaxPartials - 1) / kMaxPartials;
    per = per < 1 ? kSlabQuantum : (per + kSlabQuantum - 1) / kSlabQuantum * kSlabQuantum;
    g = (int)((n16 + per - 1) / per);
    if (g < 1) g = 1;  // empty tensor: one workgroup writes a zero partial
    amax_flat_kernel<<<g, kThreads, 0, stream>>>((const uint4*)x, n16, per, partials);
  } else if (!hadamard_cols) {
    const int64_t nblk = n / 16;
    g = grid_for(nblk, 2);
    amax_rht_rows_kernel<<<g, kThreads, 0, stream>>>((const uint4*)x, nblk, rht_mask, partials);
  } else {
    const int64_t npatch = (rows / 16) * (cols / 8);
    g = grid_for(npatch, 1);
    amax_rht_cols_kernel<<<g, kThreads, 0, stream>>>(x, rows, cols, rht_mask, partials);
  }
  scale_finalize_kernel<<<1, kThreads, 0, stream>>>(partials, g, tscale);
  return hipGetLastError();
}

}  // namespace fos
