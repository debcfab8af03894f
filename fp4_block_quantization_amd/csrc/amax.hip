// Per-tensor scale: t = max|x| / 2688 (one FP32 scale per tensor, Ultralytics
// glossary "FP4", section "How FP4 works"; 2688 = 448 * 6).
//
// One streaming pass writes one partial maximum per workgroup into the caller's
// workspace (plain stores: no atomics, no fences, nothing to clear between calls);
// either a one-workgroup kernel reduces the partials and writes t, or the quantize
// kernel that follows reduces them in every workgroup (at most 1024 partials: one
// 16-byte load per thread) and its first workgroup writes t.  Each thread folds
// |x| into a running maximum (integer max of bf16 bit patterns with the sign cleared:
// for non-negative floats the bit order is the value order); the wave reduces with
// lane shuffles and the workgroup through LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

// Block-wide max of `bits` (fp32 patterns of non-negative values) -> partials[block].
__device__ __forceinline__ void write_partial(uint32_t bits, float* partials) {
  bits = block_max_u32(bits);
  if (threadIdx.x == 0) partials[blockIdx.x] = __uint_as_float(bits);
}

// No transform: grid-stride pass over 16-byte chunks (8 bf16); every lane issues
// four independent 16-byte loads per iteration before consuming any.  At most 512
// workgroups (two per CU): enough loads in flight to stream at full bandwidth, and
// few enough partials for every quantize workgroup to reduce them itself.
constexpr int kUnroll = 4;
constexpr int kFlatMaxGrid = 512;
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const uint4* __restrict__ x,
                                                             int64_t n16, float* partials) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t m = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) m = pk_max_abs4(m, w[u]);
  }
  for (; i < n16; i += stride) m = pk_max_abs4(m, x[i]);
  write_partial(pk_max_to_f32_bits(m), partials);
}

// Hadamard along rows: every 16-value block (two 16-byte chunks) is transformed.
__global__ __launch_bounds__(kThreads) void amax_rht_rows_kernel(const uint4* __restrict__ x,
                                                                 int64_t nblk, uint32_t mask,
                                                                 float* partials) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  float m = 0.0f;
  int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; b + stride < nblk; b += 2 * stride) {   // two blocks' loads in flight per lane
    const uint4 w0 = x[2 * b], w1 = x[2 * b + 1];
    const uint4 w2 = x[2 * (b + stride)], w3 = x[2 * (b + stride) + 1];
    float v[16];
    unpack16(w0, w1, v);
    rht16(v, mask);
    m = fmaxf(m, amax16(v));
    unpack16(w2, w3, v);
    rht16(v, mask);
    m = fmaxf(m, amax16(v));
  }
  if (b < nblk) {
    float v[16];
    unpack16(x[2 * b], x[2 * b + 1], v);
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

// Reduce the partials of the tensor-scale pass and write t.
__global__ __launch_bounds__(kThreads) void scale_finalize_kernel(const float* __restrict__ partials,
                                                                  int n, float* tscale) {
  const float a = reduce_partials(partials, n);
  if (threadIdx.x == 0) tscale[0] = a / kScaleDenom;
}

// Workgroups for `work_items` items at `per_thread` items per lane, capped, and
// rounded up to a multiple of 4 (idle workgroups write a zero partial).
int grid_for(int64_t work_items, int per_thread, int cap) {
  int64_t g = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)((g + 3) & ~3);
}

}  // namespace

int tensor_scale_partials(int64_t rows, int64_t cols, bool hadamard, bool hadamard_cols) {
  const int64_t n = rows * cols;
  if (!hadamard) return grid_for(n / 8, kUnroll, kFlatMaxGrid);
  if (!hadamard_cols) return grid_for(n / 16, 2, kMaxPartials);
  return grid_for((rows / 16) * (cols / 8), 1, kMaxPartials);
}

hipError_t launch_tensor_scale(const uint16_t* x, int64_t rows, int64_t cols, bool hadamard,
                               bool hadamard_cols, uint32_t rht_mask, float* partials,
                               bool finalize, float* tscale, int* npartials,
                               hipStream_t stream) {
  const int64_t n = rows * cols;
  const int g = tensor_scale_partials(rows, cols, hadamard, hadamard_cols);
  if (!hadamard) {
    amax_flat_kernel<<<g, kThreads, 0, stream>>>((const uint4*)x, n / 8, partials);
  } else if (!hadamard_cols) {
    amax_rht_rows_kernel<<<g, kThreads, 0, stream>>>((const uint4*)x, n / 16, rht_mask, partials);
  } else {
    amax_rht_cols_kernel<<<g, kThreads, 0, stream>>>(x, rows, cols, rht_mask, partials);
  }
  if (finalize) scale_finalize_kernel<<<1, kThreads, 0, stream>>>(partials, g, tscale);
  if (npartials) *npartials = g;
  return hipGetLastError();
}

}  // namespace fos
