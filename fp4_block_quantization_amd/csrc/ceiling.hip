// Measured HBM ceilings of the running GPU: kernels that move the same bytes as the
// quantize and dequantize kernels but do no arithmetic on them.  They are not part of
// the method; the benchmark reports them beside the quantize kernels, so that a
// kernel's fraction of the published 8 TB/s can be read against what plain streaming
// reaches on the same box.  Declared in include/fos_ceiling.h.
//
// One workgroup of 256 lanes per 8 KB, each lane moving 32 bytes with two 16-byte
// non-temporal accesses:
//   ceiling_read_kernel     reads only: lane t reads 16-byte pieces t and t + 256 of the
//                           workgroup's 8 KB, so each load instruction covers 4 KB of
//                           contiguous memory; the words are folded with xor and stored
//                           only if they equal a runtime key (so the loads cannot be
//                           removed, and in practice nothing is written);
//   ceiling_copy_kernel     the same pieces written back elsewhere (read + write; each
//                           store instruction covers 4 KB, i.e. whole lines);
//   ceiling_pattern_kernel  the row-wise quantize kernel's exact traffic: lane t reads
//                           the 32-byte chunk t (pieces 2t and 2t + 1, as one 16-value
//                           block) and writes 8 bytes to one output and 1 byte to
//                           another, both with non-temporal stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fos_ceiling.h"

namespace {

constexpr int kThreads = 256;
constexpr int64_t kChunk = 32;
constexpr int64_t kWGBytes = kThreads * kChunk;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void load_chunk(const v4u* __restrict__ x, int64_t g, v4u& a, v4u& b) {
  a = __builtin_nontemporal_load(x + 2 * g);
  b = __builtin_nontemporal_load(x + 2 * g + 1);
}

__global__ __launch_bounds__(kThreads) void ceiling_read_kernel(const v4u* __restrict__ x,
                                                                uint32_t key,
                                                                uint32_t* __restrict__ sink) {
  const int64_t p = (int64_t)blockIdx.x * 2 * kThreads + threadIdx.x;
  const v4u a = __builtin_nontemporal_load(x + p);
  const v4u b = __builtin_nontemporal_load(x + p + kThreads);
  const uint32_t f = a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  if (f == key) sink[0] = f;
}

__global__ __launch_bounds__(kThreads) void ceiling_copy_kernel(const v4u* __restrict__ x,
                                                                v4u* __restrict__ y) {
  const int64_t p = (int64_t)blockIdx.x * 2 * kThreads + threadIdx.x;
  const v4u a = __builtin_nontemporal_load(x + p);
  const v4u b = __builtin_nontemporal_load(x + p + kThreads);
  __builtin_nontemporal_store(a, y + p);
  __builtin_nontemporal_store(b, y + p + kThreads);
}

__global__ __launch_bounds__(kThreads) void ceiling_pattern_kernel(const v4u* __restrict__ x,
                                                                   v2u* __restrict__ y8,
                                                                   uint8_t* __restrict__ y1) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  v4u a, b;
  load_chunk(x, g, a, b);
  __builtin_nontemporal_store(v2u{a.x ^ a.z ^ b.x ^ b.z, a.y ^ a.w ^ b.y ^ b.w}, y8 + g);
  __builtin_nontemporal_store((uint8_t)(a.x ^ b.w), y1 + g);
}

bool ok_size(size_t bytes) { return bytes > 0 && bytes % kWGBytes == 0 && bytes / kWGBytes < (1u << 24); }
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

size_t fos_ceiling_granule(void) { return (size_t)kWGBytes; }

int fos_ceiling_read(const void* x, size_t bytes, uint32_t key, uint32_t* sink, void* stream) {
  if (!x || !sink) return 1;
  if (!ok_size(bytes)) return 2;
  if (!al16(x)) return 3;
  ceiling_read_kernel<<<(unsigned)(bytes / kWGBytes), kThreads, 0, (hipStream_t)stream>>>(
      (const v4u*)x, key, sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int fos_ceiling_copy(const void* x, void* y, size_t bytes, void* stream) {
  if (!x || !y) return 1;
  if (!ok_size(bytes)) return 2;
  if (!al16(x) || !al16(y)) return 3;
  ceiling_copy_kernel<<<(unsigned)(bytes / kWGBytes), kThreads, 0, (hipStream_t)stream>>>(
      (const v4u*)x, (v4u*)y);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int fos_ceiling_pattern(const void* x, size_t bytes, void* y8, void* y1, void* stream) {
  if (!x || !y8 || !y1) return 1;
  if (!ok_size(bytes)) return 2;
  if (!al16(x) || (reinterpret_cast<uintptr_t>(y8) & 7)) return 3;
  ceiling_pattern_kernel<<<(unsigned)(bytes / kWGBytes), kThreads, 0, (hipStream_t)stream>>>(
      (const v4u*)x, (v2u*)y8, (uint8_t*)y1);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
