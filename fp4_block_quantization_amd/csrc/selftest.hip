// Device self-tests of the hardware conversions that the quantize kernels use in place
// of the bit-level rules they stand for (format: Ultralytics glossary "FP4", opening
// section and "How FP4 works"): fp32 -> E4M3 for the block scales, fp32 -> E2M1 for
// the element codes, and fp32 -> E2M1 with stochastic rounding under the draws.  Each kernel runs every input of its range through both and
// adds the number of disagreements to a device counter.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

// Self-test of the hardware E4M3 conversion: every fp32 bit pattern in [0, 448] is
// converted by e4m3_encode_pk_hw (both halves) and by e4m3_encode; each lane counts
// its disagreements and adds a nonzero count to *mismatches.
constexpr uint32_t kE4m3TestPatterns = 0x43E00001u;   // +0 .. 448.0 inclusive
__global__ __launch_bounds__(kThreads) void selftest_e4m3_kernel(unsigned long long* mismatches) {
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t bad = 0;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < kE4m3TestPatterns; i += stride) {
    const float r = __uint_as_float(i);
    const uint32_t hw = e4m3_encode_pk_hw(r, r);
    const uint32_t sw = e4m3_encode(r);
    bad += ((hw & 0xffu) != sw) + ((hw >> 8) != sw);
  }
  if (bad) atomicAdd(mismatches, (unsigned long long)bad);
}

// Self-test of the hardware E2M1 conversion (cvt_pk_fp4, scale 1) against the rule it
// stands for: nearest value of {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
// saturating at 6, the sign of v kept (also when the value rounds to 0).  Code k + 1
// wins over code k when |v| lies above their midpoint, or on it with k + 1 even.
// Every finite fp32 bit pattern is checked (grid-stride over all 2^32, NaN and Inf
// skipped); each lane adds a nonzero disagreement count to *mismatches.
__device__ __forceinline__ uint32_t e2m1_encode_rule(float v) {
  const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  const float m = fabsf(v);
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k)
    if (m > mid[k] || (m == mid[k] && ((k + 1) & 1) == 0)) c = k + 1;
  return c | (__builtin_signbit(v) ? 8u : 0u);
}
__global__ __launch_bounds__(kThreads) void selftest_e2m1_kernel(unsigned long long* mismatches) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint32_t bad = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < ((uint64_t)1 << 32);
       i += stride) {
    const uint32_t b = (uint32_t)i;
    if ((b & 0x7f800000u) == 0x7f800000u) continue;   // NaN, Inf
    const float v = __uint_as_float(b);
    const uint32_t hw = cvt_pk_fp4<0>(0u, v, v) & 0xffu;
    const uint32_t sw = e2m1_encode_rule(v);
    bad += ((hw & 0xfu) != sw) + ((hw >> 4) != sw);
  }
  if (bad) atomicAdd(mismatches, (unsigned long long)bad);
}

// Self-test of the hardware stochastic rounding to E2M1 as the quantize kernels drive
// it (operands from sr_operand, the second position's shifted right by one; conversion
// by cvt_sr_fp4_byte into each of the four bytes of a word, the other bytes kept)
// against the draw rule: with lo and hi the grid values around |v|,
// p = (|v| - lo) / (hi - lo) and p22 = p truncated to 22 fractional bits, the code is
// hi's iff (k + 0.5) / 256 < p22; the sign of v is kept; 6 and above give 6.  The rule's grid position is found here with plain comparisons
// (steps 0.5 below 2, 1 below 4, 2 above), and p = y - floor(y) with y = |v| / step,
// both exact, as is p22 = floor(p * 2^22) * 2^-22.  Every finite fp32 pattern is
// checked against all 256 draws, at both positions of a pair (with -v as the other
// value); each lane adds a nonzero disagreement count to *mismatches.
__global__ __launch_bounds__(kThreads) void selftest_e2m1_sr_kernel(unsigned long long* mismatches) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint32_t bad = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < ((uint64_t)1 << 32);
       i += stride) {
    const uint32_t b = (uint32_t)i;
    if ((b & 0x7f800000u) == 0x7f800000u) continue;   // NaN, Inf
    const float v = __uint_as_float(b);
    const float m = fabsf(v);
    const uint32_t sign = (b >> 31) << 3;
    uint32_t lo_code, hi_code;
    float p;
    if (m >= 6.0f) {
      lo_code = hi_code = 7u;
      p = 0.0f;
    } else {
      const float step = (m < 2.0f) ? 0.5f : (m < 4.0f) ? 1.0f : 2.0f;
      const float y = m / step;
      const float yl = floorf(y);
      p = floorf((y - yl) * 0x1p22f) * 0x1p-22f;
      // grid value yl * step -> its code: 2 * value below 2, then 4 (2), 5 (3), 6 (4)
      lo_code = (m < 2.0f) ? (uint32_t)yl : (m < 4.0f) ? 2u + (uint32_t)yl : 6u;
      hi_code = lo_code + 1u;
    }
    for (uint32_t k0 = 0; k0 < 256; k0 += 4) {
      const uint32_t nw = ~(k0 * 0x01010101u + 0x03020100u);   // bytes k0 .. k0 + 3
      // draw k0 + B goes to byte B of both words (first position in w1, second in w2)
      uint32_t w1 = any_word(), w2 = any_word(), expect[4], r;
#define FOS_SR_CASE(B)                                                                   \
      expect[B] = (((float)(k0 + B) + 0.5f) * 0x1p-8f < p ? hi_code : lo_code) | sign;   \
      r = sr_operand<B>(nw, 0x007fffffu);                                                \
      w1 = cvt_sr_fp4_byte<B>(w1, f32x2{v, -v}, r);                                      \
      w2 = cvt_sr_fp4_byte<B>(w2, f32x2{-v, v}, r >> 1);
      FOS_SR_CASE(0) FOS_SR_CASE(1) FOS_SR_CASE(2) FOS_SR_CASE(3)
#undef FOS_SR_CASE
#pragma unroll
      for (int B = 0; B < 4; ++B)
        bad += (((w1 >> (8 * B)) & 0xfu) != expect[B]) + (((w2 >> (8 * B + 4)) & 0xfu) != expect[B]);
    }
  }
  if (bad) atomicAdd(mismatches, (unsigned long long)bad);
}

// Self-test of the full-resolution stochastic rounding (sr_operands_full): for every
// finite fp32 v, the position P (22 fractional bits, as in the 8-bit test above) and,
// at each pair position, the draw words with u = word >> 10 on either side of the
// boundary P + u = 2^22: u = 2^22 - P must round up (when P > 0) and u = 2^22 - P - 1
// must not; at 6 and above both draws give 6.  The word's low 10 bits take a pattern
// from v's bits (the rule ignores them).
__global__ __launch_bounds__(kThreads) void selftest_e2m1_sr_full_kernel(
    unsigned long long* mismatches) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  uint32_t bad = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < ((uint64_t)1 << 32);
       i += stride) {
    const uint32_t b = (uint32_t)i;
    if ((b & 0x7f800000u) == 0x7f800000u) continue;   // NaN, Inf
    const float v = __uint_as_float(b);
    const float m = fabsf(v);
    const uint32_t sign = (b >> 31) << 3;
    uint32_t lo_code, hi_code, P;
    if (m >= 6.0f) {
      lo_code = hi_code = 7u;
      P = 0u;
    } else {
      const float step = (m < 2.0f) ? 0.5f : (m < 4.0f) ? 1.0f : 2.0f;
      const float y = m / step;
      const float yl = floorf(y);
      P = (uint32_t)floorf((y - yl) * 0x1p22f);
      lo_code = (m < 2.0f) ? (uint32_t)yl : (m < 4.0f) ? 2u + (uint32_t)yl : 6u;
      hi_code = lo_code + 1u;
    }
    const uint32_t low10 = b & 0x3ffu;
    // u below the boundary (stays down), then on it (rounds up; only when P > 0)
    const uint32_t u_down = ((1u << 22) - P - 1u) & 0x3fffffu;
    const uint32_t u_up = ((1u << 22) - P) & 0x3fffffu;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c == 1 && (P == 0u || m >= 6.0f)) continue;
      const uint32_t word = ((c ? u_up : u_down) << 10) | low10;
      const uint32_t expect = (c ? hi_code : lo_code) | sign;
      const uint32_t w1 = cvt_sr_fp4_byte<0>(0u, f32x2{v, -v}, word);
      const uint32_t w2 = cvt_sr_fp4_byte<0>(0u, f32x2{-v, v}, word >> 1);
      bad += ((w1 & 0xfu) != expect) + (((w2 >> 4) & 0xfu) != expect);
    }
    if (m >= 6.0f) {   // any draw: 6
      const uint32_t word = 0xffffffffu;
      const uint32_t w1 = cvt_sr_fp4_byte<0>(0u, f32x2{v, -v}, word);
      const uint32_t w2 = cvt_sr_fp4_byte<0>(0u, f32x2{-v, v}, word >> 1);
      bad += ((w1 & 0xfu) != (7u | sign)) + (((w2 >> 4) & 0xfu) != (7u | sign));
    }
  }
  if (bad) atomicAdd(mismatches, (unsigned long long)bad);
}

}  // namespace

hipError_t launch_selftest_e2m1_sr_full(unsigned long long* mismatches, hipStream_t s) {
  selftest_e2m1_sr_full_kernel<<<8192, kThreads, 0, s>>>(mismatches);
  return hipGetLastError();
}

hipError_t launch_selftest_e4m3(unsigned long long* mismatches, hipStream_t s) {
  selftest_e4m3_kernel<<<4096, kThreads, 0, s>>>(mismatches);
  return hipGetLastError();
}

hipError_t launch_selftest_e2m1(unsigned long long* mismatches, hipStream_t s) {
  selftest_e2m1_kernel<<<8192, kThreads, 0, s>>>(mismatches);
  return hipGetLastError();
}

hipError_t launch_selftest_e2m1_sr(unsigned long long* mismatches, hipStream_t s) {
  selftest_e2m1_sr_kernel<<<8192, kThreads, 0, s>>>(mismatches);
  return hipGetLastError();
}

}  // namespace fos
