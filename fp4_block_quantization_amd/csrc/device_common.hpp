// Device-side building blocks for the 4/6 NVFP4 kernels (gfx950).
//
// Method: Four Over Six documentation page (Hugging Face transformers docs),
// section "Four Over Six" -- each block's scale maps its largest magnitude to 6 or to
// 4, whichever gives the lower error.  Format: Ultralytics glossary "FP4", opening
// section (E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6) and section "How FP4 works"
// (16 values per FP8 E4M3 scale, plus a per-tensor FP32 scale).
//
// Arithmetic per block and candidate c in {6, 4}, all fp32 round-to-nearest-even,
// subnormals preserved (the library is built with -ffp-contract=off):
//   u_c = 1 / (t*c)               (per tensor)
//   r   = a * u_c                 (a = block max |x|; r = 0 when a == 0)
//   S   = E4M3 RNE saturating(r), D = value(S), d = D * t
//   inv = 1 / d, or 0 when d is zero or subnormal (every value becomes a signed 0)
//         (d and inv are per tensor and code: looked up in a per-workgroup table)
//   v_i = x_i * inv, code = E2M1 RNE(v_i) (hardware cvt, saturating at 6) or the
//         stochastic rounding below
//   e_i = fma(E(code_i), d, -x_i) (the exact error rounded once)
//   err = fma(e_i, e_i, err) for i ascending (2D: per row, then rows pairwise)
// and the block keeps candidate 4 iff err_4 < err_6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fos {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kScaleDenom = 2688.0f;  // largest E4M3 (448) * largest E2M1 (6)
constexpr float kMinNormal = 0x1p-126f;
constexpr int kMaxPartials = 1024;      // workgroups of the tensor-scale pass (a multiple of 4)

// ---- workgroup reductions (every thread of the workgroup must call these) ---------
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  __shared__ uint32_t part[16];
  const int nw = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = part[0];
  for (int w = 1; w < nw; ++w) m = max(m, part[w]);
  __syncthreads();
  return m;
}

// Running max of |bf16| over packed pairs: integer max of each 16-bit half with the
// sign cleared (for non-negative floats the bit order is the value order).
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
// fp32 bit pattern of the larger of the two packed bf16 magnitudes.
__device__ __forceinline__ uint32_t pk_max_to_f32_bits(uint32_t m) {
  return max(m & 0xffffu, m >> 16) << 16;
}

// Maximum of the n non-negative partial maxima written by the tensor-scale pass
// (n a multiple of 4, n <= 1024 = 4 * 256; `p` 16-byte aligned), by a workgroup of
// 256 threads: one 16-byte load per thread, then the workgroup max.
__device__ __forceinline__ float reduce_partials(const float* __restrict__ p, int n) {
  uint32_t m = 0;
  if (4 * (int)threadIdx.x < n) {
    const uint4 w = reinterpret_cast<const uint4*>(p)[threadIdx.x];
    m = max(max(w.x, w.y), max(w.z, w.w));
  }
  return __uint_as_float(block_max_u32(m));
}

// ---- bf16 ----------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack16(const uint4& a, const uint4& b, float (&x)[16]) {
  x[0] = bf16_lo(a.x);  x[1] = bf16_hi(a.x);  x[2] = bf16_lo(a.y);  x[3] = bf16_hi(a.y);
  x[4] = bf16_lo(a.z);  x[5] = bf16_hi(a.z);  x[6] = bf16_lo(a.w);  x[7] = bf16_hi(a.w);
  x[8] = bf16_lo(b.x);  x[9] = bf16_hi(b.x);  x[10] = bf16_lo(b.y); x[11] = bf16_hi(b.y);
  x[12] = bf16_lo(b.z); x[13] = bf16_hi(b.z); x[14] = bf16_lo(b.w); x[15] = bf16_hi(b.w);
}

// Round a finite fp32 to bf16 (nearest, ties to even); result in the low 16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// Two finite fp32 values -> packed bf16 (a in the low half), nearest-even, with the
// hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---- E4M3 (OCP "FN": bias 7, max 448) ------------------------------------------
// Round r >= 0 (or +inf) to the nearest E4M3 value, ties to even, saturating to 448:
// the bit-level definition that fos_selftest_e4m3 holds the hardware conversion to.
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  r = fminf(r, 448.0f);
  const uint32_t b = __float_as_uint(r);
  // normal range (r >= 2^-6): keep 3 mantissa bits, RNE on the fp32 pattern;
  // exponent re-biased from 127 to 7 (shift by 120 << 3 in the code domain).
  const uint32_t rounded = b + 0x7ffffu + ((b >> 20) & 1u);
  const uint32_t normal = (rounded >> 20) - (120u << 3);
  // subnormal range: uniform steps of 2^-9; rintf rounds to nearest even.
  const uint32_t sub = (uint32_t)rintf(r * 512.0f);
  return r < 0x1p-6f ? sub : normal;
}

// Exact value of a non-negative E4M3 code: placing the 7 code bits at fp32 bits
// 26..20 gives 2^(e-127)(1+m/8) (or m*2^-129 for e == 0); scaling by 2^120
// re-biases the exponent to 7.
__device__ __forceinline__ float e4m3_decode(uint32_t s) {
  return __uint_as_float(s << 20) * 0x1p120f;
}

// ---- E2M1 hardware conversions (scale operand 1.0 = no scaling) ------------------
// Two fp32 -> two E2M1 nibbles (round to nearest even, saturating at +-6, sign kept),
// written into byte `SEL` of `old`: first value in the low nibble.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_fp4(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}
// Byte `SEL` of `w` (two nibbles) -> two signed fp32 E2M1 values.
template <int SEL>
__device__ __forceinline__ f32x2 cvt_pk_f32_fp4(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// ---- Philox4x32-10 (Salmon et al., SC'11) ----------------------------------------
// Three-input exclusive or in one instruction (v_bitop3_b32 with truth table 0x96:
// the result bit is set where an odd number of the three input bits are).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4(xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1,
                   xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0);
  }
  return c;
}

// ---- stochastic rounding on the hardware conversion --------------------------------
// The draw rule: with lo and hi the E2M1 values around |v| (6 and above give 6),
// p = (|v| - lo) / (hi - lo) exact and p22 = p truncated to 22 fractional bits, |v|
// rounds up to hi iff q < p22, q = (k + 0.5) / 256 for the element's draw byte k.
//
// v_cvt_scalef32_sr_pk_fp4_f32 rounds the first value of its pair under a 32-bit
// operand R: it takes p to 22 fraction bits (p22: for |v| < 1, where fp32 resolves |v|
// more finely than 2^-22 of the 0.5 grid step, the bits below are dropped; above, p has
// at most 22) and the top 22 bits of R (R22), and rounds up iff p22 + R22 / 2^22 >= 1
// (saturating at 6, the sign of v kept).  With R = (~k << 24) | 0x7fffff,
// R22 = 2^22 (1 - q) - 1, so it rounds up iff p22 >= q + 2^-22, that is iff p22 > q (both
// are multiples of 2^-22): the draw rule.  The second value of the pair is rounded the
// same way under R shifted left by one (the bit shifted in does not reach the top 22
// bits), so it takes its element's operand shifted right by one.  fos_selftest_e2m1_sr
// checks both positions on the device for every finite fp32 value and every k.
//
// Operands of one block: byte i of the block's Philox output (counter
// (b_lo, b_hi, 0, stream)) is element i's draw k_i; r_i = (~k_i << 24) | 0x7fffff for
// even i (first position of pair i/2) and that shifted right by one for odd i (second
// position).
// (nw = ~(Philox word); fill = 0x7fffff)
template <int B>
__device__ __forceinline__ uint32_t sr_operand(uint32_t nw, uint32_t fill) {
  return __builtin_amdgcn_perm(nw, fill, 0x04020100u + ((uint32_t)B << 24));
}
__device__ __forceinline__ void sr_operands(uint64_t block, uint32_t stream, uint32_t k0,
                                            uint32_t k1, uint32_t (&r)[16]) {
  const uint4 w = philox4x32_10(make_uint4((uint32_t)block, (uint32_t)(block >> 32), 0u, stream),
                                k0, k1);
  const uint32_t nw[4] = {~w.x, ~w.y, ~w.z, ~w.w};
  // the fill constant in a vector register: the four selectors can then be scalar operands
  // (a VOP3 instruction takes at most one scalar operand)
  uint32_t fill;
  asm volatile("v_mov_b32 %0, 0x7fffff" : "=v"(fill));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    r[4 * m + 0] = sr_operand<0>(nw[m], fill);
    r[4 * m + 1] = sr_operand<1>(nw[m], fill) >> 1;
    r[4 * m + 2] = sr_operand<2>(nw[m], fill);
    r[4 * m + 3] = sr_operand<3>(nw[m], fill) >> 1;
  }
}
// Full-resolution draws: element i of the block takes the whole word i % 4 of the call
// with counter (b_lo, b_hi, i / 4, stream), four calls per block.  The conversion rounds
// the first value of a pair up iff p22 * 2^22 + (R >> 10) >= 2^22, and the second under
// R shifted left by one, so the first position takes the word and the second the word
// shifted right by one: both then round up iff p22 * 2^22 + (word >> 10) >= 2^22, a
// chance of exactly p22.  fos_selftest_e2m1_sr_full checks that boundary on the device.
__device__ __forceinline__ void sr_operands_full(uint64_t block, uint32_t stream, uint32_t k0,
                                                 uint32_t k1, uint32_t (&r)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 w = philox4x32_10(
        make_uint4((uint32_t)block, (uint32_t)(block >> 32), (uint32_t)j, stream), k0, k1);
    r[4 * j + 0] = w.x;
    r[4 * j + 1] = w.y >> 1;
    r[4 * j + 2] = w.z;
    r[4 * j + 3] = w.w >> 1;
  }
}
// Operands of a block's draws for stochastic-rounding mode kSR (1: 8-bit draws, 2: full
// resolution).
template <int kSR>
__device__ __forceinline__ void sr_draws(uint64_t block, uint32_t stream, uint32_t k0,
                                         uint32_t k1, uint32_t (&r)[16]) {
  if constexpr (kSR == 2)
    sr_operands_full(block, stream, k0, k1, r);
  else
    sr_operands(block, stream, k0, k1, r);
}

// Stochastic codes of the pair v = (v0, v1) into byte SEL of `w`, the other three bytes
// of `w` kept: under v0's operand the byte's low nibble is v0's code, under v1's
// (shifted) operand its high nibble is v1's code; the other nibble of the byte is then
// unspecified.  Scale operand 1.0 = no scaling.  The compiler's builtin for this
// instruction does not tie its `old` operand to the destination register, so the
// bytes it should keep are lost; a read-write inline-assembly operand keeps them (the
// instruction only reads and writes registers).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_fp4_byte(uint32_t w, f32x2 v, uint32_t r) {
  static_assert(SEL >= 0 && SEL < 4, "byte select");
  if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(w) : "v"(v), "v"(r));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(w) : "v"(v), "v"(r));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(w) : "v"(v), "v"(r));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(w) : "v"(v), "v"(r));
  return w;
}
// A register the code words start from: every byte is written before it is read, so
// its value does not matter and no instruction sets it.
__device__ __forceinline__ uint32_t any_word() {
  uint32_t w;
  asm volatile("" : "=v"(w));   // volatile: each call its own register, no copies
  return w;
}

// ---- random-sign 16-point Hadamard transform ---------------------------------------
// Butterflies with strides kFirst, ..., 8: (y_j, y_j+h) <- (y_j + y_j+h, y_j - y_j+h);
// from stride 1 the result is H16 y (Sylvester order).
template <int kFirst = 1>
__device__ __forceinline__ void fwht16(float (&y)[16]) {
#pragma unroll
  for (int h = kFirst; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      const float a = y[j], b = y[j + h];
      y[j] = a + b;
      y[j + h] = a - b;
    }
  }
}

// Sign bit k of the transform (bit k of `mask`) at bit 31.  The mask is the same for
// every lane, so these are scalar operations and each sign reaches the vector
// instruction as a scalar operand.
__device__ __forceinline__ uint32_t rht_sign_bit(uint32_t mask, int k) {
  return ((mask >> k) & 1u) << 31;
}

// Forward transform of bf16 values: y_k = x_k * (+-1/4) (sign k from bit k of `mask`),
// then H16.  The factor +-1/4 is the fp32 pattern of 1/4 (0x3e800000) with the sign
// bit set.  For a bf16 value x (8 significant bits, exponent at least -133) the product
// x * (+-1/4) is exact in fp32, so the first butterfly takes the odd element's factor
// inside a fused multiply-add: fma(x_odd, +-c_odd, x_even * c_even) is the rounded sum
// (or difference) of the two scaled values, bit for bit, signed zeros included, and the
// odd elements need no multiply of their own (8 VALU instructions fewer per block).
// Every caller passes values unpacked from bf16.
__device__ __forceinline__ void rht16(float (&y)[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const float ce = __uint_as_float(0x3e800000u | rht_sign_bit(mask, j));
    const float co = __uint_as_float(0x3e800000u | rht_sign_bit(mask, j + 1));
    const float a = y[j] * ce, b = y[j + 1];
    y[j] = __builtin_fmaf(b, co, a);
    y[j + 1] = __builtin_fmaf(b, -co, a);
  }
  fwht16<2>(y);
}

// Inverse transform ((H/4)^-1 = H/4, S^-1 = S): y_k *= 1/4, then H16, then the signs
// (a sign flip of the fp32 pattern).
__device__ __forceinline__ void irht16(float (&y)[16], uint32_t mask) {
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] *= 0.25f;
  fwht16(y);
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = __uint_as_float(__float_as_uint(y[k]) ^ rht_sign_bit(mask, k));
}

// ---- one candidate scale for one 16-value block ------------------------------------
struct Cand {
  uint32_t s;     // E4M3 byte
  uint32_t lo;    // nibbles of elements 0..7 (element 2k low nibble of byte k)
  uint32_t hi;    // nibbles of elements 8..15
  float err;      // sequential fp32 sum of squared errors
  float d;        // block decode scale D * t
};

// Per-tensor table of the decode scale and element reciprocal of every E4M3 code:
// entry S holds (d, inv) with d = D(S) * t and inv = 1 / d, or 0 when d is zero or
// subnormal; entry 128 holds (u6, u4) = (1 / (t * 6), 1 / (t * 4)).  d takes one of
// at most 127 values per tensor, so each workgroup computes the divisions once here
// instead of twice per block.  Built by a workgroup of at least 129 threads; ends
// with a workgroup barrier.
constexpr int kScaleTableSize = 129;
__device__ __forceinline__ void build_scale_table(float2* tab, float t) {
  const int i = threadIdx.x;
  if (i < 128) {
    const float d = e4m3_decode((uint32_t)i) * t;
    tab[i] = make_float2(d, (d >= kMinNormal) ? 1.0f / d : 0.0f);
  } else if (i == 128) {
    tab[128] = make_float2(1.0f / (t * 6.0f), 1.0f / (t * 4.0f));
  }
  __syncthreads();
}

// E4M3 scale bytes of both candidates of a block: r_c = RN(a * u_c), clamped to 448
// (0 when a == 0, also when u_c is infinite), converted by the hardware
// (v_cvt_pk_fp8_f32: OCP E4M3, nearest-even, subnormals kept) -- one instruction for
// the two candidates.  On [0, 448] the conversion returns e4m3_encode's code for
// every fp32 value; fos_selftest_e4m3 checks that exhaustively on the device.
__device__ __forceinline__ uint32_t e4m3_encode_pk_hw(float r0, float r1) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false) & 0xffffu;
}
__device__ __forceinline__ void cand_scale_bytes(float a, float u6, float u4, uint32_t& s6,
                                                 uint32_t& s4) {
  const bool zero = a == 0.0f;
  const float r6 = zero ? 0.0f : fminf(a * u6, 448.0f);
  const float r4 = zero ? 0.0f : fminf(a * u4, 448.0f);
  const uint32_t w = e4m3_encode_pk_hw(r6, r4);
  s6 = w & 0xffu;
  s4 = w >> 8;
}

// Decode scale and element reciprocal of a candidate's scale byte.
__device__ __forceinline__ void cand_lookup(uint32_t s, const float2* tab, float& d, float& inv) {
  const float2 e = tab[s];
  d = e.x;
  inv = e.y;
}

// Round-to-nearest-even codes of 16 values with the hardware conversion, and the
// sequential squared error of the dequantized values.
__device__ __forceinline__ void cand_codes_rne(const float (&x)[16], float d, float inv,
                                               Cand& c) {
  uint32_t lo = 0, hi = 0;
  lo = cvt_pk_fp4<0>(lo, x[0] * inv, x[1] * inv);
  lo = cvt_pk_fp4<1>(lo, x[2] * inv, x[3] * inv);
  lo = cvt_pk_fp4<2>(lo, x[4] * inv, x[5] * inv);
  lo = cvt_pk_fp4<3>(lo, x[6] * inv, x[7] * inv);
  hi = cvt_pk_fp4<0>(hi, x[8] * inv, x[9] * inv);
  hi = cvt_pk_fp4<1>(hi, x[10] * inv, x[11] * inv);
  hi = cvt_pk_fp4<2>(hi, x[12] * inv, x[13] * inv);
  hi = cvt_pk_fp4<3>(hi, x[14] * inv, x[15] * inv);
  f32x2 e[8];
  e[0] = cvt_pk_f32_fp4<0>(lo); e[1] = cvt_pk_f32_fp4<1>(lo);
  e[2] = cvt_pk_f32_fp4<2>(lo); e[3] = cvt_pk_f32_fp4<3>(lo);
  e[4] = cvt_pk_f32_fp4<0>(hi); e[5] = cvt_pk_f32_fp4<1>(hi);
  e[6] = cvt_pk_f32_fp4<2>(hi); e[7] = cvt_pk_f32_fp4<3>(hi);
  float err = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float e0 = __builtin_fmaf(e[j].x, d, -x[2 * j]);
    err = __builtin_fmaf(e0, e0, err);
    const float e1 = __builtin_fmaf(e[j].y, d, -x[2 * j + 1]);
    err = __builtin_fmaf(e1, e1, err);
  }
  c.lo = lo;
  c.hi = hi;
  c.err = err;
}

// Stochastic-rounding codes (hardware conversion under the draws' operands, see above)
// and the sequential squared error of the decoded values.  Each pair of elements is
// converted twice, once for each of its codes, into the byte of its pair; the two
// words of a half-block are merged nibble by nibble.
__device__ __forceinline__ void cand_codes_sr(const float (&x)[16], float d, float inv,
                                              const uint32_t (&r)[16], Cand& c) {
  // e*: byte j holds pair j's conversion under the even element's operand (low nibble
  // valid); o*: under the odd element's (high nibble valid); then one merge per word.
  uint32_t e0 = any_word(), o0 = any_word(), e1 = any_word(), o1 = any_word();
#define FOS_SR_PAIR(J, E, O)                                                          \
  {                                                                                   \
    const f32x2 v = {x[2 * (J)] * inv, x[2 * (J) + 1] * inv};                         \
    E = cvt_sr_fp4_byte<(J) & 3>(E, v, r[2 * (J)]);                                   \
    O = cvt_sr_fp4_byte<(J) & 3>(O, v, r[2 * (J) + 1]);                               \
  }
  FOS_SR_PAIR(0, e0, o0) FOS_SR_PAIR(1, e0, o0) FOS_SR_PAIR(2, e0, o0) FOS_SR_PAIR(3, e0, o0)
  FOS_SR_PAIR(4, e1, o1) FOS_SR_PAIR(5, e1, o1) FOS_SR_PAIR(6, e1, o1) FOS_SR_PAIR(7, e1, o1)
#undef FOS_SR_PAIR
  const uint32_t lo = (e0 & 0x0f0f0f0fu) | (o0 & 0xf0f0f0f0u);
  const uint32_t hi = (e1 & 0x0f0f0f0fu) | (o1 & 0xf0f0f0f0u);
  f32x2 e[8];
  e[0] = cvt_pk_f32_fp4<0>(lo); e[1] = cvt_pk_f32_fp4<1>(lo);
  e[2] = cvt_pk_f32_fp4<2>(lo); e[3] = cvt_pk_f32_fp4<3>(lo);
  e[4] = cvt_pk_f32_fp4<0>(hi); e[5] = cvt_pk_f32_fp4<1>(hi);
  e[6] = cvt_pk_f32_fp4<2>(hi); e[7] = cvt_pk_f32_fp4<3>(hi);
  float err = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float d0 = __builtin_fmaf(e[j].x, d, -x[2 * j]);
    err = __builtin_fmaf(d0, d0, err);
    const float d1 = __builtin_fmaf(e[j].y, d, -x[2 * j + 1]);
    err = __builtin_fmaf(d1, d1, err);
  }
  c.lo = lo;
  c.hi = hi;
  c.err = err;
}

// Store one block's nibbles and scale byte with non-temporal stores, for kernels whose
// workgroups write whole runs of consecutive blocks (the row-wise kernels): the
// outputs are written once and not read back, and keeping them out of the caches
// measurably shortens the quantize step.  Kernels that write scattered pieces of
// lines (tile, 2D) keep cached stores, which let L2 merge the pieces.
__device__ __forceinline__ void store_block_stream(uint8_t* data, uint8_t* scales,
                                                   int64_t data_off, int64_t scale_off,
                                                   const Cand& c) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(v2u{c.lo, c.hi}, reinterpret_cast<v2u*>(data + data_off));
  __builtin_nontemporal_store((uint8_t)c.s, scales + scale_off);
}

// Per-lane 16-value block amax (a chain of 3-input maxima with |.| modifiers).
__device__ __forceinline__ float amax16(const float (&x)[16]) {
  float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fabsf(x[2]));
#pragma unroll
  for (int i = 3; i < 15; i += 2) m = fmaxf(fmaxf(m, fabsf(x[i])), fabsf(x[i + 1]));
  return fmaxf(m, fabsf(x[15]));
}

// Quantize one 1D block with both candidates (or 6 alone) and return the winner.
template <bool kFourOverSix, bool kSR>
__device__ __forceinline__ Cand quantize_block(const float (&x)[16], const float2* tab,
                                               float u6, float u4, const uint32_t (&srr)[16]) {
  const float a = amax16(x);
  Cand c6, c4;
  float inv6, inv4;
  cand_scale_bytes(a, u6, u4, c6.s, c4.s);
  cand_lookup(c6.s, tab, c6.d, inv6);
  if (kSR) cand_codes_sr(x, c6.d, inv6, srr, c6); else cand_codes_rne(x, c6.d, inv6, c6);
  if (!kFourOverSix) return c6;
  cand_lookup(c4.s, tab, c4.d, inv4);
  if (kSR) cand_codes_sr(x, c4.d, inv4, srr, c4); else cand_codes_rne(x, c4.d, inv4, c4);
  return (c4.err < c6.err) ? c4 : c6;
}

}  // namespace fos
