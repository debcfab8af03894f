// MXFP4: 32 E2M1 values under one power-of-two E8M0 scale (Ultralytics glossary "FP4",
// section "How FP4 works": the OCP Microscaling format; section "FP4 for inference
// and training": MI350-class accelerators run it natively).
//
// Scale rule (the OCP MX specification's, which the page names): shared exponent
// e = floor(log2(max |x|)) - 2 clamped to [-127, 127] (-127 for a zero block), scale
// byte e + 127; elements are round-to-nearest-even E2M1 of x / 2^e, saturating at 6.
// Dividing by a power of two is exact, so the hardware conversion of x * 2^-e gives
// the codes directly.
//
// Kernels:
//   mx_quant_kernel     lane = one 32-value block (four 16-byte loads, one 16-byte
//                       store of nibbles, one scale byte); two blocks per lane.
//   mx_dequant_kernel   output-major like the NVFP4 one: value = E * 2^e.
//   mx_gemm_kernel      Y = deq(A) deq(B)^T on the scaled FP4 matrix cores
//                       (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E2M1): the
//                       packed bytes and E8M0 scales go to the MFMA as they are, with
//                       no conversion; 256x256 tiles, K staged through LDS in 256-wide
//                       double-buffered stages as in the NVFP4 qlinear kernel.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

using namespace gemm;

constexpr int kThreads = 256;

// Outputs are written once: non-temporal stores.  (The input stays on cached loads: a
// lane's four 16-byte loads are 64 bytes apart across the wave, and uncached they
// would fetch the shared lines more than once.)
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ quantize

// Shared exponent from the block maximum's fp32 pattern: floor(log2 a) = exponent
// field - 127 for normal a; zero and subnormal maxima clamp to -127.
__device__ __forceinline__ int mx_shared_exponent(float amax) {
  const int ef = (int)(__float_as_uint(amax) >> 23);
  return ef == 0 ? -127 : max(ef - 127 - 2, -127);
}

constexpr int kMxBlocksPerWG = 2 * kThreads;

__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const uint4* __restrict__ x,
                                                            int64_t nblk, uint8_t* __restrict__ data,
                                                            uint8_t* __restrict__ scales) {
  const int64_t b0 = (int64_t)blockIdx.x * kMxBlocksPerWG + threadIdx.x;
  uint4 w[8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t b = b0 + q * kThreads;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[4 * q + j] = make_uint4(0, 0, 0, 0);
    if (b < nblk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) w[4 * q + j] = x[4 * b + j];
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t b = b0 + q * kThreads;
    if (b >= nblk) break;
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 u = w[4 * q + j];
      v[8 * j + 0] = bf16_lo(u.x); v[8 * j + 1] = bf16_hi(u.x);
      v[8 * j + 2] = bf16_lo(u.y); v[8 * j + 3] = bf16_hi(u.y);
      v[8 * j + 4] = bf16_lo(u.z); v[8 * j + 5] = bf16_hi(u.z);
      v[8 * j + 6] = bf16_lo(u.w); v[8 * j + 7] = bf16_hi(u.w);
    }
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
#pragma unroll
    for (int i = 3; i < 31; i += 2) m = fmaxf(fmaxf(m, fabsf(v[i])), fabsf(v[i + 1]));
    m = fmaxf(m, fabsf(v[31]));
    const int e = mx_shared_exponent(m);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, e in [-127, 125]
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t r = 0;
      r = cvt_pk_fp4<0>(r, v[8 * k + 0] * inv, v[8 * k + 1] * inv);
      r = cvt_pk_fp4<1>(r, v[8 * k + 2] * inv, v[8 * k + 3] * inv);
      r = cvt_pk_fp4<2>(r, v[8 * k + 4] * inv, v[8 * k + 5] * inv);
      r = cvt_pk_fp4<3>(r, v[8 * k + 6] * inv, v[8 * k + 7] * inv);
      o[k] = r;
    }
    __builtin_nontemporal_store(v4u{o[0], o[1], o[2], o[3]}, reinterpret_cast<v4u*>(data) + b);
    __builtin_nontemporal_store((uint8_t)(e + 127), scales + b);
  }
}

// ------------------------------------------------------------------ dequantize

// 2^(s - 127) for an E8M0 byte (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

constexpr int kUnroll = 4;

template <bool kBF16>
__device__ __forceinline__ void mx_dequant_chunk(const uint8_t* __restrict__ data,
                                                 const uint8_t* __restrict__ scales, int64_t g,
                                                 void* __restrict__ out) {
  if (kBF16) {
    // 8 values = one 4-byte word of nibbles; block g/4
    const uint32_t q = reinterpret_cast<const uint32_t*>(data)[g];
    const float d = e8m0_value(scales[g >> 2]);
    const f32x2 e0 = cvt_pk_f32_fp4<0>(q), e1 = cvt_pk_f32_fp4<1>(q);
    const f32x2 e2 = cvt_pk_f32_fp4<2>(q), e3 = cvt_pk_f32_fp4<3>(q);
    uint4 o;
    o.x = pack_bf16x2(e0.x * d, e0.y * d);
    o.y = pack_bf16x2(e1.x * d, e1.y * d);
    o.z = pack_bf16x2(e2.x * d, e2.y * d);
    o.w = pack_bf16x2(e3.x * d, e3.y * d);
    __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(out) + g);
  } else {
    // 4 values = one 2-byte half-word of nibbles; block g/8
    const uint32_t q = reinterpret_cast<const uint16_t*>(data)[g];
    const float d = e8m0_value(scales[g >> 3]);
    const f32x2 e0 = cvt_pk_f32_fp4<0>(q), e1 = cvt_pk_f32_fp4<1>(q);
    typedef float v4f __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(v4f{e0.x * d, e0.y * d, e1.x * d, e1.y * d},
                                reinterpret_cast<v4f*>(out) + g);
  }
}

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint8_t* __restrict__ data,
                                                              const uint8_t* __restrict__ scales,
                                                              int64_t nchunk, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; g + (kUnroll - 1) * stride < nchunk; g += kUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mx_dequant_chunk<kBF16>(data, scales, g + u * stride, out);
  }
  for (; g < nchunk; g += stride) mx_dequant_chunk<kBF16>(data, scales, g, out);
}

// ------------------------------------------------------------------ GEMM
// K stage of 256: per row 128 bytes of nibbles (8 granules of 16 bytes = 32 values,
// XOR-swizzled as in the NVFP4 kernel) and 8 E8M0 bytes.  Two stages of 68 KB.
constexpr int kMxSuper = 256;
constexpr int kMxRowBytes = kMxSuper / 2;
constexpr int kMxRowScales = kMxSuper / 32;
constexpr int kMxTile = 256;

struct MxStage {
  uint8_t a[kMxTile * kMxRowBytes];
  uint8_t b[kMxTile * kMxRowBytes];
  uint8_t sa[kMxTile * kMxRowScales];
  uint8_t sb[kMxTile * kMxRowScales];
};

struct MxOperands {
  __amdgpu_buffer_rsrc_t a, sa, b, sb;
  uint32_t oa[2], ob[2];      // per-lane data offsets for even / odd row-groups
  uint32_t osa, osb;          // per-lane scale offsets
  uint32_t group_stride;      // bytes between data row-groups (8 rows)
  uint32_t scale_stride;      // bytes between scale row-groups (32 rows)
};

// This wave's share of one stage: 64 rows of each operand, 8 + 8 data copies (8 rows
// of 128 bytes each) and 2 + 2 scale copies (32 rows of 8 bytes each), issued as two
// halves of 10 copies (half j: data row-groups 4j..4j+3 and scale row-group j).
__device__ __forceinline__ void mx_stage_load_half(MxStage& st, const MxOperands& p, int sc,
                                                   int wave, int j) {
  const int od = sc * kMxRowBytes, os = sc * kMxRowScales;
#pragma unroll
  for (int q = 4 * j; q < 4 * j + 4; ++q) {
    const int so = od + q * (int)p.group_stride;
    dma16(p.a, st.a + (64 * wave + 8 * q) * kMxRowBytes, p.oa[q & 1], so);
    dma16(p.b, st.b + (64 * wave + 8 * q) * kMxRowBytes, p.ob[q & 1], so);
  }
  const int so = os + j * (int)p.scale_stride;
  dma4(p.sa, st.sa + (64 * wave + 32 * j) * kMxRowScales, p.osa, so);
  dma4(p.sb, st.sb + (64 * wave + 32 * j) * kMxRowScales, p.osb, so);
}
__device__ __forceinline__ void mx_stage_load(MxStage& st, const MxOperands& p, int sc, int wave) {
  mx_stage_load_half(st, p, sc, wave, 0);
  mx_stage_load_half(st, p, sc, wave, 1);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 mx_operand(const uint8_t* base, int row, int g) {
  const uint4 v =
      *reinterpret_cast<const uint4*>(base + row * kMxRowBytes + ((g ^ ((row >> 1) & 7)) << 4));
  return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// Multiply the four 64-wide k-steps of a stage, and (kLoad) copy stage `next_sc` of
// the operands into `next` meanwhile.  In k-step s, lane (lr, h) supplies row lr's 32
// values of k block 2s + h (granule 2s + h) and that block's E8M0 scale (byte 2s + h
// of the row's 8).  All scale bytes and the first k-step's operands are read up
// front; each k-step's 8 operand reads for the next k-step are issued between its
// first 8 MFMAs (scheduling groups: one MFMA, one LDS read), so that every read has
// at least 8 MFMAs (about 256 cycles) to land.  The next stage's 20 copies go out in
// k-steps 0 and 1, one after each of their first 10 MFMAs, leaving k-steps 2 and 3
// for them to land.  (Issued in one burst, the copies hold up the wave's instruction
// stream for hundreds of cycles while the matrix pipe idles; left to itself the
// scheduler also reads each operand right before its first use and waits for it.)
constexpr int NKS = kMxSuper / 64;
template <bool kLoad>
__device__ __forceinline__ void mx_stage_mma(const MxStage& st, f32x16 (&acc)[4][4], int ra,
                                             int rb, int h, MxStage& next, const MxOperands& p,
                                             int next_sc, int wave) {
  __builtin_amdgcn_sched_barrier(0);
  uint2 sa[4], sb[4];
  i32x8 A[4], B[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa[i] = *reinterpret_cast<const uint2*>(st.sa + (ra + 32 * i) * kMxRowScales);
    sb[i] = *reinterpret_cast<const uint2*>(st.sb + (rb + 32 * i) * kMxRowScales);
    A[i] = mx_operand(st.a, ra + 32 * i, h);
    B[i] = mx_operand(st.b, rb + 32 * i, h);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int sh = 8 * h;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    int xa[4], xb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xa[i] = (int)(((s < 2) ? sa[i].x : sa[i].y) >> (16 * (s & 1) + sh));
      xb[i] = (int)(((s < 2) ? sb[i].x : sb[i].y) >> (16 * (s & 1) + sh));
    }
    i32x8 An[4], Bn[4];
    if (s + 1 < NKS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        An[i] = mx_operand(st.a, ra + 32 * i, 2 * (s + 1) + h);
        Bn[i] = mx_operand(st.b, rb + 32 * i, 2 * (s + 1) + h);
      }
    }
    const bool copies = kLoad && s < 2;
    if (copies) mx_stage_load_half(next, p, next_sc, wave, s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[i][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[i], B[n], acc[i][n], 4, 4,
                                                                     0, xa[i], 0, xb[n]);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);       // the 8 scale shifts
    if (s + 1 < NKS) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        if (copies) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one copy
      }
      if (copies) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < NKS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = An[i];
        B[i] = Bn[i];
      }
    }
  }
  // MFMAs touch no memory, so without this the scheduler may sink them below the
  // next workgroup barrier
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mx_gemm_kernel(const uint8_t* __restrict__ ad, const uint8_t* __restrict__ as,
                    const uint8_t* __restrict__ bd, const uint8_t* __restrict__ bs, int M, int N,
                    int K, int tiles_m, int tiles_n, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) MxStage st0;
  __shared__ __attribute__((aligned(16))) MxStage st1;
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const int tm = tc.tm, tn = tc.tn;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, h = lane >> 5;
  const uint32_t kb2 = K / 2, kb32 = K / 32;

  MxOperands p;
  p.a = __builtin_amdgcn_make_buffer_rsrc((void*)ad, 0, (int)((uint32_t)M * kb2), kRsrcWord3);
  p.sa = __builtin_amdgcn_make_buffer_rsrc((void*)as, 0, (int)((uint32_t)M * kb32), kRsrcWord3);
  p.b = __builtin_amdgcn_make_buffer_rsrc((void*)bd, 0, (int)((uint32_t)N * kb2), kRsrcWord3);
  p.sb = __builtin_amdgcn_make_buffer_rsrc((void*)bs, 0, (int)((uint32_t)N * kb32), kRsrcWord3);
  {
    // data: DMA lane l of row-group q writes LDS slot (l & 7) of local row 64*wave +
    // 8*q + (l >> 3) and fetches the granule the swizzle puts there
    const int sub = lane >> 3, slot = lane & 7;
    const int r0 = 64 * wave + sub;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const uint32_t g = slot ^ (((sub >> 1) + 4 * par) & 7);
      p.oa[par] = (uint32_t)(tm * kMxTile + r0) * kb2 + 16 * g;
      p.ob[par] = (uint32_t)(tn * kMxTile + r0) * kb2 + 16 * g;
    }
    p.group_stride = 8 * kb2;
    // scales: lane l of copy j fetches dword l & 1 of local row 64*wave + 32*j + l/2
    const int srow = 64 * wave + (lane >> 1);
    p.osa = (uint32_t)(tm * kMxTile + srow) * kb32 + 4 * (lane & 1);
    p.osb = (uint32_t)(tn * kMxTile + srow) * kb32 + 4 * (lane & 1);
    p.scale_stride = 32 * kb32;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

  const int ra = (wave >> 1) * 128 + lr;
  const int rb = (wave & 1) * 128 + lr;
  const int nsc = K / kMxSuper;
  mx_stage_load(st0, p, 0, wave);
  int sc = 0;
  for (; sc + 1 < nsc; sc += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    mx_stage_mma<true>(st0, acc, ra, rb, h, st1, p, sc + 1, wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // unconditional (a redundant copy of the last stage when none is left): a branch
    // here lets the compiler sink the previous stage's MFMAs past the barrier
    mx_stage_mma<true>(st1, acc, ra, rb, h, st0, p, min(sc + 2, nsc - 1), wave);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (sc < nsc) mx_stage_mma<false>(st0, acc, ra, rb, h, st1, p, 0, wave);
  store_tile(y, M, N, tm, tn, wave, lr, h, 1.0f, acc);
}

}  // namespace

int64_t mx_quantize_grid(int64_t rows, int64_t cols) {
  return (rows * cols / 32 + kMxBlocksPerWG - 1) / kMxBlocksPerWG;
}

int64_t mx_gemm_grid(int64_t M, int64_t N) {
  return ((M + kMxTile - 1) / kMxTile) * ((N + kMxTile - 1) / kMxTile);
}

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* data,
                              uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * cols / 32;
  if (nblk == 0) return hipSuccess;
  const int64_t grid = mx_quantize_grid(rows, cols);
  mx_quant_kernel<<<grid, kThreads, 0, s>>>((const uint4*)x, nblk, data, scales);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* data, const uint8_t* scales, int64_t rows,
                                int64_t cols, bool bf16_out, void* out, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const int64_t nchunk = bf16_out ? n / 8 : n / 4;
  int64_t grid = (nchunk + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (grid > 8192) grid = 8192;
  if (bf16_out)
    mx_dequant_kernel<true><<<grid, kThreads, 0, s>>>(data, scales, nchunk, out);
  else
    mx_dequant_kernel<false><<<grid, kThreads, 0, s>>>(data, scales, nchunk, out);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t* ad, const uint8_t* as, const uint8_t* bd,
                          const uint8_t* bs, int64_t M, int64_t N, int64_t K, uint16_t* y,
                          hipStream_t s) {
  const int tiles_m = (int)((M + kMxTile - 1) / kMxTile);
  const int tiles_n = (int)((N + kMxTile - 1) / kMxTile);
  mx_gemm_kernel<<<tiles_m * tiles_n, 256, 0, s>>>(ad, as, bd, bs, (int)M, (int)N, (int)K,
                                                   tiles_m, tiles_n, y);
  return hipGetLastError();
}

}  // namespace fos
