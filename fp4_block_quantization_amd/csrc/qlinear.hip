// Simulated quantized linear forward, Y = deq(Xq) . deq(Wq)^T (Four Over Six
// documentation page, section "Four Over Six": where native FP4 matrix operations
// are missing, the quantized linear layer is simulated with a higher-precision
// matrix multiplication of the dequantized operands; Ultralytics glossary "FP4",
// section "FP4 for inference and training": FP4 products accumulate in higher
// precision).
//
// Every dequantized operand value E2M1 * E4M3 has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16; fp16 x fp16 products are exact in
// fp32.  The kernel therefore forms E*D in fp16 registers (hardware E2M1->f16 and
// E4M3->f16 conversions, one packed f16 multiply per pair) and feeds them straight to
// v_mfma_f32_32x32x16_f16 with fp32 accumulation; the tensor scales t_x * t_w are
// applied in fp32 in the epilogue, then the result is rounded to bf16.
//
// Tiling: a 256-thread workgroup owns a 256x256 tile of Y, each wave a 128x128
// quarter held as 4x4 MFMA accumulators (256 fp32 per lane).  Both operands are
// K-major, so a lane's 8 MFMA k-slots come from one 4-byte word of packed nibbles; A
// and B use the same k mapping, so the reordering of k inside a chunk cancels in the
// sum.  Two kernels:
//   qlinear_lds_kernel (K % 256 == 0): packed operands are copied global -> LDS in
//     256-wide K stages (double-buffered) and dequantized from LDS, software-pipelined
//     against the MFMAs;
//   qlinear_kernel (any K % 64 == 0): each wave reads its packed operands straight
//     from L2 into registers, three register stages deep.
// Workgroups are remapped so that each XCD (dispatched round-robin) runs a contiguous
// group of 4 tile-rows x all tile-columns.
#include "device_common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

using namespace gemm;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;

__device__ __forceinline__ h8 dequant8(uint32_t w, h2 dd) {
  const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * dd;
  const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * dd;
  const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * dd;
  const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * dd;
  return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ uint32_t word(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------- register-staged kernel
// Packed operands of one 64-wide K chunk for one lane: 16 bytes of nibbles per A row
// tile and per B column tile, and the two E4M3 scale bytes that cover them.  Lane
// half h (lane / 32) takes the 32 consecutive k values [32h, 32h + 32) of the chunk
// in one 16-byte load per row, and k-step j uses word j of it.
template <int TI, int TJ>
struct Stage {
  uint4 a[TI], b[TJ];
  uint32_t sa[TI], sb[TJ];
};

// Operands are read through buffer resources (descriptor in SGPRs, 32-bit per-lane
// byte offsets): rows past M or N fall outside the resource and read as zero, and
// the per-chunk advance is a scalar offset.
template <int TI, int TJ>
struct Operands {
  __amdgpu_buffer_rsrc_t a, sa, b, sb;
  uint32_t oa[TI], osa[TI], ob[TJ], osb[TJ];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The four scale bytes of a row's chunk are one aligned dword; lane half h uses
// bytes 2h and 2h + 1 (selected when the scales are converted).
template <int TI, int TJ>
__device__ __forceinline__ void load_stage(Stage<TI, TJ>& st, const Operands<TI, TJ>& p, int kc) {
  const int ob = kc * (kChunk / 2), os = kc * (kChunk / 16);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    st.a[i] = ld16(p.a, p.oa[i], ob);
    st.sa[i] = __builtin_amdgcn_raw_buffer_load_b32(p.sa, p.osa[i], os, 0);
  }
#pragma unroll
  for (int n = 0; n < TJ; ++n) {
    st.b[n] = ld16(p.b, p.ob[n], ob);
    st.sb[n] = __builtin_amdgcn_raw_buffer_load_b32(p.sb, p.osb[n], os, 0);
  }
}

template <int TI, int TJ>
__device__ __forceinline__ void mma_stage(const Stage<TI, TJ>& st, f32x16 (&acc)[TI][TJ],
                                          uint32_t sh) {
  h2 da[TI][2], db[TJ][2];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const h2 sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(st.sa[i] >> sh, 1.0f, false);
    da[i][0] = h2{sa.x, sa.x};
    da[i][1] = h2{sa.y, sa.y};
  }
#pragma unroll
  for (int n = 0; n < TJ; ++n) {
    const h2 sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(st.sb[n] >> sh, 1.0f, false);
    db[n][0] = h2{sb.x, sb.x};
    db[n][1] = h2{sb.y, sb.y};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h8 A[TI], B[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) A[i] = dequant8(word(st.a[i], j), da[i][j >> 1]);
#pragma unroll
    for (int n = 0; n < TJ; ++n) B[n] = dequant8(word(st.b[n], j), db[n][j >> 1]);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int n = 0; n < TJ; ++n)
        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[n], acc[i][n], 0, 0, 0);
  }
}

// Workgroup = 4 waves in a 2x2 arrangement; each wave owns TI x TJ MFMA tiles of
// 32x32, so the workgroup tile is (64*TI) x (64*TJ); WAVES_PER_EU waves share a SIMD.
template <int TI, int TJ, int STAGES, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void qlinear_kernel(const uint8_t* __restrict__ xd, const uint8_t* __restrict__ xs,
                    const float* __restrict__ xt, const uint8_t* __restrict__ wd,
                    const uint8_t* __restrict__ ws, const float* __restrict__ wt, int M, int N,
                    int K, int tiles_m, int tiles_n, uint16_t* __restrict__ y) {
  constexpr int kWM = 32 * TI, kWN = 32 * TJ;     // wave tile
  constexpr int kBM = 2 * kWM, kBN = 2 * kWN;     // workgroup tile
  // ---- tile assignment: contiguous range per XCD, grouped along M inside it
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const int tm = tc.tm, tn = tc.tn;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int m0 = tm * kBM + (wave >> 1) * kWM;
  const int n0 = tn * kBN + (wave & 1) * kWN;
  const uint32_t kb2 = K / 2, kb16 = K / 16;
  const uint32_t sh = 16 * h;   // this lane's scale byte pair within the dword

  Operands<TI, TJ> p;
  p.a = __builtin_amdgcn_make_buffer_rsrc((void*)xd, 0, (int)((uint32_t)M * kb2), kRsrcWord3);
  p.sa = __builtin_amdgcn_make_buffer_rsrc((void*)xs, 0, (int)((uint32_t)M * kb16), kRsrcWord3);
  p.b = __builtin_amdgcn_make_buffer_rsrc((void*)wd, 0, (int)((uint32_t)N * kb2), kRsrcWord3);
  p.sb = __builtin_amdgcn_make_buffer_rsrc((void*)ws, 0, (int)((uint32_t)N * kb16), kRsrcWord3);
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const uint32_t r = m0 + 32 * i + lr;
    p.oa[i] = r * kb2 + 16 * h;
    p.osa[i] = r * kb16;
  }
#pragma unroll
  for (int n = 0; n < TJ; ++n) {
    const uint32_t c = n0 + 32 * n + lr;
    p.ob[n] = c * kb2 + 16 * h;
    p.osb[n] = c * kb16;
  }

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int n = 0; n < TJ; ++n) acc[i][n] = f32x16{};

  // register stages: chunk kc is multiplied while the next STAGES-1 chunks load
  const int nk = K / kChunk;
  Stage<TI, TJ> st[STAGES];
  int kc = 0;
  if (nk >= 2 * STAGES) {
    // unconditional prologue and a branch-free steady state, so the compiler can
    // wait on exactly the stage it consumes (any guarded load in or before the loop
    // makes it wait for every load instead); scheduling barriers keep each stage's
    // refill right after its last use (left alone, the scheduler sinks all refills
    // to the end of the loop body)
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      load_stage(st[s], p, s);
      __builtin_amdgcn_sched_barrier(0);   // keep stage order: stage 0 must be oldest
    }
    for (; kc + 2 * STAGES - 1 < nk; kc += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        mma_stage(st[s], acc, sh);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(st[s], p, kc + s + STAGES);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nk) load_stage(st[s], p, s);
  }
  for (; kc < nk; kc += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      if (kc + s < nk) {
        mma_stage(st[s], acc, sh);
        if (kc + s + STAGES < nk) load_stage(st[s], p, kc + s + STAGES);
      }
    }
  }

  // ---- epilogue: lane (lr, h) holds, for accumulator element a, row
  // (a & 3) + 8 * (a >> 2) + 4 * h and column lr of each 32x32 tile.
  const float s = xt[0] * wt[0];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int n = 0; n < TJ; ++n) {
      const int col = n0 + 32 * n + lr;
      if (col >= N) continue;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int row = m0 + 32 * i + (a & 3) + 8 * (a >> 2) + 4 * h;
        if (row < M) y[(int64_t)row * N + col] = (uint16_t)f32_to_bf16_rne(acc[i][n][a] * s);
      }
    }
  }
}

// ---------------------------------------------------------------- LDS-staged kernel
// K is consumed in super-chunks of 256 (128 bytes of nibbles and 16 scale bytes per
// row).  Each super-chunk of the workgroup's 256 A rows and 256 B rows is copied
// global -> LDS with buffer loads that write LDS directly (no VGPRs): a wave
// instruction moves 8 rows x 128 bytes, i.e. whole cache lines, so the L1 sees one
// request per line instead of one per 32-byte piece.  The 16-byte granules of a row
// are XOR-swizzled (slot = granule ^ ((row >> 1) & 7)) so that the per-lane
// ds_read_b128 of 16 consecutive rows hits distinct banks.  Two LDS stages of 72 KB:
// the next super-chunk is in flight while the current one is multiplied, with one
// workgroup barrier per super-chunk.
constexpr int kSuper = 256;                 // K per LDS stage
constexpr int kRowBytes = kSuper / 2;       // 128 bytes of nibbles per row per stage
constexpr int kRowScales = kSuper / 16;     // 16 scale bytes per row per stage
constexpr int kTileRows = 256;
constexpr int kDataBytes = kTileRows * kRowBytes;     // 32 KB per operand
constexpr int kScaleBytes = kTileRows * kRowScales;   // 4 KB per operand

struct LdsStage {
  uint8_t a[kDataBytes];
  uint8_t b[kDataBytes];
  uint8_t sa[kScaleBytes];
  uint8_t sb[kScaleBytes];
};

struct LdsOperands {
  __amdgpu_buffer_rsrc_t a, sa, b, sb;
  uint32_t oa[2], ob[2];      // per-lane offsets for even / odd row-groups
  uint32_t osa, osb;          // per-lane scale-row offsets
  uint32_t group_stride;      // bytes between row-groups (8 rows)
};

// This wave's share of one super-chunk: 8 + 8 data instructions and 1 + 1 scale
// instructions (64 rows of each operand per wave).  Row-group q of the wave starts
// 8*q rows further on; the granule swizzle only depends on q's parity, so the
// per-lane offset is one of two values and the rest is a scalar offset.  Part j < 8
// copies row-group j of both operands, part 8 both scale blocks.
__device__ __forceinline__ void stage_load_part(LdsStage& st, const LdsOperands& p, int sc,
                                                int wave, int j) {
  if (j < 8) {
    const int so = sc * kRowBytes + j * (int)p.group_stride;
    dma16(p.a, st.a + (64 * wave + 8 * j) * kRowBytes, p.oa[j & 1], so);
    dma16(p.b, st.b + (64 * wave + 8 * j) * kRowBytes, p.ob[j & 1], so);
  } else {
    const int os = sc * kRowScales;
    dma16(p.sa, st.sa + 64 * wave * kRowScales, p.osa, os);
    dma16(p.sb, st.sb + 64 * wave * kRowScales, p.osb, os);
  }
}
constexpr int kLoadParts = 9;
__device__ __forceinline__ void stage_load(LdsStage& st, const LdsOperands& p, int sc, int wave) {
#pragma unroll
  for (int j = 0; j < kLoadParts; ++j) stage_load_part(st, p, sc, wave, j);
}

template <bool kHi>
__device__ __forceinline__ h2 scale_pair(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
}

__device__ __forceinline__ uint4 lds_granule(const uint8_t* base, int row, int g) {
  return *reinterpret_cast<const uint4*>(base + row * kRowBytes + ((g ^ ((row >> 1) & 7)) << 4));
}

// E4M3 scale pairs of granule group gq as fp16 pairs (d[i][0] for the group's first 16
// k values, d[i][1] for the next 16).
__device__ __forceinline__ void group_scales(const uint2 (&sc)[4], int gq, h2 (&d)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (gq < 2) ? sc[i].x : sc[i].y;
    const h2 pr = (gq & 1) ? scale_pair<true>(w) : scale_pair<false>(w);
    d[i][0] = h2{pr.x, pr.x};
    d[i][1] = h2{pr.y, pr.y};
  }
}

// Multiply one super-chunk held in LDS: 16 k-steps of 16 MFMAs (4 granule groups of
// 4 k-steps).  Software-pipelined: the operands of k-step s + 1 are dequantized while
// the 16 MFMAs of k-step s issue (one MFMA, then up to five VALU instructions,
// repeated), so the conversion runs in the MFMA pipe's shadow instead of in front of
// it; the next group's granules are read from LDS three k-steps before they are used.
// With kLoad, the copies of super-chunk `next_sc` into `next` go out two per k-step
// in k-steps 0-8, right after the k-step's first MFMA, which leaves seven k-steps for
// them to land.  (Issued in one burst, they hold up the wave's in-order instruction
// stream while the matrix pipe idles.)
template <bool kLoad>
__device__ __forceinline__ void stage_mma(const LdsStage& st, f32x16 (&acc)[4][4], int ra,
                                          int rb, int h, LdsStage& next, const LdsOperands& p,
                                          int next_sc, int wave) {
  uint2 sca[4], scb[4];
  uint4 ga[4], gb[4], na[4], nb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sca[i] = *reinterpret_cast<const uint2*>(st.sa + (ra + 32 * i) * kRowScales + 8 * h);
    scb[i] = *reinterpret_cast<const uint2*>(st.sb + (rb + 32 * i) * kRowScales + 8 * h);
    ga[i] = lds_granule(st.a, ra + 32 * i, 4 * h);
    gb[i] = lds_granule(st.b, rb + 32 * i, 4 * h);
  }
  h2 da[4][2], db[4][2];
  group_scales(sca, 0, da);
  group_scales(scb, 0, db);
  h8 A[4], B[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    A[i] = dequant8(word(ga[i], 0), da[i][0]);
    B[i] = dequant8(word(gb[i], 0), db[i][0]);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int gq = s >> 2, jj = s & 3;
    if (jj == 0 && gq < 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        na[i] = lds_granule(st.a, ra + 32 * i, 4 * h + gq + 1);
        nb[i] = lds_granule(st.b, rb + 32 * i, 4 * h + gq + 1);
      }
    }
    h8 An[4], Bn[4];
    if (s < 15) {
      const int gq1 = (s + 1) >> 2, jj1 = (s + 1) & 3;
      if (jj1 == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ga[i] = na[i];
          gb[i] = nb[i];
        }
        group_scales(sca, gq1, da);
        group_scales(scb, gq1, db);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        An[i] = dequant8(word(ga[i], jj1), da[i][jj1 >> 1]);
        Bn[i] = dequant8(word(gb[i], jj1), db[i][jj1 >> 1]);
      }
    }
    const bool copies = kLoad && s < kLoadParts;
    if (copies) stage_load_part(next, p, next_sc, wave, s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[n], acc[i][n], 0, 0, 0);
    if (jj == 0 && gq < 3) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      if (copies && m == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // the copies
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then up to five VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s < 15) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = An[i];
        B[i] = Bn[i];
      }
    }
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void qlinear_lds_kernel(const uint8_t* __restrict__ xd, const uint8_t* __restrict__ xs,
                        const float* __restrict__ xt, const uint8_t* __restrict__ wd,
                        const uint8_t* __restrict__ ws, const float* __restrict__ wt, int M,
                        int N, int K, int tiles_m, int tiles_n, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) LdsStage st0;
  __shared__ __attribute__((aligned(16))) LdsStage st1;
  // ---- tile assignment: contiguous range per XCD, grouped along M inside it
  const TileCoord tc = tile_of(blockIdx.x, tiles_m, tiles_n);
  const int tm = tc.tm, tn = tc.tn;

  // the wave index is made explicitly uniform so that the LDS destinations of the
  // direct loads (M0) are scalar values rather than per-lane registers
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 31, h = lane >> 5;
  const uint32_t kb2 = K / 2, kb16 = K / 16;

  LdsOperands p;
  p.a = __builtin_amdgcn_make_buffer_rsrc((void*)xd, 0, (int)((uint32_t)M * kb2), kRsrcWord3);
  p.sa = __builtin_amdgcn_make_buffer_rsrc((void*)xs, 0, (int)((uint32_t)M * kb16), kRsrcWord3);
  p.b = __builtin_amdgcn_make_buffer_rsrc((void*)wd, 0, (int)((uint32_t)N * kb2), kRsrcWord3);
  p.sb = __builtin_amdgcn_make_buffer_rsrc((void*)ws, 0, (int)((uint32_t)N * kb16), kRsrcWord3);
  {
    // DMA lane l of row-group q writes LDS slot (l & 7) of local row 64*wave + 8*q +
    // (l >> 3); it fetches the granule that the swizzle puts in that slot:
    // g = slot ^ ((row >> 1) & 7) = slot ^ (((l >> 4) + 4 * (q & 1)) & 7).
    const int sub = lane >> 3, slot = lane & 7;
    const int r0 = 64 * wave + sub;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const uint32_t g = slot ^ (((sub >> 1) + 4 * par) & 7);
      p.oa[par] = (uint32_t)(tm * kTileRows + r0) * kb2 + 16 * g;
      p.ob[par] = (uint32_t)(tn * kTileRows + r0) * kb2 + 16 * g;
    }
    p.group_stride = 8 * kb2;
    p.osa = (uint32_t)(tm * kTileRows + 64 * wave + lane) * kb16;
    p.osb = (uint32_t)(tn * kTileRows + 64 * wave + lane) * kb16;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

  const int ra = (wave >> 1) * 128 + lr;     // this lane's first A row in the tile
  const int rb = (wave & 1) * 128 + lr;      // and first B row
  const int nsc = K / kSuper;
  // Each step: wait for this wave's copies of the stage about to be used, barrier
  // (so every wave's copies have landed and the other stage is no longer read), then
  // multiply while copying the next super-chunk into the other stage.  A single-exit
  // loop keeps the 256 accumulator registers in place.
  stage_load(st0, p, 0, wave);
  int sc = 0;
  for (; sc + 1 < nsc; sc += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stage_mma<true>(st0, acc, ra, rb, h, st1, p, sc + 1, wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // unconditional (a redundant copy of the last super-chunk when none is left): a
    // branch here lets the compiler sink the previous stage's MFMAs past the barrier
    stage_mma<true>(st1, acc, ra, rb, h, st0, p, min(sc + 2, nsc - 1), wave);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (sc < nsc) stage_mma<false>(st0, acc, ra, rb, h, st1, p, 0, wave);

  store_tile(y, M, N, tm, tn, wave, lr, h, xt[0] * wt[0], acc);
}

hipError_t launch_lds(const uint8_t* xd, const uint8_t* xs, const float* xt, const uint8_t* wd,
                      const uint8_t* ws, const float* wt, int64_t M, int64_t N, int64_t K,
                      uint16_t* y, hipStream_t s) {
  const int tiles_m = (int)((M + kTileRows - 1) / kTileRows);
  const int tiles_n = (int)((N + kTileRows - 1) / kTileRows);
  qlinear_lds_kernel<<<tiles_m * tiles_n, 256, 0, s>>>(xd, xs, xt, wd, ws, wt, (int)M, (int)N,
                                                       (int)K, tiles_m, tiles_n, y);
  return hipGetLastError();
}

template <int TI, int TJ, int STAGES, int WPE>
hipError_t launch_cfg(const uint8_t* xd, const uint8_t* xs, const float* xt, const uint8_t* wd,
                      const uint8_t* ws, const float* wt, int64_t M, int64_t N, int64_t K,
                      uint16_t* y, hipStream_t s) {
  constexpr int kBM = 64 * TI, kBN = 64 * TJ;
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + kBN - 1) / kBN);
  qlinear_kernel<TI, TJ, STAGES, WPE><<<tiles_m * tiles_n, 256, 0, s>>>(
      xd, xs, xt, wd, ws, wt, (int)M, (int)N, (int)K, tiles_m, tiles_n, y);
  return hipGetLastError();
}

}  // namespace

// Both kernels tile the output in 256 x 256 blocks (launch_cfg<4, 4, ...>: 64 * 4).
int64_t qlinear_grid(int64_t M, int64_t N) {
  static_assert(64 * 4 == kTileRows, "both qlinear kernels use the same output tile");
  return ((M + kTileRows - 1) / kTileRows) * ((N + kTileRows - 1) / kTileRows);
}

hipError_t launch_qlinear(const uint8_t* xd, const uint8_t* xs, const float* xt,
                          const uint8_t* wd, const uint8_t* ws, const float* wt, int64_t M,
                          int64_t N, int64_t K, uint16_t* y, hipStream_t s) {
  // K in whole 256-wide super-chunks: LDS-staged kernel; otherwise (K % 64 == 0) the
  // register-staged kernel
  if (K % kSuper == 0) return launch_lds(xd, xs, xt, wd, ws, wt, M, N, K, y, s);
  return launch_cfg<4, 4, 3, 1>(xd, xs, xt, wd, ws, wt, M, N, K, y, s);
}

}  // namespace fos
