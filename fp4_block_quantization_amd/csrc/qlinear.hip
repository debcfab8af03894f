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
// K-major, so a lane's 8 MFMA k-slots come from one 4-byte word of packed nibbles:
// for a 64-wide K chunk, lane half h (lane / 32) takes the 32 consecutive k values
// [32h, 32h + 32) in one 16-byte load per row, and k-step j uses word j.  A and B use
// the same k mapping, so the reordering of k inside the chunk cancels in the sum.
// No LDS is used: each wave reads its packed operands straight from L2 (the 2x
// re-read within a workgroup is 4 KB per wave per chunk), and the next chunk is
// prefetched into registers while the current one is multiplied.  Workgroups are
// remapped so that each XCD (dispatched round-robin) runs a contiguous group of
// 4 tile-rows x all tile-columns.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;
constexpr int kChunk = 64;
constexpr int kGroupM = 4;

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

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void qlinear_kernel(const uint8_t* __restrict__ xd, const uint8_t* __restrict__ xs,
                    const float* __restrict__ xt, const uint8_t* __restrict__ wd,
                    const uint8_t* __restrict__ ws, const float* __restrict__ wt, int M, int N,
                    int K, int tiles_m, int tiles_n, uint16_t* __restrict__ y) {
  // ---- tile assignment: contiguous range per XCD, grouped along M inside it
  const int nwg = tiles_m * tiles_n;
  const int w = blockIdx.x;
  const int L = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (L / per_group) * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in_g = L % per_group;
  const int tm = first_m + in_g % gsize;
  const int tn = in_g / gsize;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int m0 = tm * kTile + (wave >> 1) * 128;
  const int n0 = tn * kTile + (wave & 1) * 128;
  const int64_t kb2 = K / 2, kb16 = K / 16;

  const uint8_t* pa[4];
  const uint8_t* psa[4];
  const uint8_t* pb[4];
  const uint8_t* psb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = min(m0 + 32 * i + lr, M - 1);
    pa[i] = xd + r * kb2 + 16 * h;
    psa[i] = xs + r * kb16 + 2 * h;
    const int64_t c = min(n0 + 32 * i + lr, N - 1);
    pb[i] = wd + c * kb2 + 16 * h;
    psb[i] = ws + c * kb16 + 2 * h;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x16{};

  uint4 ca[4], cb[4];
  uint32_t csa[4], csb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ca[i] = *reinterpret_cast<const uint4*>(pa[i]);
    cb[i] = *reinterpret_cast<const uint4*>(pb[i]);
    csa[i] = *reinterpret_cast<const uint16_t*>(psa[i]);
    csb[i] = *reinterpret_cast<const uint16_t*>(psb[i]);
  }

  const int nk = K / kChunk;
  for (int kc = 0; kc < nk; ++kc) {
    uint4 na[4], nb[4];
    uint32_t nsa[4], nsb[4];
    if (kc + 1 < nk) {
      const int64_t ob = (int64_t)(kc + 1) * (kChunk / 2), os = (int64_t)(kc + 1) * (kChunk / 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        na[i] = *reinterpret_cast<const uint4*>(pa[i] + ob);
        nb[i] = *reinterpret_cast<const uint4*>(pb[i] + ob);
        nsa[i] = *reinterpret_cast<const uint16_t*>(psa[i] + os);
        nsb[i] = *reinterpret_cast<const uint16_t*>(psb[i] + os);
      }
    }
    h2 da[4][2], db[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h2 sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(csa[i], 1.0f, false);
      const h2 sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(csb[i], 1.0f, false);
      da[i][0] = h2{sa.x, sa.x};
      da[i][1] = h2{sa.y, sa.y};
      db[i][0] = h2{sb.x, sb.x};
      db[i][1] = h2{sb.y, sb.y};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h8 A[4], B[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        A[i] = dequant8(word(ca[i], j), da[i][j >> 1]);
        B[i] = dequant8(word(cb[i], j), db[i][j >> 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B[n], acc[i][n], 0, 0, 0);
    }
    if (kc + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ca[i] = na[i];
        cb[i] = nb[i];
        csa[i] = nsa[i];
        csb[i] = nsb[i];
      }
    }
  }

  // ---- epilogue: lane (lr, h) holds, for accumulator element a, row
  // (a & 3) + 8 * (a >> 2) + 4 * h and column lr of each 32x32 tile.
  const float s = xt[0] * wt[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
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

}  // namespace

hipError_t launch_qlinear(const uint8_t* xd, const uint8_t* xs, const float* xt,
                          const uint8_t* wd, const uint8_t* ws, const float* wt, int64_t M,
                          int64_t N, int64_t K, uint16_t* y, hipStream_t s) {
  const int tiles_m = (int)((M + kTile - 1) / kTile);
  const int tiles_n = (int)((N + kTile - 1) / kTile);
  qlinear_kernel<<<tiles_m * tiles_n, 256, 0, s>>>(xd, xs, xt, wd, ws, wt, (int)M, (int)N, (int)K,
                                                   tiles_m, tiles_n, y);
  return hipGetLastError();
}

}  // namespace fos
