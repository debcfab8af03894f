// Building blocks shared by the GEMM kernels (simulated NVFP4 qlinear and native
// MXFP4): buffer resources, global -> LDS copies, the workgroup -> tile map and the
// epilogue of a 256x256 tile held as 4x4 MFMA 32x32 accumulators per wave.
#pragma once

#include "device_common.hpp"

namespace fos {
namespace gemm {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer: 32-bit data format
constexpr int kGroupM = 4;              // tile-rows per group in the tile map

// Global -> LDS copy of 16 (or 4) bytes per lane: lane l's bytes land at
// lds_base + size * l (the LDS base is wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base, uint32_t voff,
                                      int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base, uint32_t voff,
                                     int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, soff, 0, 0);
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8 XCDs,
// each with its own L2: the map gives every XCD a contiguous range of tiles, and
// inside it walks groups of kGroupM tile-rows column by column, so that a group's A
// rows and the current B columns stay in that XCD's L2.
struct TileCoord {
  int tm, tn;
};
__device__ __forceinline__ TileCoord tile_of(int w, int tiles_m, int tiles_n) {
  const int nwg = tiles_m * tiles_n;
  const int L = (nwg % 8 == 0) ? (w % 8) * (nwg / 8) + (w / 8) : w;
  const int per_group = kGroupM * tiles_n;
  const int first_m = (L / per_group) * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first_m);
  const int in_g = L % per_group;
  return TileCoord{first_m + in_g % gsize, in_g / gsize};
}

// Epilogue of a full 256x256 tile (Y below 4 GiB): scale by s, round pairs to bf16
// with the hardware conversion (nearest-even), and store 4 bytes per lane.  In the
// MFMA layout, element a of lane (lr, h) is row (a & 3) + 8 (a >> 2) + 4h, column lr:
// elements a, a + 1 are vertically adjacent, lanes lr, lr + 1 horizontally adjacent.
// Adjacent lanes swap one packed pair (DPP) so that the even lane holds row r,
// columns (c, c + 1) and the odd lane row r + 1, columns (c - 1, c).  The row offsets
// are scalar, so each store is one buffer instruction with no address math.
__device__ __forceinline__ void store_tile_full(uint16_t* y, int M, int N, int m0, int n0,
                                                int lr, int h, float s,
                                                const f32x16 (&acc)[4][4]) {
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
      (void*)y, 0, (int)((uint32_t)M * (uint32_t)N * 2u), kRsrcWord3);
  const int odd = lr & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  const uint32_t row_bytes = (uint32_t)N * 2u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t voff = (uint32_t)(m0 + 32 * i + 4 * h + odd) * row_bytes +
                            (uint32_t)(n0 + 32 * n + lr - odd) * 2u;
#pragma unroll
      for (int a = 0; a < 16; a += 2) {
        const uint32_t p = pack_bf16x2(acc[i][n][a] * s, acc[i][n][a + 1] * s);
        const uint32_t q = __builtin_amdgcn_update_dpp(0u, p, 0xB1, 0xF, 0xF, false);
        const uint32_t out = __builtin_amdgcn_perm(q, p, sel);
        const int drow = (a & 3) + 8 * (a >> 2);
        __builtin_amdgcn_raw_buffer_store_b32(out, ry, voff, (int)(drow * row_bytes), 0);
      }
    }
  }
}

// Epilogue of any tile: full tiles take store_tile_full, edge tiles store element by
// element inside [M) x [N).
__device__ __forceinline__ void store_tile(uint16_t* y, int M, int N, int tm, int tn, int wave,
                                           int lr, int h, float s, const f32x16 (&acc)[4][4]) {
  const int m0 = tm * 256 + (wave >> 1) * 128;
  const int n0 = tn * 256 + (wave & 1) * 128;
  if ((tm + 1) * 256 <= M && (tn + 1) * 256 <= N && (int64_t)M * N * 2 < ((int64_t)1 << 32)) {
    store_tile_full(y, M, N, m0, n0, lr, h, s, acc);
    return;
  }
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

}  // namespace gemm
}  // namespace fos
