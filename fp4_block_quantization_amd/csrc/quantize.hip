// 4/6 NVFP4 quantization kernels (Four Over Six documentation page, section "Four
// Over Six": per block, the scale maps the block maximum to 6 or to 4, whichever
// gives the lower error; options: 2D block scaling, transposed inputs, random
// Hadamard transform, stochastic rounding).
//
// Three kernels, all one-pass over the bf16 input with every 16-value block held in
// one lane's registers while both candidates are evaluated:
//   quant_rows_kernel  row-wise 1D output: the tensor is a flat run of 16-value
//                      blocks; lane = one block; two 16-byte loads, one 8-byte store
//                      of nibbles and one scale byte.
//   quant_tile_kernel  column-wise output (optionally row-wise from the same read):
//                      a 128x64 tile goes through LDS (XOR-swizzled 16-byte groups,
//                      so the column reads spread over the banks); each lane then
//                      reads two adjacent 16-row column blocks as 16 dwords.  With
//                      row-wise output a workgroup walks 4 tiles along its rows and
//                      writes the row-wise record through LDS in whole lines.
//   quant_2d_kernel    16x16 tiles: the 16 lanes of a DPP row hold the 16 rows of a
//                      tile (two tile rows per workgroup); tile max and error sums use
//                      DPP row permutes; row-wise output goes out through LDS in whole
//                      lines; column-wise output is the LDS transpose of the same nibbles.
// Every workgroup first finishes the tensor scale (from the scale pass's partial
// maxima, or the caller's t) and builds a table of (d, 1/d) for all E4M3 codes.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fos {

namespace {

constexpr int kThreads = 256;

struct TensorConsts {
  const float2* tab;   // per-code (d, inv), in LDS
  float u6, u4;
};

// The inputs of the tensor scale -- this thread's four of the scale pass's partial
// maxima, or the caller's t -- loaded before the kernel's own input.  Vector loads
// complete in the order they are issued, so the wait for these leaves the input loads
// in flight during the workgroup's set-up; loaded after the input, as before, the
// set-up waited for the input too (2D kernel 28.5 -> 25.2 us, row + column tile
// kernel 29.4 -> 28.5 us at their bench shapes).
struct TensorPre {
  uint32_t p[4];
  float t;
};
constexpr int kRawBufferWord3 = 0x00020000;   // gfx9 raw buffer, 32-bit data format
__device__ __forceinline__ TensorPre tensor_prefetch(const QuantArgs& a) {
  TensorPre pre;
  // The partial maxima through a buffer resource, with no branch around the loads (a
  // branch made the compiler wait for them at its join, before the input loads): the
  // buffer holds no bytes when there are no partials, and dwords past its end read 0,
  // the neutral value of the maximum.
  const int bytes = a.partials ? 4 * a.npartials : 0;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.partials, 0, bytes, kRawBufferWord3);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    pre.p[k] = __builtin_amdgcn_raw_buffer_load_b32(r, 16u * threadIdx.x + 4 * k, 0, 0);
  pre.t = a.partials ? 0.0f : a.tscale[0];
  return pre;
}

// t from the caller's device scalar, or (fused finish of the tensor-scale pass)
// from the pass's partial maxima, reduced by every workgroup; workgroup 0 stores t.
// Then the workgroup's scale table.  Every thread of the workgroup must call this
// (it synchronizes the workgroup).
__device__ __forceinline__ TensorConsts tensor_consts(const QuantArgs& a, float2* tab,
                                                      const TensorPre& pre) {
  float t;
  if (a.partials) {
    const uint32_t m = max(max(pre.p[0], pre.p[1]), max(pre.p[2], pre.p[3]));
    t = __uint_as_float(block_max_u32(m)) / kScaleDenom;
    if (blockIdx.x == 0 && threadIdx.x == 0) a.tscale_out[0] = t;
  } else {
    t = pre.t;
  }
  build_scale_table(tab, t);
  TensorConsts c;
  c.tab = tab;
  const float2 u = tab[128];
  c.u6 = u.x;
  c.u4 = u.y;
  return c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD
// i % 8), each with its own L2.  This renumbering gives every XCD a contiguous range of
// workgroup numbers, so that neighbouring workgroups, which write the pieces of the
// same output lines, run on one XCD and its L2 merges the pieces before they go out.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t i, uint32_t G) {
  const uint32_t x = i % 8, k = i / 8, q = G / 8, r = G % 8;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

__device__ __forceinline__ void store_block(uint8_t* data, uint8_t* scales, int64_t data_off,
                                            int64_t scale_off, const Cand& c) {
  *reinterpret_cast<uint2*>(data + data_off) = make_uint2(c.lo, c.hi);
  scales[scale_off] = (uint8_t)c.s;
}

// (Row-wise kernels, whose workgroups write whole runs of consecutive blocks, use
// store_block_stream instead.)

// ------------------------------------------------------------------ row-wise, 1D
// One block per lane: a workgroup covers 256 consecutive blocks, each lane issues its
// block's two 16-byte loads before the workgroup's set-up and quantizes it from
// registers.  With one block per lane the Hadamard + stochastic-rounding variant needs
// 61 VGPRs (8 waves per SIMD) instead of the 92 (5 waves) of two blocks per lane; that
// variant is bound by VALU issue and the extra waves hide its dependent chains.
constexpr int kRowsPerWG = kThreads;

template <bool k46, int kSR, bool kRHT>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(QuantArgs a, int64_t nblk) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  // Addresses: the workgroup's first block (scalar) plus a 32-bit lane offset.
  const int64_t b0 = (int64_t)blockIdx.x * kRowsPerWG;
  const int lane = (int)threadIdx.x;
  const int last = (int)min(nblk - 1 - b0, (int64_t)(kRowsPerWG - 1));   // >= 0
  const int64_t b = b0 + lane;
  const TensorPre pre = tensor_prefetch(a);
  // input read once: non-temporal loads.  Lanes past the last block (nblk >= 1: empty
  // tensors launch nothing) load the last block again and store nothing.
  const v4u* xv = reinterpret_cast<const v4u*>(a.x) + 2 * b0;
  const int bl = min(lane, last);
  const v4u l0 = __builtin_nontemporal_load(xv + 2 * bl);
  const v4u l1 = __builtin_nontemporal_load(xv + 2 * bl + 1);
  const uint4 w0 = make_uint4(l0.x, l0.y, l0.z, l0.w);
  const uint4 w1 = make_uint4(l1.x, l1.y, l1.z, l1.w);
  __builtin_amdgcn_sched_barrier(0);   // keep the set-up after the input loads
  __shared__ float2 tab[kScaleTableSize];
  const TensorConsts tc = tensor_consts(a, tab, pre);
  if (lane > last) return;
  float v[16];
  unpack16(w0, w1, v);
  if (kRHT) rht16(v, a.rht_mask);
  uint32_t srr[16];
  if (kSR) sr_draws<kSR>((uint64_t)b, 0u, a.sr_k0, a.sr_k1, srr);
  const Cand c = quantize_block<k46, (kSR != 0)>(v, tc.tab, tc.u6, tc.u4, srr);
  store_block_stream(a.row_data + 8 * b0, a.row_scales + b0, 8 * lane, lane, c);
}

// ------------------------------------------------------------------ column-wise tiles
// A TR x 64 tile (TR = 128 or 256 rows) is read once: each lane loads TR/64 rows x 16
// columns (two 16-byte loads per row), quantizes those row blocks from registers
// (row-wise output) and writes them to LDS; after one barrier each lane reads 16-row
// column pieces back and quantizes TR/64 column blocks.
//
// With row-wise output, a workgroup walks kRowSub tiles along its rows (TR x 256
// columns) and stages the row-wise nibbles and scale bytes in LDS: a row's 16 blocks
// are 128 contiguous bytes of nibbles, written at the end as whole lines with
// non-temporal stores (stored per tile, each wave instruction wrote 16 rows x 32
// bytes, and those row-wise stores took a quarter of the kernel's time).  The next
// tile's loads are issued before the current tile's column phase.  Two or eight tiles
// per workgroup, and workgroups renumbered XCD by XCD, measured no faster.
constexpr int kTileC = 64;
constexpr int kColTileRows = 128;  // rows of a column-wise tile
constexpr int kRowSub = 4;         // tiles along a row per workgroup with row-wise output

template <int TR, bool k46, int kSR, bool kRHT, bool kRows>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(QuantArgs a) {
  constexpr int kSub = kRows ? kRowSub : 1;
  constexpr int kIt = TR / 64;          // rows per lane in the load phase
  constexpr int kNRB = TR / 16;         // 16-row blocks per tile
  constexpr int kLanesPerRB = kThreads / kNRB;
  constexpr int kH = 32 / kLanesPerRB;  // dword columns (column pairs) per lane
  constexpr int kRowBlocks = 4 * kSub;  // row blocks per row of the workgroup
  // TR rows x 32 dwords (64 bf16); logical dword q of row r lives at q ^ sw(r),
  // sw(r) = 4 * ((r >> 4) & 7).
  __shared__ uint32_t lds[TR * 32];
  __shared__ uint2 rnib[kRows ? TR : 1][kRows ? kRowBlocks : 1];
  __shared__ __attribute__((aligned(16))) uint8_t rsc[kRows ? TR : 1][kRows ? kRowBlocks : 1];
  const int64_t R = a.rows, C = a.cols;
  const int64_t span = (int64_t)kTileC * kSub;
  const int64_t wg_c = (C + span - 1) / span;
  const int64_t R0 = (int64_t)(blockIdx.x / wg_c) * TR;
  const int64_t CW = (int64_t)(blockIdx.x % wg_c) * span;   // first column of the workgroup
  const int tid = threadIdx.x;
  const int j = tid & 3;

  // all of the lane's 16-byte loads of a tile are in flight before anything waits on them
  uint4 w[2 * kIt];
  auto load_tile = [&](int64_t C0) {
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
      const int row = (tid >> 2) + 64 * k;
      // rows and columns past the tensor load its last row / 16 columns (no branch);
      // their values are never quantized or stored
      const int64_t gr = min(R0 + row, R - 1), gc = min(C0 + 16 * j, C - 16);
      const uint4* p = reinterpret_cast<const uint4*>(a.x + gr * C + gc);
      w[2 * k] = p[0];
      w[2 * k + 1] = p[1];
    }
  };
  const TensorPre pre = tensor_prefetch(a);
  load_tile(CW);
  __builtin_amdgcn_sched_barrier(0);   // keep the set-up after the input loads
  __shared__ float2 tab[kScaleTableSize];
  const TensorConsts tc = tensor_consts(a, tab, pre);

  // Tiles of this workgroup (uniform), each a row phase (row-wise blocks from registers, the
  // tile into LDS) and, after a barrier, a column phase from LDS; the next tile's loads go out
  // before the barrier.  Written as two phase functions over a run-time tile count, the
  // column-only kernel keeps more of its LDS reads in flight (22.3 -> 21.1 us at 8192x4096).
  const int nsub = (int)min((int64_t)kSub, (C - CW + kTileC - 1) / kTileC);
  auto row_phase = [&](int s) {
    const int64_t C0 = CW + (int64_t)kTileC * s;
#pragma unroll
    for (int k = 0; k < kIt; ++k) {
      const int row = (tid >> 2) + 64 * k;
      const int64_t gr = R0 + row, gc = C0 + 16 * j;
      const uint4 w0 = w[2 * k], w1 = w[2 * k + 1];
      const int sw = 4 * ((row >> 4) & 7);
      *reinterpret_cast<uint4*>(&lds[row * 32 + ((8 * j) ^ sw)]) = w0;
      *reinterpret_cast<uint4*>(&lds[row * 32 + ((8 * j + 4) ^ sw)]) = w1;
      if (kRows && gr < R && gc < C) {
        float v[16];
        unpack16(w0, w1, v);
        uint32_t srr[16];
        const int64_t blk = gr * (C / 16) + gc / 16;
        if (kSR) sr_draws<kSR>((uint64_t)blk, 0u, a.sr_k0, a.sr_k1, srr);
        const Cand c = quantize_block<k46, (kSR != 0)>(v, tc.tab, tc.u6, tc.u4, srr);
        rnib[row][4 * s + j] = make_uint2(c.lo, c.hi);
        rsc[row][4 * s + j] = (uint8_t)c.s;
      }
    }
  };
  auto col_phase = [&](int s) {
    const int64_t C0 = CW + (int64_t)kTileC * s;
    const int rb = tid % kNRB;
    const int sw = 4 * (rb & 7);
    const int64_t nrb = R / 16;
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      const int p = tid / kNRB + kLanesPerRB * h;
      const int64_t gr0 = R0 + 16 * rb, gc = C0 + 2 * p;
      if (gr0 >= R || gc >= C) continue;
      float va[16], vb[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t wd = lds[(16 * rb + i) * 32 + (p ^ sw)];
        va[i] = bf16_lo(wd);
        vb[i] = bf16_hi(wd);
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        float (&v)[16] = t2 ? vb : va;
        const int64_t col = gc + t2;
        if (kRHT) rht16(v, a.rht_mask);
        const int64_t blk = col * nrb + gr0 / 16;
        uint32_t srr[16];
        if (kSR) sr_draws<kSR>((uint64_t)blk, 1u, a.sr_k0, a.sr_k1, srr);
        const Cand c = quantize_block<k46, (kSR != 0)>(v, tc.tab, tc.u6, tc.u4, srr);
        store_block(a.col_data, a.col_scales, 8 * blk, blk, c);
      }
    }
  };
#pragma unroll 1
  for (int s = 0; s < nsub; ++s) {
    row_phase(s);
    if (s + 1 < nsub) load_tile(CW + (int64_t)kTileC * (s + 1));
    __syncthreads();
    col_phase(s);
    __syncthreads();   // the next row phase overwrites the tile; the flush reads other rows
  }

  if (kRows) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const int64_t vb = min(span, C - CW) / 16;      // valid row blocks per row
    constexpr int kChunks = kRowBlocks / 2;        // 16-byte chunks of nibbles per row
#pragma unroll
    for (int it = 0; it < TR * kChunks / kThreads; ++it) {
      const int ch = tid + kThreads * it;
      const int row = ch / kChunks, b0 = 2 * (ch % kChunks);
      const int64_t gr = R0 + row;
      if (gr >= R || b0 >= vb) continue;
      uint8_t* dst = a.row_data + gr * (C / 2) + CW / 2 + 8 * b0;
      const uint2 n0 = rnib[row][b0];
      if (b0 + 1 < vb && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        const uint2 n1 = rnib[row][b0 + 1];
        __builtin_nontemporal_store(v4u{n0.x, n0.y, n1.x, n1.y}, reinterpret_cast<v4u*>(dst));
      } else {
        *reinterpret_cast<uint2*>(dst) = n0;
        if (b0 + 1 < vb) *reinterpret_cast<uint2*>(dst + 8) = rnib[row][b0 + 1];
      }
    }
    if (tid < TR) {
      const int64_t gr = R0 + tid;
      if (gr < R) {
        uint8_t* dst = a.row_scales + gr * (C / 16) + CW / 16;
        if (vb == kRowBlocks && kRowBlocks == 16 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          const uint4 sv = *reinterpret_cast<const uint4*>(&rsc[tid][0]);
          __builtin_nontemporal_store(v4u{sv.x, sv.y, sv.z, sv.w}, reinterpret_cast<v4u*>(dst));
        } else {
          for (int b = 0; b < vb; ++b) dst[b] = rsc[tid][b];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 2D 16x16 tiles
// Reductions over the 16 lanes of a DPP row, every lane receiving the result.  The
// partners are lane ^ 1, lane ^ 2 (quad permutes), then the mirrored lane of the other
// quad (row_half_mirror) and of the other half row (row_mirror); for the sum this is
// the pairwise order ((p0 + p1) + (p2 + p3)) + ... up to commutativity of each add.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
// Maximum of non-negative values, taken on their bit patterns (for non-negative floats
// the unsigned order is the value order): one max with a DPP operand per step, where a
// float max would also quiet a possible NaN in the permuted copy.
__device__ __forceinline__ float row16_max(float f) {
  uint32_t v = __float_as_uint(f);
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  return __uint_as_float(max(v, dpp_u32<0x140>(v)));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f32<0xB1>(v);
  v = v + dpp_f32<0x4E>(v);
  v = v + dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}

// A workgroup covers two vertically adjacent rows of 16 tiles; the 16 lanes of a DPP
// row hold the 16 rows of one tile (one 16-value row block each), for both tile rows.
constexpr int k2dTileRows = 2;

template <bool k46, int kSR, bool kRows, bool kCols>
__global__ __launch_bounds__(kThreads) void quant_2d_kernel(QuantArgs a) {
  __shared__ uint2 tr[k2dTileRows][16][17];
  // row-wise outputs of the workgroup, staged so that the global stores cover whole
  // lines: [tile row][row][tile] nibbles (a row of 16 tiles is 128 contiguous bytes)
  // and scale bytes (16 contiguous bytes).  Stored directly, each wave instruction
  // wrote 16 rows x 32 bytes of nibbles and 16 rows x 4 bytes of scales; staged, 8
  // threads write one 128-byte line of nibbles with non-temporal stores like the
  // row-wise kernel, and one thread a row's 16 scale bytes.
  __shared__ uint2 rnib[kRows ? k2dTileRows : 1][16][16];
  __shared__ uint8_t rsc[kRows ? k2dTileRows : 1][16][16];
  const int64_t R = a.rows, C = a.cols;
  const uint32_t tiles_c = (uint32_t)(C / 16);
  const uint32_t wg_per_row = (tiles_c + 15) / 16;
  // neighbouring workgroups share the lines of the row-wise scales (16 bytes each of a
  // 128-byte line): XCD-contiguous numbering, so that one L2 merges them
  const uint32_t wg = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t R0 = (int64_t)(wg / wg_per_row) * (16 * k2dTileRows);
  const int tid = threadIdx.x;
  const int row = tid & 15, tl = tid >> 4;
  const uint32_t T = (wg % wg_per_row) * 16 + tl;
  const bool valid = T < tiles_c;

  const TensorPre pre = tensor_prefetch(a);
  uint4 w[2 * k2dTileRows];
#pragma unroll
  for (int q = 0; q < k2dTileRows; ++q) {
    // tiles past the tensor load its last tile row / column (no branch); their values
    // are never stored
    const int64_t rr = min(R0 + 16 * q + row, R - 1);
    const uint32_t Tc = min(T, tiles_c - 1);
    const uint4* p = reinterpret_cast<const uint4*>(a.x + rr * C + 16 * (int64_t)Tc);
    w[2 * q] = p[0];
    w[2 * q + 1] = p[1];
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the set-up after the input loads
  __shared__ float2 tab[kScaleTableSize];
  const TensorConsts tc = tensor_consts(a, tab, pre);

#pragma unroll
  for (int q = 0; q < k2dTileRows; ++q) {
    const int64_t Rq = R0 + 16 * q;
    if (Rq >= R) break;                         // uniform across the workgroup
    float v[16];
    unpack16(w[2 * q], w[2 * q + 1], v);
    uint32_t srr[16];
    const int64_t rblk = (Rq + row) * tiles_c + T;    // row-wise block id of this row
    if (kSR) sr_draws<kSR>((uint64_t)rblk, 0u, a.sr_k0, a.sr_k1, srr);

    const float am = row16_max(amax16(v));
    Cand c6, c4;
    float inv6, inv4;
    cand_scale_bytes(am, tc.u6, tc.u4, c6.s, c4.s);
    cand_lookup(c6.s, tc.tab, c6.d, inv6);
    if (kSR) cand_codes_sr(v, c6.d, inv6, srr, c6); else cand_codes_rne(v, c6.d, inv6, c6);
    c6.err = row16_sum(c6.err);
    Cand c = c6;
    if (k46) {
      cand_lookup(c4.s, tc.tab, c4.d, inv4);
      if (kSR) cand_codes_sr(v, c4.d, inv4, srr, c4); else cand_codes_rne(v, c4.d, inv4, c4);
      c4.err = row16_sum(c4.err);
      if (c4.err < c6.err) c = c4;
    }
    if (kRows) {
      rnib[q][row][tl] = make_uint2(c.lo, c.hi);
      rsc[q][row][tl] = (uint8_t)c.s;
    }
    if (kCols) {
      tr[q][tl][row] = make_uint2(c.lo, c.hi);
      __syncthreads();
      if (valid) {
        const int cc = row;                      // this lane now owns column cc of the tile
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint2 qq = tr[q][tl][i];
          const uint32_t word = (cc < 8) ? qq.x : qq.y;
          const uint32_t nib = (word >> (4 * (cc & 7))) & 0xfu;
          if (i < 8) lo |= nib << (4 * i); else hi |= nib << (4 * (i - 8));
        }
        const int64_t col = 16 * (int64_t)T + cc;
        const int64_t cblk = col * (R / 16) + Rq / 16;
        *reinterpret_cast<uint2*>(a.col_data + 8 * cblk) = make_uint2(lo, hi);
        a.col_scales[cblk] = (uint8_t)c.s;
      }
    }
  }
  if (kRows) {
    __syncthreads();
    // thread t stores tiles 2j, 2j + 1 (16 bytes of nibbles) of row r of tile row q
    const int q = tid >> 7, r = (tid >> 3) & 15, j = tid & 7;
    const int64_t gr = R0 + 16 * q + r;
    const uint32_t T0 = (wg % wg_per_row) * 16;
    const uint32_t t0 = T0 + 2 * j;
    if (gr < R && t0 < tiles_c) {
      uint8_t* dst = a.row_data + gr * (C / 2) + 8 * (int64_t)t0;
      const uint2 n0 = rnib[q][r][2 * j];
      if (t0 + 1 < tiles_c) {
        const uint2 n1 = rnib[q][r][2 * j + 1];
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          typedef uint32_t v4u __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(v4u{n0.x, n0.y, n1.x, n1.y}, reinterpret_cast<v4u*>(dst));
        }
        else {
          *reinterpret_cast<uint2*>(dst) = n0;
          *reinterpret_cast<uint2*>(dst + 8) = n1;
        }
      } else {
        *reinterpret_cast<uint2*>(dst) = n0;
      }
    }
    // threads 0-31 store the 16 scale bytes of row r of tile row q
    if (tid < 16 * k2dTileRows) {
      const int qs = tid >> 4, rs = tid & 15;
      const int64_t grs = R0 + 16 * qs + rs;
      if (grs < R) {
        uint8_t* dst = a.row_scales + grs * (C / 16) + T0;
        if (T0 + 16 <= tiles_c && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          typedef uint32_t v4u __attribute__((ext_vector_type(4)));
          const uint4 sv = *reinterpret_cast<const uint4*>(&rsc[qs][rs][0]);
          // a cached store: the 8 workgroups that share this 128-byte line run on one XCD
          // (xcd_contiguous), whose L2 merges the pieces (non-temporal 16-byte pieces
          // each cost a 32-byte write: 1.11x the kernel's output bytes instead of 1.00x)
          *reinterpret_cast<v4u*>(dst) = v4u{sv.x, sv.y, sv.z, sv.w};
        } else {
          for (uint32_t t = 0; t < 16 && T0 + t < tiles_c; ++t) dst[t] = rsc[qs][rs][t];
        }
      }
    }
  }
}

template <bool k46, int kSR>
hipError_t dispatch_2d(const QuantArgs& a, hipStream_t s) {
  const int64_t grid = quantize_grid(a);
  if (a.rows_out && a.cols_out)
    quant_2d_kernel<k46, kSR, true, true><<<grid, kThreads, 0, s>>>(a);
  else if (a.rows_out)
    quant_2d_kernel<k46, kSR, true, false><<<grid, kThreads, 0, s>>>(a);
  else
    quant_2d_kernel<k46, kSR, false, true><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <bool k46, int kSR, bool kRHT>
hipError_t dispatch_1d(const QuantArgs& a, hipStream_t s) {
  const int64_t grid = quantize_grid(a);
  if (!a.cols_out) {
    quant_rows_kernel<k46, kSR, kRHT><<<grid, kThreads, 0, s>>>(a, a.rows * a.cols / 16);
    return hipGetLastError();
  }
  constexpr int TR = kColTileRows;
  if (a.rows_out)
    quant_tile_kernel<TR, k46, kSR, kRHT, true><<<grid, kThreads, 0, s>>>(a);
  else
    quant_tile_kernel<TR, k46, kSR, kRHT, false><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <bool k46, int kSR>
hipError_t dispatch_rule(const QuantArgs& a, hipStream_t s) {
  if (a.two_d) return dispatch_2d<k46, kSR>(a, s);
  return a.hadamard ? dispatch_1d<k46, kSR, true>(a, s) : dispatch_1d<k46, kSR, false>(a, s);
}

}  // namespace

int64_t quantize_grid(const QuantArgs& a) {
  if (a.rows == 0 || a.cols == 0) return 0;
  if (a.two_d)  // k2dTileRows tile rows x 16 tile columns per workgroup
    return ((a.rows / 16 + k2dTileRows - 1) / k2dTileRows) * ((a.cols / 16 + 15) / 16);
  if (!a.cols_out) return (a.rows * a.cols / 16 + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t span = (int64_t)kTileC * (a.rows_out ? kRowSub : 1);
  return ((a.rows + kColTileRows - 1) / kColTileRows) * ((a.cols + span - 1) / span);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.four_over_six) {
    if (a.sr == 2) return dispatch_rule<true, 2>(a, s);
    return a.sr ? dispatch_rule<true, 1>(a, s) : dispatch_rule<true, 0>(a, s);
  }
  if (a.sr == 2) return dispatch_rule<false, 2>(a, s);
  return a.sr ? dispatch_rule<false, 1>(a, s) : dispatch_rule<false, 0>(a, s);
}

}  // namespace fos
