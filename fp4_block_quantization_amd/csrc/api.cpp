// C ABI of the 4/6 NVFP4 library: argument validation (before any HIP call) and
// kernel dispatch.  See include/fos.h for the contract of every entry point.
#include "../../include/fos.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

// Scratch of fos_quantize_noalloc: the partial maxima of the tensor-scale pass, in a
// device array that the library owns, so that the call allocates nothing and needs
// no workspace argument.  Each GPU holds its own copy (at its own address) until the
// process ends.  On the host `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, once per device (scratch_ptr below).
constexpr int kScratchFloats = fos::kMaxPartials;
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr size_t kWorkspaceBytes = sizeof(float) * fos::kMaxPartials;
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Sign mask of the random Hadamard transform: bit k of word 0 of
// Philox4x32-10(key = seed, counter = 0) (Salmon et al., SC'11).
uint32_t hadamard_mask(uint64_t seed) {
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  return c0 & 0xffffu;
}

fos_status check_config(const fos_quant_config* cfg) {
  if (!cfg) return FOS_E_NULL;
  if (cfg->struct_size != sizeof(fos_quant_config)) return FOS_E_FLAGS;
  if (cfg->rule > FOS_RULE_6ONLY || cfg->rounding > FOS_ROUND_STOCHASTIC_FULL ||
      cfg->block > FOS_BLOCK_2D || cfg->hadamard > 1)
    return FOS_E_FLAGS;
  if (cfg->outputs == 0 || (cfg->outputs & ~(uint32_t)(FOS_OUT_ROWWISE | FOS_OUT_COLWISE)))
    return FOS_E_FLAGS;
  if (cfg->hadamard && (cfg->block == FOS_BLOCK_2D ||
                        cfg->outputs == (FOS_OUT_ROWWISE | FOS_OUT_COLWISE)))
    return FOS_E_FLAGS;
  return FOS_OK;
}

bool wants_cols(const fos_quant_config* cfg) { return (cfg->outputs & FOS_OUT_COLWISE) != 0; }
bool wants_rows(const fos_quant_config* cfg) { return (cfg->outputs & FOS_OUT_ROWWISE) != 0; }

fos_status check_input(const fos_quant_config* cfg, const void* x, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return FOS_E_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return FOS_E_SHAPE;
  if (cols % 16) return FOS_E_SHAPE;
  if ((wants_cols(cfg) || cfg->block == FOS_BLOCK_2D) && rows % 16) return FOS_E_SHAPE;
  if (rows * cols > 0) {
    if (!x) return FOS_E_NULL;
    if (!aligned(x, 16)) return FOS_E_ALIGN;
  }
  return FOS_OK;
}

fos_status check_outputs(const fos_quant_config* cfg, int64_t rows, int64_t cols,
                         const uint8_t* row_data, const uint8_t* row_scales,
                         const uint8_t* col_data, const uint8_t* col_scales) {
  if (rows * cols == 0) return FOS_OK;
  if (wants_rows(cfg)) {
    if (!row_data || !row_scales) return FOS_E_NULL;
    if (!aligned(row_data, 8)) return FOS_E_ALIGN;
  }
  if (wants_cols(cfg)) {
    if (!col_data || !col_scales) return FOS_E_NULL;
    if (!aligned(col_data, 8)) return FOS_E_ALIGN;
  }
  return FOS_OK;
}

fos_status check_scale_and_workspace(const float* tscale, const void* ws, size_t ws_bytes) {
  if (!tscale) return FOS_E_NULL;
  if (!aligned(tscale, 4)) return FOS_E_ALIGN;
  if (!ws || ws_bytes < kWorkspaceBytes || !aligned(ws, 16)) return FOS_E_WORKSPACE;
  return FOS_OK;
}

// Device address of `scratch` on the device that runs `stream` (the current device
// for the null stream).  Looked up with that device current the first time it is
// needed on the device, then kept.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

fos_status scratch_ptr(hipStream_t stream, float** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FOS_E_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return FOS_E_HIP;
    dev = d;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return FOS_E_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      if (dev != cur && hipSetDevice(dev) != hipSuccess) return FOS_E_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur && hipSetDevice(cur) != hipSuccess) return FOS_E_HIP;
      if (e != hipSuccess || !p) return FOS_E_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<float*>(p);
  return FOS_OK;
}

fos::QuantArgs make_args(const fos_quant_config* cfg, const void* x, int64_t rows, int64_t cols,
                         const float* tscale, uint8_t* row_data, uint8_t* row_scales,
                         uint8_t* col_data, uint8_t* col_scales) {
  fos::QuantArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.rows = rows;
  a.cols = cols;
  a.tscale = tscale;
  a.partials = nullptr;
  a.npartials = 0;
  a.tscale_out = nullptr;
  a.row_data = row_data;
  a.row_scales = row_scales;
  a.col_data = col_data;
  a.col_scales = col_scales;
  a.rht_mask = cfg->hadamard ? hadamard_mask(cfg->hadamard_seed) : 0u;
  a.sr_k0 = (uint32_t)cfg->sr_seed;
  a.sr_k1 = (uint32_t)(cfg->sr_seed >> 32);
  a.four_over_six = cfg->rule == FOS_RULE_4OVER6;
  a.sr = cfg->rounding == FOS_ROUND_STOCHASTIC_FULL ? 2 : cfg->rounding == FOS_ROUND_STOCHASTIC;
  a.two_d = cfg->block == FOS_BLOCK_2D;
  a.rows_out = wants_rows(cfg);
  a.cols_out = wants_cols(cfg);
  a.hadamard = cfg->hadamard != 0;
  return a;
}

// Tensor-scale pass: partial maxima into the workspace, their count into *npartials,
// and (with `finalize`) t into *tscale.
fos_status launch_scale(const fos_quant_config* cfg, const void* x, int64_t rows, int64_t cols,
                        float* tscale, void* ws, bool finalize, int* npartials, hipStream_t s) {
  const bool had = cfg->hadamard != 0;
  const uint32_t mask = had ? hadamard_mask(cfg->hadamard_seed) : 0u;
  const hipError_t e = fos::launch_tensor_scale(static_cast<const uint16_t*>(x), rows, cols, had,
                                                had && wants_cols(cfg), mask,
                                                static_cast<float*>(ws), finalize, tscale,
                                                npartials, s);
  return e == hipSuccess ? FOS_OK : FOS_E_HIP;
}

// Y[M][N] = deq(A) deq(B)^T for records A [M][K], B [N][K] blocked along K.
fos_status check_gemm(const uint8_t* a_data, const uint8_t* a_scales, const float* a_t,
                      const uint8_t* b_data, const uint8_t* b_scales, const float* b_t,
                      int64_t M, int64_t N, int64_t K, const void* y) {
  if (M < 1 || N < 1 || K < 64 || K % 64 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return FOS_E_SHAPE;
  if (N > kMaxElems / M || K > kMaxElems / M || K > kMaxElems / N) return FOS_E_SHAPE;
  // each packed operand is addressed through one buffer resource (< 4 GiB)
  if ((M + 256) * (K / 2) >= ((int64_t)1 << 32) || (N + 256) * (K / 2) >= ((int64_t)1 << 32))
    return FOS_E_SHAPE;
  if (fos::qlinear_grid(M, N) > fos::kMaxGrid) return FOS_E_SHAPE;
  if (!a_data || !a_scales || !a_t || !b_data || !b_scales || !b_t || !y) return FOS_E_NULL;
  if (!aligned(a_data, 16) || !aligned(b_data, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(y, 2) || !aligned(a_t, 4) || !aligned(b_t, 4))
    return FOS_E_ALIGN;
  return FOS_OK;
}

fos_status launch_gemm(const uint8_t* a_data, const uint8_t* a_scales, const float* a_t,
                       const uint8_t* b_data, const uint8_t* b_scales, const float* b_t,
                       int64_t M, int64_t N, int64_t K, void* y, void* stream) {
  return fos::launch_qlinear(a_data, a_scales, a_t, b_data, b_scales, b_t, M, N, K,
                             static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

// Workspace of fos_qlinear_fwd_act: X's record, then the scale pass's scratch.
struct ActLayout {
  size_t scales, scratch, total;
};
bool act_layout(int64_t M, int64_t K, ActLayout& L) {
  if (M < 0 || K < 0 || M >= kMaxDim || K >= kMaxDim) return false;
  const uint64_t n = (uint64_t)M * (uint64_t)K;   // < 2^62
  const auto up = [](uint64_t v) { return (v + 255) & ~(uint64_t)255; };
  const uint64_t sc = up(n / 2), scr = up(sc + n / 16), tot = scr + kWorkspaceBytes;
  if (tot > (uint64_t)SIZE_MAX) return false;
  L.scales = (size_t)sc;
  L.scratch = (size_t)scr;
  L.total = (size_t)tot;
  return true;
}

fos_status check_dequantize(const uint8_t* data, const uint8_t* scales, const float* tensor_scale,
                            int64_t rows, int64_t cols, int out_dtype, const void* out) {
  if (out_dtype != FOS_OUT_F32 && out_dtype != FOS_OUT_BF16) return FOS_E_FLAGS;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return FOS_E_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return FOS_E_SHAPE;
  if (cols % 16) return FOS_E_SHAPE;
  if (rows * cols == 0) return FOS_OK;
  if (!data || !scales || !tensor_scale || !out) return FOS_E_NULL;
  if (!aligned(data, 8) || !aligned(out, 16) || !aligned(tensor_scale, 4)) return FOS_E_ALIGN;
  return FOS_OK;
}

// Validation shared by fos_quantize and fos_quantize_noalloc (all but the workspace).
fos_status check_quantize(const fos_quant_config* cfg, const void* x, int64_t rows, int64_t cols,
                          uint8_t* row_data, uint8_t* row_scales, uint8_t* col_data,
                          uint8_t* col_scales, const float* tensor_scale) {
  fos_status st = check_config(cfg);
  if (st != FOS_OK) return st;
  if ((st = check_input(cfg, x, rows, cols)) != FOS_OK) return st;
  if (!tensor_scale) return FOS_E_NULL;
  if (!aligned(tensor_scale, 4)) return FOS_E_ALIGN;
  if ((st = check_outputs(cfg, rows, cols, row_data, row_scales, col_data, col_scales)) != FOS_OK)
    return st;
  const fos::QuantArgs a =
      make_args(cfg, x, rows, cols, nullptr, row_data, row_scales, col_data, col_scales);
  if (fos::quantize_grid(a) > fos::kMaxGrid) return FOS_E_SHAPE;
  return FOS_OK;
}

// The tensor-scale pass into `scratch` (partial maxima), then the quantize kernel, which
// reduces them; arguments already validated.
fos_status quantize_validated(const fos_quant_config* cfg, const void* x, int64_t rows,
                              int64_t cols, uint8_t* row_data, uint8_t* row_scales,
                              uint8_t* col_data, uint8_t* col_scales, float* tensor_scale,
                              float* scratch_mem, hipStream_t s) {
  fos::QuantArgs a =
      make_args(cfg, x, rows, cols, nullptr, row_data, row_scales, col_data, col_scales);
  // an empty tensor launches no quantize kernel: the scale pass writes t (= 0) itself
  const bool empty = rows * cols == 0;
  int npartials = 0;
  fos_status st;
  if ((st = launch_scale(cfg, x, rows, cols, tensor_scale, scratch_mem, empty, &npartials, s)) !=
      FOS_OK)
    return st;
  if (empty) return FOS_OK;
  a.partials = scratch_mem;
  a.npartials = npartials;
  a.tscale_out = tensor_scale;
  return fos::launch_quantize(a, s) == hipSuccess ? FOS_OK : FOS_E_HIP;
}

}  // namespace

extern "C" {

int fos_abi_version(void) { return FOS_ABI_VERSION; }

const char* fos_status_string(fos_status s) {
  switch (s) {
    case FOS_OK: return "FOS_OK";
    case FOS_E_NULL: return "FOS_E_NULL: required pointer is NULL";
    case FOS_E_SHAPE: return "FOS_E_SHAPE: unsupported tensor shape";
    case FOS_E_ALIGN: return "FOS_E_ALIGN: misaligned pointer";
    case FOS_E_FLAGS: return "FOS_E_FLAGS: invalid or unsupported option";
    case FOS_E_WORKSPACE: return "FOS_E_WORKSPACE: workspace missing or too small";
    case FOS_E_HIP: return "FOS_E_HIP: HIP launch failed";
  }
  return "FOS_E_UNKNOWN";
}

size_t fos_quantize_workspace_bytes(void) { return kWorkspaceBytes; }

size_t fos_workspace_bytes(void) { return kWorkspaceBytes; }

fos_status fos_tensor_scale(const fos_quant_config* cfg, const void* x, int64_t rows,
                            int64_t cols, float* tensor_scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  fos_status st = check_config(cfg);
  if (st != FOS_OK) return st;
  if ((st = check_input(cfg, x, rows, cols)) != FOS_OK) return st;
  if ((st = check_scale_and_workspace(tensor_scale, workspace, workspace_bytes)) != FOS_OK)
    return st;
  return launch_scale(cfg, x, rows, cols, tensor_scale, workspace, true, nullptr,
                      static_cast<hipStream_t>(stream));
}

fos_status fos_quantize_scaled(const fos_quant_config* cfg, const void* x, int64_t rows,
                               int64_t cols, const float* tensor_scale, uint8_t* row_data,
                               uint8_t* row_scales, uint8_t* col_data, uint8_t* col_scales,
                               void* stream) {
  fos_status st = check_config(cfg);
  if (st != FOS_OK) return st;
  if ((st = check_input(cfg, x, rows, cols)) != FOS_OK) return st;
  if (!tensor_scale) return FOS_E_NULL;
  if (!aligned(tensor_scale, 4)) return FOS_E_ALIGN;
  if ((st = check_outputs(cfg, rows, cols, row_data, row_scales, col_data, col_scales)) != FOS_OK)
    return st;
  const fos::QuantArgs a =
      make_args(cfg, x, rows, cols, tensor_scale, row_data, row_scales, col_data, col_scales);
  if (fos::quantize_grid(a) > fos::kMaxGrid) return FOS_E_SHAPE;
  return fos::launch_quantize(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FOS_OK
                                                                                 : FOS_E_HIP;
}

fos_status fos_quantize(const fos_quant_config* cfg, const void* x, int64_t rows, int64_t cols,
                        uint8_t* row_data, uint8_t* row_scales, uint8_t* col_data,
                        uint8_t* col_scales, float* tensor_scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  fos_status st = check_config(cfg);
  if (st != FOS_OK) return st;
  if ((st = check_input(cfg, x, rows, cols)) != FOS_OK) return st;
  if ((st = check_scale_and_workspace(tensor_scale, workspace, workspace_bytes)) != FOS_OK)
    return st;
  if ((st = check_quantize(cfg, x, rows, cols, row_data, row_scales, col_data, col_scales,
                           tensor_scale)) != FOS_OK)
    return st;
  return quantize_validated(cfg, x, rows, cols, row_data, row_scales, col_data, col_scales,
                            tensor_scale, static_cast<float*>(workspace),
                            static_cast<hipStream_t>(stream));
}

fos_status fos_quantize_noalloc(const fos_quant_config* cfg, const void* x, int64_t rows,
                                int64_t cols, uint8_t* row_data, uint8_t* row_scales,
                                uint8_t* col_data, uint8_t* col_scales, float* tensor_scale,
                                void* stream) {
  fos_status st = check_quantize(cfg, x, rows, cols, row_data, row_scales, col_data, col_scales,
                                 tensor_scale);
  if (st != FOS_OK) return st;
  // the scale pass writes at most kMaxPartials partial maxima, whatever the shape; a
  // pass that needed more than `scratch` holds is refused before anything runs
  if (fos::tensor_scale_partials(rows, cols, cfg->hadamard != 0,
                                 cfg->hadamard != 0 && wants_cols(cfg)) > kScratchFloats)
    return FOS_E_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* mem = nullptr;
  if ((st = scratch_ptr(s, &mem)) != FOS_OK) return st;
  return quantize_validated(cfg, x, rows, cols, row_data, row_scales, col_data, col_scales,
                            tensor_scale, mem, s);
}

fos_status fos_selftest_e4m3(unsigned long long* mismatches, void* stream) {
  if (!mismatches) return FOS_E_NULL;
  if (!aligned(mismatches, 8)) return FOS_E_ALIGN;
  return fos::launch_selftest_e4m3(mismatches, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_selftest_e2m1(unsigned long long* mismatches, void* stream) {
  if (!mismatches) return FOS_E_NULL;
  if (!aligned(mismatches, 8)) return FOS_E_ALIGN;
  return fos::launch_selftest_e2m1(mismatches, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_selftest_e2m1_sr(unsigned long long* mismatches, void* stream) {
  if (!mismatches) return FOS_E_NULL;
  if (!aligned(mismatches, 8)) return FOS_E_ALIGN;
  return fos::launch_selftest_e2m1_sr(mismatches, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_selftest_e2m1_sr_full(unsigned long long* mismatches, void* stream) {
  if (!mismatches) return FOS_E_NULL;
  if (!aligned(mismatches, 8)) return FOS_E_ALIGN;
  return fos::launch_selftest_e2m1_sr_full(mismatches, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_dequantize(const uint8_t* data, const uint8_t* scales, const float* tensor_scale,
                          int64_t rows, int64_t cols, int out_dtype, void* out, void* stream) {
  const fos_status st = check_dequantize(data, scales, tensor_scale, rows, cols, out_dtype, out);
  if (st != FOS_OK || rows * cols == 0) return st;
  return fos::launch_dequantize(data, scales, tensor_scale, rows, cols, out_dtype == FOS_OUT_BF16,
                                out, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_dequantize_hadamard(const uint8_t* data, const uint8_t* scales,
                                   const float* tensor_scale, int64_t rows, int64_t cols,
                                   uint64_t hadamard_seed, int out_dtype, void* out,
                                   void* stream) {
  const fos_status st = check_dequantize(data, scales, tensor_scale, rows, cols, out_dtype, out);
  if (st != FOS_OK || rows * cols == 0) return st;
  return fos::launch_dequantize_hadamard(data, scales, tensor_scale, rows, cols,
                                         hadamard_mask(hadamard_seed), out_dtype == FOS_OUT_BF16,
                                         out, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_qlinear_fwd(const uint8_t* x_data, const uint8_t* x_scales,
                           const float* x_tensor_scale, const uint8_t* w_data,
                           const uint8_t* w_scales, const float* w_tensor_scale, int64_t M,
                           int64_t N, int64_t K, void* y_bf16, void* stream) {
  const fos_status st = check_gemm(x_data, x_scales, x_tensor_scale, w_data, w_scales,
                                   w_tensor_scale, M, N, K, y_bf16);
  if (st != FOS_OK) return st;
  return launch_gemm(x_data, x_scales, x_tensor_scale, w_data, w_scales, w_tensor_scale, M, N, K,
                     y_bf16, stream);
}

size_t fos_qlinear_act_workspace_bytes(int64_t M, int64_t K) {
  ActLayout L;
  return act_layout(M, K, L) ? L.total : 0;
}

fos_status fos_qlinear_fwd_act(const fos_quant_config* cfg, const void* x_bf16,
                               float* x_tensor_scale, int x_scale_given,
                               const uint8_t* w_data, const uint8_t* w_scales,
                               const float* w_tensor_scale, int64_t M, int64_t N, int64_t K,
                               void* y_bf16, void* workspace, size_t workspace_bytes,
                               void* stream) {
  fos_status st = check_config(cfg);
  if (st != FOS_OK) return st;
  if (cfg->outputs != FOS_OUT_ROWWISE) return FOS_E_FLAGS;
  if ((st = check_input(cfg, x_bf16, M, K)) != FOS_OK) return st;
  ActLayout L;
  if (!act_layout(M, K, L)) return FOS_E_SHAPE;
  if (!x_tensor_scale) return FOS_E_NULL;
  if (!aligned(x_tensor_scale, 4)) return FOS_E_ALIGN;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total) return FOS_E_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xd = ws;
  uint8_t* xs = ws + L.scales;
  void* scratch = ws + L.scratch;
  if ((st = check_gemm(xd, xs, x_tensor_scale, w_data, w_scales, w_tensor_scale, M, N, K,
                       y_bf16)) != FOS_OK)
    return st;
  fos::QuantArgs a = make_args(cfg, x_bf16, M, K, x_scale_given ? x_tensor_scale : nullptr, xd,
                               xs, nullptr, nullptr);
  if (fos::quantize_grid(a) > fos::kMaxGrid) return FOS_E_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!x_scale_given) {
    int npartials = 0;
    if ((st = launch_scale(cfg, x_bf16, M, K, x_tensor_scale, scratch, false, &npartials, s)) !=
        FOS_OK)
      return st;
    a.partials = static_cast<const float*>(scratch);
    a.npartials = npartials;
    a.tscale_out = x_tensor_scale;
  }
  if (fos::launch_quantize(a, s) != hipSuccess) return FOS_E_HIP;
  return launch_gemm(xd, xs, x_tensor_scale, w_data, w_scales, w_tensor_scale, M, N, K, y_bf16,
                     stream);
}

fos_status fos_qlinear_bwd(const uint8_t* dy_data, const uint8_t* dy_scales,
                           const float* dy_tensor_scale, const uint8_t* dyt_data,
                           const uint8_t* dyt_scales, const float* dyt_tensor_scale,
                           const uint8_t* xt_data, const uint8_t* xt_scales,
                           const float* xt_tensor_scale, const uint8_t* wt_data,
                           const uint8_t* wt_scales, const float* wt_tensor_scale, int64_t M,
                           int64_t N, int64_t K, void* dx_bf16, void* dw_bf16, void* stream) {
  if (!dx_bf16 && !dw_bf16) return FOS_E_NULL;
  fos_status st;
  // dX [M][K] = deq(dY) deq(W^T)^T: inner dimension N
  if (dx_bf16 && (st = check_gemm(dy_data, dy_scales, dy_tensor_scale, wt_data, wt_scales,
                                  wt_tensor_scale, M, K, N, dx_bf16)) != FOS_OK)
    return st;
  // dW [N][K] = deq(dY^T) deq(X^T)^T: inner dimension M
  if (dw_bf16 && (st = check_gemm(dyt_data, dyt_scales, dyt_tensor_scale, xt_data, xt_scales,
                                  xt_tensor_scale, N, K, M, dw_bf16)) != FOS_OK)
    return st;
  if (dx_bf16 && (st = launch_gemm(dy_data, dy_scales, dy_tensor_scale, wt_data, wt_scales,
                                   wt_tensor_scale, M, K, N, dx_bf16, stream)) != FOS_OK)
    return st;
  if (dw_bf16)
    return launch_gemm(dyt_data, dyt_scales, dyt_tensor_scale, xt_data, xt_scales,
                       xt_tensor_scale, N, K, M, dw_bf16, stream);
  return FOS_OK;
}

fos_status fos_mx_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* data,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return FOS_E_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return FOS_E_SHAPE;
  if (cols % 32) return FOS_E_SHAPE;
  if (fos::mx_quantize_grid(rows, cols) > fos::kMaxGrid) return FOS_E_SHAPE;
  if (rows * cols == 0) return FOS_OK;
  if (!x || !data || !scales) return FOS_E_NULL;
  if (!aligned(x, 16) || !aligned(data, 16)) return FOS_E_ALIGN;
  return fos::launch_mx_quantize(static_cast<const uint16_t*>(x), rows, cols, data, scales,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_mx_dequantize(const uint8_t* data, const uint8_t* scales, int64_t rows,
                             int64_t cols, int out_dtype, void* out, void* stream) {
  if (out_dtype != FOS_OUT_F32 && out_dtype != FOS_OUT_BF16) return FOS_E_FLAGS;
  if (rows < 0 || cols < 0 || rows >= kMaxDim || cols >= kMaxDim) return FOS_E_SHAPE;
  if (rows > 0 && cols > kMaxElems / rows) return FOS_E_SHAPE;
  if (cols % 32) return FOS_E_SHAPE;
  if (rows * cols == 0) return FOS_OK;
  if (!data || !scales || !out) return FOS_E_NULL;
  if (!aligned(data, 4) || !aligned(out, 16)) return FOS_E_ALIGN;
  return fos::launch_mx_dequantize(data, scales, rows, cols, out_dtype == FOS_OUT_BF16, out,
                                   static_cast<hipStream_t>(stream)) == hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

fos_status fos_mx_qlinear_fwd(const uint8_t* a_data, const uint8_t* a_scales,
                              const uint8_t* b_data, const uint8_t* b_scales, int64_t M,
                              int64_t N, int64_t K, void* y_bf16, void* stream) {
  if (M < 1 || N < 1 || K < 256 || K % 256 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return FOS_E_SHAPE;
  if (N > kMaxElems / M || K > kMaxElems / M || K > kMaxElems / N) return FOS_E_SHAPE;
  if ((M + 256) * (K / 2) >= ((int64_t)1 << 32) || (N + 256) * (K / 2) >= ((int64_t)1 << 32))
    return FOS_E_SHAPE;
  if (fos::mx_gemm_grid(M, N) > fos::kMaxGrid) return FOS_E_SHAPE;
  if (!a_data || !a_scales || !b_data || !b_scales || !y_bf16) return FOS_E_NULL;
  if (!aligned(a_data, 16) || !aligned(b_data, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(y_bf16, 2))
    return FOS_E_ALIGN;
  return fos::launch_mx_gemm(a_data, a_scales, b_data, b_scales, M, N, K,
                             static_cast<uint16_t*>(y_bf16), static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? FOS_OK
             : FOS_E_HIP;
}

}  // extern "C"
