// C ABI of the FP8 linear-layer path (declared in include/te_mi355x.h).
//
// Every entry point validates its arguments on the host before any launch, then
// enqueues kernels on the caller's stream.  Errors never throw across the ABI:
// they return a te_status and leave text in a thread-local buffer.  Nothing
// falls back to another precision: an unsupported combination is an error.
// TE_LOG_LEVEL=1 prints each distinct dispatched kernel variant once,
// TE_LOG_LEVEL=2 prints every launch (the pages' [LP-opt] "実モデルにおける結果の
// 解釈" recommends checking which kernels actually run).

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>

#include "../../include/te_mi355x.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

te_status fail(te_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

int log_level() {
  static int lvl = [] {
    const char* e = std::getenv("TE_LOG_LEVEL");
    return e ? std::atoi(e) : 0;
  }();
  return lvl;
}

void log_dispatch(const char* op, const char* variant, const char* detail) {
  const int lvl = log_level();
  if (lvl <= 0) return;
  static std::mutex mu;
  static std::set<std::string> seen;
  std::lock_guard<std::mutex> lock(mu);
  std::string key = std::string(op) + ":" + variant;
  if (lvl == 1 && !seen.insert(key).second) return;
  std::fprintf(stderr, "[te_mi355x] %s -> %s %s\n", op, variant, detail ? detail : "");
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// gfx950 check on every call (the runtime's device attributes; nothing is cached here):
// gfx950 reports compute capability 9.5.
te_status check_device() {
  int dev = 0, major = 0, minor = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TE_ERR_HIP, "hipGetDevice failed");
  if (hipDeviceGetAttribute(&major, hipDeviceAttributeComputeCapabilityMajor, dev) != hipSuccess ||
      hipDeviceGetAttribute(&minor, hipDeviceAttributeComputeCapabilityMinor, dev) != hipSuccess)
    return fail(TE_ERR_HIP, "hipDeviceGetAttribute failed");
  if (major != 9 || minor != 5)
    return fail(TE_ERR_UNSUPPORTED, "device %d has compute capability %d.%d; this library is built for gfx950 (9.5) only",
                dev, major, minor);
  return TE_OK;
}

te_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return TE_OK;
}

bool is_fp8(int d) { return d == TE_E4M3 || d == TE_E5M2; }
bool is_hp(int d) { return d == TE_F32 || d == TE_BF16; }

te_status check_cast_common(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_dtype,
                            int mode, int margin, const float* scale, const float* scale_inv,
                            const float* amax) {
  if (rows < 0 || cols < 0) return fail(TE_ERR_SHAPE, "negative shape (%lld, %lld)", (long long)rows, (long long)cols);
  if (!is_hp(x_dtype)) return fail(TE_ERR_DTYPE, "x_dtype must be TE_F32 or TE_BF16 (got %d)", x_dtype);
  if (!is_fp8(out_dtype)) return fail(TE_ERR_DTYPE, "out_dtype must be TE_E4M3 or TE_E5M2 (got %d)", out_dtype);
  if (mode != TE_SCALE_DELAYED && mode != TE_SCALE_CURRENT && mode != TE_SCALE_CURRENT_FROM_AMAX)
    return fail(TE_ERR_ARG, "bad scaling mode %d", mode);
  if (margin < 0 || margin > 126) return fail(TE_ERR_ARG, "margin must be in [0, 126] (got %d)", margin);
  if (!scale || !scale_inv || !amax) return fail(TE_ERR_NULL, "scale, scale_inv and amax are required");
  if (rows * cols > 0 && !x) return fail(TE_ERR_NULL, "x is NULL");
  if (x && !aligned16(x)) return fail(TE_ERR_ALIGN, "x is not 16-byte aligned");
  if (cols != 0 && rows > (int64_t(1) << 62) / cols) return fail(TE_ERR_SHAPE, "shape too large");
  return TE_OK;
}

// The grid-amax workspace of a call whose mode reduces an amax (every mode but
// TE_SCALE_CURRENT_FROM_AMAX): required, 16-byte aligned.
te_status check_amax_workspace(const void* ws, bool needed) {
  if (!needed) return TE_OK;
  if (!ws) return fail(TE_ERR_NULL, "amax_workspace is NULL (te_amax_workspace_bytes() bytes, zeroed before first use)");
  if (!aligned16(ws)) return fail(TE_ERR_ALIGN, "amax_workspace is not 16-byte aligned");
  return TE_OK;
}

constexpr int64_t kAmaxWsBytes = 8448;  // sizeof(te::AmaxWork)

}  // namespace

extern "C" {

const char* te_get_last_error(void) { return g_err; }

const char* te_version(void) { return "te_mi355x 0.1 (gfx950)"; }

const char* te_gemm_variant(void) { return te::last_gemm_variant(); }

int64_t te_amax_workspace_bytes(void) { return kAmaxWsBytes; }

te_status te_amax_cast(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_dtype, int mode,
                       int margin, float* scale, float* scale_inv, float* amax, uint8_t* out,
                       void* amax_workspace, void* stream) {
  te_status st = check_cast_common(x, x_dtype, rows, cols, out_dtype, mode, margin, scale, scale_inv, amax);
  if (st != TE_OK) return st;
  if (out && !aligned16(out)) return fail(TE_ERR_ALIGN, "out is not 16-byte aligned");
  if ((st = check_amax_workspace(amax_workspace, mode != TE_SCALE_CURRENT_FROM_AMAX)) != TE_OK) return st;
  if ((st = check_device()) != TE_OK) return st;
  log_dispatch("te_amax_cast",
               mode == TE_SCALE_CURRENT ? "amax_pass+cast_pass"
                                        : (mode == TE_SCALE_DELAYED ? "fused_amax_cast" : "cast_pass_from_amax"),
               out_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  return hip_status(te::launch_amax_cast(x, x_dtype, rows * cols, out_dtype == TE_E5M2, mode, margin, scale,
                                         scale_inv, amax, out, amax_workspace, static_cast<hipStream_t>(stream)),
                    "te_amax_cast launch");
}

te_status te_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_dtype, int mode,
                            int margin, float* scale, float* scale_inv, float* amax, uint8_t* out_row,
                            uint8_t* out_col, void* amax_workspace, void* stream) {
  te_status st = check_cast_common(x, x_dtype, rows, cols, out_dtype, mode, margin, scale, scale_inv, amax);
  if (st != TE_OK) return st;
  if (rows * cols > 0 && !out_row && !out_col) return fail(TE_ERR_NULL, "out_row and out_col are both NULL");
  if ((out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)))
    return fail(TE_ERR_ALIGN, "outputs must be 16-byte aligned");
  if ((rows + 127) / 128 > 65535) return fail(TE_ERR_SHAPE, "rows too large for the tile grid");
  if ((st = check_amax_workspace(amax_workspace, mode != TE_SCALE_CURRENT_FROM_AMAX)) != TE_OK) return st;
  if ((st = check_device()) != TE_OK) return st;
  log_dispatch("te_cast_transpose", "tile128x128", out_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  return hip_status(te::launch_cast_transpose(x, x_dtype, rows, cols, out_dtype == TE_E5M2, mode, margin, scale,
                                              scale_inv, amax, out_row, out_col, nullptr, nullptr, amax_workspace,
                                              static_cast<hipStream_t>(stream)),
                    "te_cast_transpose launch");
}

int64_t te_cast_transpose_dbias_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  return kAmaxWsBytes + ((rows + 127) / 128) * cols * static_cast<int64_t>(sizeof(float));
}

int64_t te_mx_scale_panel_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0 || cols % 128 != 0) return -1;
  return ((rows + 255) / 256) * 256 * (cols / 32);
}

te_status te_cast_transpose_dbias(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_dtype,
                                  int mode, int margin, float* scale, float* scale_inv, float* amax,
                                  uint8_t* out_row, uint8_t* out_col, float* dbias, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  te_status st = check_cast_common(x, x_dtype, rows, cols, out_dtype, mode, margin, scale, scale_inv, amax);
  if (st != TE_OK) return st;
  if (rows * cols > 0 && !out_row && !out_col) return fail(TE_ERR_NULL, "out_row and out_col are both NULL");
  if ((out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)))
    return fail(TE_ERR_ALIGN, "outputs must be 16-byte aligned");
  if ((rows + 127) / 128 > 65535) return fail(TE_ERR_SHAPE, "rows too large for the tile grid");
  if (cols > 0 && !dbias) return fail(TE_ERR_NULL, "dbias is NULL");
  const int64_t need = te_cast_transpose_dbias_workspace_bytes(rows, cols);
  if (!workspace || workspace_bytes < need)
    return fail(TE_ERR_ARG, "workspace of %lld bytes needed (got %lld)", (long long)need, (long long)workspace_bytes);
  if (!aligned16(workspace)) return fail(TE_ERR_ALIGN, "workspace must be 16-byte aligned");
  if ((st = check_device()) != TE_OK) return st;
  log_dispatch("te_cast_transpose_dbias", "tile128x128_colsum", out_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return hip_status(te::launch_cast_transpose(x, x_dtype, rows, cols, out_dtype == TE_E5M2, mode, margin, scale,
                                              scale_inv, amax, out_row, out_col, dbias,
                                              reinterpret_cast<float*>(ws + kAmaxWsBytes), ws,
                                              static_cast<hipStream_t>(stream)),
                    "te_cast_transpose_dbias launch");
}

int64_t te_cast_transpose_dbias_noalloc_max_bytes(void) { return te::kStaticScratchBytes; }

te_status te_cast_transpose_dbias_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_dtype,
                                          int mode, int margin, float* scale, float* scale_inv, float* amax,
                                          uint8_t* out_row, uint8_t* out_col, float* dbias, void* stream) {
  te_status st = check_cast_common(x, x_dtype, rows, cols, out_dtype, mode, margin, scale, scale_inv, amax);
  if (st != TE_OK) return st;
  if (rows * cols > 0 && !out_row && !out_col) return fail(TE_ERR_NULL, "out_row and out_col are both NULL");
  if ((out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)))
    return fail(TE_ERR_ALIGN, "outputs must be 16-byte aligned");
  if ((rows + 127) / 128 > 65535) return fail(TE_ERR_SHAPE, "rows too large for the tile grid");
  if (cols > 0 && !dbias) return fail(TE_ERR_NULL, "dbias is NULL");
  const int64_t need = te_cast_transpose_dbias_workspace_bytes(rows, cols);
  if (need > te::kStaticScratchBytes)
    return fail(TE_ERR_SHAPE,
                "te_cast_transpose_dbias_noalloc: [%lld, %lld] needs %lld bytes of scratch, above the static "
                "maximum of %lld (use te_cast_transpose_dbias with a workspace)",
                (long long)rows, (long long)cols, (long long)need, (long long)te::kStaticScratchBytes);
  if ((st = check_device()) != TE_OK) return st;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(te::static_scratch(&ws, s), "te_cast_transpose_dbias_noalloc scratch")) != TE_OK) return st;
  log_dispatch("te_cast_transpose_dbias_noalloc", "tile128x128_colsum_static_scratch",
               out_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  uint8_t* w = static_cast<uint8_t*>(ws);
  return hip_status(te::launch_cast_transpose(x, x_dtype, rows, cols, out_dtype == TE_E5M2, mode, margin, scale,
                                              scale_inv, amax, out_row, out_col, dbias,
                                              reinterpret_cast<float*>(w + kAmaxWsBytes), w, s),
                    "te_cast_transpose_dbias_noalloc launch");
}

te_status te_layernorm_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, const void* gamma,
                           const void* beta, int param_dtype, float eps, int out_dtype, int mode, int margin,
                           float* scale, float* scale_inv, float* amax, uint8_t* out, float* mu, float* rsigma,
                           void* amax_workspace, void* stream) {
  te_status st = check_cast_common(x, x_dtype, rows, cols, out_dtype, mode, margin, scale, scale_inv, amax);
  if (st != TE_OK) return st;
  if (mode == TE_SCALE_CURRENT_FROM_AMAX)
    return fail(TE_ERR_UNSUPPORTED, "te_layernorm_fp8 computes the amax of its own output (delayed or current)");
  if (rows > 0 && cols == 0) return fail(TE_ERR_SHAPE, "LayerNorm needs cols > 0");
  if (cols % 16 != 0) return fail(TE_ERR_SHAPE, "cols must be a multiple of 16 (got %lld)", (long long)cols);
  if (!is_hp(param_dtype)) return fail(TE_ERR_DTYPE, "param_dtype must be TE_F32 or TE_BF16 (got %d)", param_dtype);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(TE_ERR_ARG, "eps must be finite and >= 0");
  if (rows > 0 && (!gamma || !beta || !out)) return fail(TE_ERR_NULL, "gamma, beta and out are required");
  if ((out && !aligned16(out)) || (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
    return fail(TE_ERR_ALIGN, "out, gamma and beta must be 16-byte aligned");
  if ((st = check_amax_workspace(amax_workspace, true)) != TE_OK) return st;
  if ((st = check_device()) != TE_OK) return st;
  log_dispatch("te_layernorm_fp8", mode == TE_SCALE_CURRENT ? "row_per_block_two_pass" : "row_per_block",
               out_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  return hip_status(te::launch_layernorm_fp8(x, x_dtype, rows, cols, gamma, beta, param_dtype, eps,
                                             out_dtype == TE_E5M2, mode == TE_SCALE_CURRENT, margin, scale,
                                             scale_inv, amax, out, mu, rsigma, amax_workspace,
                                             static_cast<hipStream_t>(stream)),
                    "te_layernorm_fp8 launch");
}

te_status te_scale_update(float* amax_history, float* scale, float* scale_inv, int n, int hist_len,
                          int fp8_dtype, int algo, int margin, void* stream) {
  if (n < 0) return fail(TE_ERR_SHAPE, "n must be >= 0");
  if (hist_len < 1 || hist_len > 4096) return fail(TE_ERR_SHAPE, "hist_len must be in [1, 4096]");
  if (!is_fp8(fp8_dtype)) return fail(TE_ERR_DTYPE, "fp8_dtype must be TE_E4M3 or TE_E5M2");
  if (algo != TE_AMAX_MAX && algo != TE_AMAX_MOST_RECENT) return fail(TE_ERR_ARG, "bad amax algo %d", algo);
  if (margin < 0 || margin > 126) return fail(TE_ERR_ARG, "margin must be in [0, 126]");
  if (n > 0 && (!amax_history || !scale || !scale_inv)) return fail(TE_ERR_NULL, "NULL state pointer");
  te_status st = check_device();
  if (st != TE_OK) return st;
  log_dispatch("te_scale_update", algo == TE_AMAX_MAX ? "max" : "most_recent", "");
  return hip_status(te::launch_scale_update(amax_history, scale, scale_inv, n, hist_len, fp8_dtype == TE_E5M2,
                                            algo == TE_AMAX_MOST_RECENT, margin, static_cast<hipStream_t>(stream)),
                    "te_scale_update launch");
}

// The fused epilogue of te_fp8_gemm_amax: amax of the output, FP8 output with a scale.
struct FusedOut {
  float* amax;
  void* amax_ws;
  const float* d_scale;
  float* d_scale_inv;
};

static te_status gemm_impl(const void* a, int a_dtype, const void* a_scale, const void* b, int b_dtype,
                           const void* b_scale, int gran, int64_t m, int64_t n, int64_t k, const void* bias,
                           int bias_dtype, void* d, int d_dtype, int accumulate, void* stream, int splits = 1,
                           void* workspace = nullptr, int64_t workspace_bytes = 0, const FusedOut* fz = nullptr) {
  if (m < 0 || n < 0 || k < 0) return fail(TE_ERR_SHAPE, "negative GEMM shape");
  if (n % 16 != 0 || k % 16 != 0)
    return fail(TE_ERR_SHAPE, "n and k must be multiples of 16 (got n=%lld k=%lld)", (long long)n, (long long)k);
  if (gran != TE_GRAN_TENSOR && gran != TE_GRAN_MX_BLOCK32 && gran != TE_GRAN_MX_BLOCK32_PANEL)
    return fail(TE_ERR_ARG, "bad granularity %d", gran);
  const bool panel = gran == TE_GRAN_MX_BLOCK32_PANEL;
  if (panel) gran = TE_GRAN_MX_BLOCK32;  // same checks as the row-major MX layout, plus k % 128
  if (panel && k % 128 != 0) return fail(TE_ERR_SHAPE, "MX panel scales need k %% 128 == 0 (got k=%lld)", (long long)k);
  const bool bf16 = a_dtype == TE_BF16 && b_dtype == TE_BF16;
  const bool fp4 = a_dtype == TE_E2M1 && b_dtype == TE_E2M1;
  if (!bf16 && !fp4 && !(is_fp8(a_dtype) && is_fp8(b_dtype)))
    return fail(TE_ERR_DTYPE, "a/b dtypes must both be FP8 (E4M3/E5M2), both TE_E2M1 or both TE_BF16 (got %d, %d)",
                a_dtype, b_dtype);
  if (bf16 && gran != TE_GRAN_TENSOR) return fail(TE_ERR_UNSUPPORTED, "BF16 GEMM takes no block scales");
  if (fp4 && gran != TE_GRAN_MX_BLOCK32) return fail(TE_ERR_UNSUPPORTED, "E2M1 operands need MX block scales");
  if (fp4 && k % 256 != 0) return fail(TE_ERR_SHAPE, "MXFP4 GEMM needs k %% 256 == 0 (got k=%lld)", (long long)k);
  if (gran == TE_GRAN_MX_BLOCK32 && k % 32 != 0) return fail(TE_ERR_SHAPE, "MX GEMM needs k %% 32 == 0");
  const bool d_fp8 = fz != nullptr && is_fp8(d_dtype);
  if (d_dtype != TE_BF16 && d_dtype != TE_F32 && !d_fp8)
    return fail(TE_ERR_DTYPE, fz ? "d_dtype must be TE_BF16, TE_F32, TE_E4M3 or TE_E5M2"
                                 : "d_dtype must be TE_BF16 or TE_F32");
  if (fz) {
    if (gran != TE_GRAN_TENSOR) return fail(TE_ERR_UNSUPPORTED, "te_fp8_gemm_amax takes per-tensor FP8 or BF16 operands");
    if (!fz->amax) return fail(TE_ERR_NULL, "amax is required");
    if (d_fp8 && (!fz->d_scale || !fz->d_scale_inv))
      return fail(TE_ERR_NULL, "an FP8 output needs d_scale and d_scale_inv");
    if (!fz->amax_ws) return fail(TE_ERR_NULL, "amax_workspace is NULL (te_amax_workspace_bytes() bytes, zeroed)");
    if (!aligned16(fz->amax_ws)) return fail(TE_ERR_ALIGN, "amax_workspace is not 16-byte aligned");
  }
  if (bias && bias_dtype != TE_BF16 && bias_dtype != TE_F32) return fail(TE_ERR_DTYPE, "bias_dtype must be TE_BF16 or TE_F32");
  if (m >= (int64_t(1) << 31) || n >= (int64_t(1) << 31)) return fail(TE_ERR_SHAPE, "m and n must be < 2^31");
  const int64_t kb = fp4 ? k / 2 : k * (bf16 ? 2 : 1);
  if (kb * 256 >= (int64_t(1) << 31)) return fail(TE_ERR_SHAPE, "k too large (256 rows of k must fit 2 GiB)");
  if (m == 0 || n == 0) {
    if (fz) {  // an empty output still reports amax = 0 (and the FP8 output's scale_inv)
      te_status st0 = check_device();
      if (st0 != TE_OK) return st0;
      te::GemmArgs g0;
      g0.m = m;
      g0.n = n;
      g0.amax = fz->amax;
      g0.d_scale = fz->d_scale;
      g0.d_scale_inv = fz->d_scale_inv;
      g0.d_fp8 = d_fp8 ? (d_dtype == TE_E5M2 ? 2 : 1) : 0;
      return hip_status(te::launch_gemm(g0, static_cast<hipStream_t>(stream)), "te_fp8_gemm_amax launch");
    }
    g_err[0] = '\0';
    return TE_OK;
  }
  if (k == 0) return fail(TE_ERR_SHAPE, "k must be > 0 when m and n are");
  if (!a || !b || !d) return fail(TE_ERR_NULL, "a, b and d are required");
  if (!bf16 && (!a_scale || !b_scale)) return fail(TE_ERR_NULL, "FP8 GEMM needs a_scale and b_scale");
  if (!aligned16(a) || !aligned16(b) || !aligned16(d)) return fail(TE_ERR_ALIGN, "a, b, d must be 16-byte aligned");
  if (gran == TE_GRAN_MX_BLOCK32 && (!aligned16(a_scale) || !aligned16(b_scale)))
    return fail(TE_ERR_ALIGN, "MX scale arrays must be 16-byte aligned");
  te_status st = check_device();
  if (st != TE_OK) return st;
  te::GemmArgs g;
  g.a = a;
  g.b = b;
  g.a_scale = a_scale;
  g.b_scale = b_scale;
  g.bias = bias;
  g.d = d;
  g.m = m;
  g.n = n;
  g.k = k;
  g.a_fmt = a_dtype;
  g.b_fmt = b_dtype;
  g.mx = gran == TE_GRAN_MX_BLOCK32;
  g.mx_panel = panel ? 1 : 0;
  g.bias_bf16 = bias_dtype == TE_BF16;
  g.d_bf16 = d_dtype == TE_BF16;
  g.accumulate = accumulate;
  if (fz) {
    g.amax = fz->amax;
    g.amax_ws = fz->amax_ws;
    g.d_scale = fz->d_scale;
    g.d_scale_inv = fz->d_scale_inv;
    g.d_fp8 = d_fp8 ? (d_dtype == TE_E5M2 ? 2 : 1) : 0;
    g.d_bf16 = d_dtype == TE_BF16;
  }
  if (splits > 1) {
    // split-K: per-tensor FP8 or BF16, at most one split per 128-byte k stage, and an
    // fp32 workspace of splits * m * n floats
    const int64_t stages = (kb + 127) / 128;
    if (gran != TE_GRAN_TENSOR) return fail(TE_ERR_UNSUPPORTED, "split-K takes per-tensor FP8 or BF16 operands");
    if (accumulate) return fail(TE_ERR_UNSUPPORTED, "split-K does not accumulate into D");
    if (splits > stages || splits > 64)
      return fail(TE_ERR_ARG, "splits must be <= the k stages (%lld) and <= 64 (got %d)", (long long)stages, splits);
    if (m * n * splits >= (int64_t(1) << 31)) return fail(TE_ERR_SHAPE, "split-K workspace above 2^31 floats");
    if (!workspace || !aligned16(workspace)) return fail(TE_ERR_ALIGN, "split-K needs a 16-byte aligned workspace");
    if (workspace_bytes < splits * m * n * static_cast<int64_t>(sizeof(float)))
      return fail(TE_ERR_ARG, "split-K workspace too small: %lld bytes for %lld", (long long)workspace_bytes,
                  (long long)(splits * m * n * static_cast<int64_t>(sizeof(float))));
    g.splits = splits;
    g.workspace = workspace;
  }
  hipError_t e = te::launch_gemm(g, static_cast<hipStream_t>(stream));
  if (log_level() > 0) {
    char detail[128];
    std::snprintf(detail, sizeof(detail), "m=%lld n=%lld k=%lld", (long long)m, (long long)n, (long long)k);
    log_dispatch("te_fp8_gemm", te::last_gemm_variant(), detail);
  }
  return hip_status(e, "te_fp8_gemm launch");
}

te_status te_fp8_gemm(const void* a, int a_dtype, const void* a_scale, const void* b, int b_dtype,
                      const void* b_scale, int gran, int64_t m, int64_t n, int64_t k, const void* bias,
                      int bias_dtype, void* d, int d_dtype, void* stream) {
  return gemm_impl(a, a_dtype, a_scale, b, b_dtype, b_scale, gran, m, n, k, bias, bias_dtype, d, d_dtype, 0,
                   stream);
}

te_status te_fp8_gemm_amax(const void* a, int a_dtype, const void* a_scale, const void* b, int b_dtype,
                           const void* b_scale, int64_t m, int64_t n, int64_t k, const void* bias, int bias_dtype,
                           void* d, int d_dtype, const float* d_scale, float* d_scale_inv, float* amax,
                           void* amax_workspace, void* stream) {
  const FusedOut fz{amax, amax_workspace, d_scale, d_scale_inv};
  return gemm_impl(a, a_dtype, a_scale, b, b_dtype, b_scale, TE_GRAN_TENSOR, m, n, k, bias, bias_dtype, d, d_dtype, 0,
                   stream, 1, nullptr, 0, &fz);
}

int64_t te_fp8_gemm_splitk_workspace_bytes(int64_t m, int64_t n, int splits) {
  if (m < 0 || n < 0 || splits < 1) return -1;
  return splits > 1 ? static_cast<int64_t>(splits) * m * n * static_cast<int64_t>(sizeof(float)) : 0;
}

te_status te_fp8_gemm_splitk(const void* a, int a_dtype, const void* a_scale, const void* b, int b_dtype,
                             const void* b_scale, int64_t m, int64_t n, int64_t k, const void* bias, int bias_dtype,
                             void* d, int d_dtype, int splits, void* workspace, int64_t workspace_bytes,
                             void* stream) {
  if (splits < 1) return fail(TE_ERR_ARG, "splits must be >= 1 (got %d)", splits);
  return gemm_impl(a, a_dtype, a_scale, b, b_dtype, b_scale, TE_GRAN_TENSOR, m, n, k, bias, bias_dtype, d, d_dtype,
                   0, stream, splits, workspace, workspace_bytes);
}

te_status te_fp8_gemm_accumulate(const void* a, int a_dtype, const void* a_scale, const void* b, int b_dtype,
                                 const void* b_scale, int gran, int64_t m, int64_t n, int64_t k,
                                 const void* bias, int bias_dtype, float* d, void* stream) {
  return gemm_impl(a, a_dtype, a_scale, b, b_dtype, b_scale, gran, m, n, k, bias, bias_dtype, d, TE_F32, 1,
                   stream);
}

namespace {
te_status check_mxfp8_args(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem_dtype,
                           const uint8_t* out_row, const uint8_t* scale_row, const uint8_t* out_col,
                           const uint8_t* scale_col) {
  if (rows < 0 || cols < 0) return fail(TE_ERR_SHAPE, "negative shape");
  if (!is_hp(x_dtype)) return fail(TE_ERR_DTYPE, "x_dtype must be TE_F32 or TE_BF16");
  if (!is_fp8(elem_dtype)) return fail(TE_ERR_DTYPE, "elem_dtype must be TE_E4M3 or TE_E5M2");
  const bool row = out_row || scale_row, col = out_col || scale_col;
  if (!row && !col && rows * cols > 0) return fail(TE_ERR_NULL, "both output pairs are NULL");
  if ((out_row == nullptr) != (scale_row == nullptr)) return fail(TE_ERR_NULL, "out_row and scale_row go together");
  if ((out_col == nullptr) != (scale_col == nullptr)) return fail(TE_ERR_NULL, "out_col and scale_col go together");
  if (row && cols % 32 != 0) return fail(TE_ERR_SHAPE, "row-wise MXFP8 needs cols %% 32 == 0");
  if (col && rows % 32 != 0) return fail(TE_ERR_SHAPE, "column-wise MXFP8 needs rows %% 32 == 0");
  if (rows * cols > 0 && !x) return fail(TE_ERR_NULL, "x is NULL");
  if ((x && !aligned16(x)) || (out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)))
    return fail(TE_ERR_ALIGN, "x and outputs must be 16-byte aligned");
  if ((rows + 127) / 128 > 65535) return fail(TE_ERR_SHAPE, "rows too large for the tile grid");
  return TE_OK;
}
}  // namespace

te_status te_mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem_dtype,
                            uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                            void* stream) {
  te_status st = check_mxfp8_args(x, x_dtype, rows, cols, elem_dtype, out_row, scale_row, out_col, scale_col);
  if (st != TE_OK) return st;
  if ((st = check_device()) != TE_OK) return st;
  const bool row = out_row != nullptr, col = out_col != nullptr;
  log_dispatch("te_mxfp8_quantize", row && col ? "tile128x64_row+col" : (row ? "tile128x64_row" : "tile128x64_col"),
               elem_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  return hip_status(te::launch_mxfp8_quantize(x, x_dtype, rows, cols, elem_dtype == TE_E5M2, out_row, scale_row,
                                              out_col, scale_col, static_cast<hipStream_t>(stream)),
                    "te_mxfp8_quantize launch");
}

int64_t te_mxfp8_quantize_dbias_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return -1;
  return (rows + 127) / 128 * cols * static_cast<int64_t>(sizeof(float));
}

te_status te_mxfp8_quantize_dbias(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem_dtype,
                                  uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                  float* dbias, void* workspace, int64_t workspace_bytes, void* stream) {
  te_status st = check_mxfp8_args(x, x_dtype, rows, cols, elem_dtype, out_row, scale_row, out_col, scale_col);
  if (st != TE_OK) return st;
  if (cols > 0 && !dbias) return fail(TE_ERR_NULL, "dbias is NULL");
  const int64_t need = te_mxfp8_quantize_dbias_workspace_bytes(rows, cols);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(TE_ERR_ARG, "workspace of %lld bytes needed (got %lld)", (long long)need, (long long)workspace_bytes);
  if (workspace && !aligned16(workspace)) return fail(TE_ERR_ALIGN, "workspace must be 16-byte aligned");
  if ((st = check_device()) != TE_OK) return st;
  log_dispatch("te_mxfp8_quantize_dbias", "tile_colsum", elem_dtype == TE_E5M2 ? "E5M2" : "E4M3");
  return hip_status(te::launch_mxfp8_quantize(x, x_dtype, rows, cols, elem_dtype == TE_E5M2, out_row, scale_row,
                                              out_col, scale_col, static_cast<hipStream_t>(stream), dbias,
                                              static_cast<float*>(workspace)),
                    "te_mxfp8_quantize_dbias launch");
}

te_status te_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* out_row,
                            uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col, void* stream) {
  if (rows < 0 || cols < 0) return fail(TE_ERR_SHAPE, "negative shape");
  if (!is_hp(x_dtype)) return fail(TE_ERR_DTYPE, "x_dtype must be TE_F32 or TE_BF16");
  const bool row = out_row || scale_row, col = out_col || scale_col;
  if (!row && !col) return fail(TE_ERR_NULL, "both output pairs are NULL");
  if ((out_row == nullptr) != (scale_row == nullptr)) return fail(TE_ERR_NULL, "out_row and scale_row go together");
  if ((out_col == nullptr) != (scale_col == nullptr)) return fail(TE_ERR_NULL, "out_col and scale_col go together");
  if (row && cols % 32 != 0) return fail(TE_ERR_SHAPE, "row-wise MXFP4 needs cols %% 32 == 0");
  if (col && rows % 32 != 0) return fail(TE_ERR_SHAPE, "column-wise MXFP4 needs rows %% 32 == 0");
  if (rows * cols > 0 && !x) return fail(TE_ERR_NULL, "x is NULL");
  if ((x && !aligned16(x)) || (out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)))
    return fail(TE_ERR_ALIGN, "x and outputs must be 16-byte aligned");
  if ((rows + 127) / 128 > 65535) return fail(TE_ERR_SHAPE, "rows too large for the tile grid");
  te_status st = check_device();
  if (st != TE_OK) return st;
  log_dispatch("te_mxfp4_quantize", row && col ? "tile128x64_row+col" : (row ? "tile128x64_row" : "tile128x64_col"),
               "E2M1");
  return hip_status(te::launch_mxfp4_quantize(x, x_dtype, rows, cols, out_row, scale_row, out_col, scale_col,
                                              static_cast<hipStream_t>(stream)),
                    "te_mxfp4_quantize launch");
}

// MX quantization with the scales in the GEMM's panel layout (te_fp8_gemm with
// TE_GRAN_MX_BLOCK32_PANEL): bf16 input of whole 128 x 128 tiles only.
static te_status mx_quantize_panel(const char* name, const void* x, int x_dtype, int64_t rows, int64_t cols,
                                   int fp4, int elem_dtype, uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col,
                                   uint8_t* scale_col, void* stream) {
  if (rows < 0 || cols < 0) return fail(TE_ERR_SHAPE, "negative shape");
  if (x_dtype != TE_BF16) return fail(TE_ERR_UNSUPPORTED, "%s: panel scales need TE_BF16 input", name);
  if (!fp4 && !is_fp8(elem_dtype)) return fail(TE_ERR_DTYPE, "elem_dtype must be TE_E4M3 or TE_E5M2");
  const bool row = out_row || scale_row, col = out_col || scale_col;
  if (!row && !col) return fail(TE_ERR_NULL, "both output pairs are NULL");
  if ((out_row == nullptr) != (scale_row == nullptr)) return fail(TE_ERR_NULL, "out_row and scale_row go together");
  if ((out_col == nullptr) != (scale_col == nullptr)) return fail(TE_ERR_NULL, "out_col and scale_col go together");
  if (rows % 128 != 0 || cols % 128 != 0)
    return fail(TE_ERR_UNSUPPORTED, "%s: panel scales need rows and cols multiples of 128 (got %lld x %lld)", name,
                (long long)rows, (long long)cols);
  if (cols * 128 * 2 >= (int64_t(1) << 31) || rows * 128 >= (int64_t(1) << 31))
    return fail(TE_ERR_SHAPE, "%s: a 128-row (column) band must fit 2 GiB", name);
  if (rows * cols > 0 && !x) return fail(TE_ERR_NULL, "x is NULL");
  if ((x && !aligned16(x)) || (out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)) ||
      (scale_row && !aligned16(scale_row)) || (scale_col && !aligned16(scale_col)))
    return fail(TE_ERR_ALIGN, "x, outputs and scale arrays must be 16-byte aligned");
  te_status st = check_device();
  if (st != TE_OK) return st;
  log_dispatch(name, row && col ? "tile128x128_row+col_panel" : (row ? "tile128x128_row_panel" : "tile128x128_col_panel"),
               fp4 ? "E2M1" : (elem_dtype == TE_E5M2 ? "E5M2" : "E4M3"));
  return hip_status(te::launch_mx_quantize_panel(x, rows, cols, fp4, !fp4 && elem_dtype == TE_E5M2, out_row, scale_row,
                                                 out_col, scale_col, static_cast<hipStream_t>(stream)),
                    name);
}

te_status te_mxfp8_quantize_panel(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem_dtype,
                                  uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                  void* stream) {
  return mx_quantize_panel("te_mxfp8_quantize_panel", x, x_dtype, rows, cols, 0, elem_dtype, out_row, scale_row,
                           out_col, scale_col, stream);
}

te_status te_mxfp4_quantize_recipe(const void* x, int x_dtype, int64_t rows, int64_t cols, int flags,
                                   uint32_t rht_sign_mask, uint64_t sr_seed, uint8_t* out_row, uint8_t* scale_row,
                                   uint8_t* out_col, uint8_t* scale_col, void* stream) {
  const char* name = "te_mxfp4_quantize_recipe";
  if (rows < 0 || cols < 0) return fail(TE_ERR_SHAPE, "negative shape");
  if (x_dtype != TE_BF16) return fail(TE_ERR_UNSUPPORTED, "%s: TE_BF16 input only", name);
  if (flags & ~(TE_MX4_RHT | TE_MX4_SR | TE_MX4_2D)) return fail(TE_ERR_ARG, "%s: unknown flags 0x%x", name, flags);
  const bool rht = flags & TE_MX4_RHT, sr = flags & TE_MX4_SR, two_d = flags & TE_MX4_2D;
  const bool row = out_row || scale_row, col = out_col || scale_col;
  if (!row && !col) return fail(TE_ERR_NULL, "both output pairs are NULL");
  if ((out_row == nullptr) != (scale_row == nullptr)) return fail(TE_ERR_NULL, "out_row and scale_row go together");
  if ((out_col == nullptr) != (scale_col == nullptr)) return fail(TE_ERR_NULL, "out_col and scale_col go together");
  if (two_d && (rht || sr)) return fail(TE_ERR_ARG, "%s: TE_MX4_2D (weights) takes neither RHT nor SR", name);
  if (rht && !col) return fail(TE_ERR_ARG, "%s: TE_MX4_RHT transforms the column copy, which is missing", name);
  if (rows % 128 != 0 || cols % 128 != 0)
    return fail(TE_ERR_UNSUPPORTED, "%s: rows and cols must be multiples of 128 (got %lld x %lld)", name,
                (long long)rows, (long long)cols);
  if (cols * 128 * 2 >= (int64_t(1) << 31) || rows * 128 >= (int64_t(1) << 31))
    return fail(TE_ERR_SHAPE, "%s: a 128-row (column) band must fit 2 GiB", name);
  if (rows * cols > 0 && !x) return fail(TE_ERR_NULL, "x is NULL");
  if ((x && !aligned16(x)) || (out_row && !aligned16(out_row)) || (out_col && !aligned16(out_col)) ||
      (scale_row && !aligned16(scale_row)) || (scale_col && !aligned16(scale_col)))
    return fail(TE_ERR_ALIGN, "x, outputs and scale arrays must be 16-byte aligned");
  te_status st = check_device();
  if (st != TE_OK) return st;
  log_dispatch(name, two_d ? "tile128x128_2d_blocks" : (sr ? (rht ? "tile128x128_rht_sr" : "tile128x128_sr")
                                                           : (rht ? "tile128x128_rht" : "tile128x128")),
               "E2M1");
  return hip_status(te::launch_mxfp4_recipe(x, rows, cols, rht, sr, two_d, rht_sign_mask, sr_seed, out_row, scale_row,
                                            out_col, scale_col, static_cast<hipStream_t>(stream)),
                    name);
}

te_status te_mxfp4_quantize_panel(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* out_row,
                                  uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col, void* stream) {
  return mx_quantize_panel("te_mxfp4_quantize_panel", x, x_dtype, rows, cols, 1, TE_E4M3, out_row, scale_row, out_col,
                           scale_col, stream);
}

}  // extern "C"
