// Internal launcher declarations shared by the C-ABI layer (api.cpp) and the
// kernel translation units.  Host-side only; arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace te {

// dtype codes mirror te_dtype in te_mi355x.h
enum : int { F32 = 0, BF16 = 1, E4M3 = 2, E5M2 = 3, E8M0 = 4, E2M1 = 5 };

// ---- quantizers (quant.hip) ----
// Scaling modes of the quantizers: 0 delayed, 1 current (amax pass + cast pass),
// 2 current with the amax already in *amax (cast pass only).  `ws`: the caller's
// grid-amax workspace (AmaxWork, grid_amax.hpp).
hipError_t launch_amax_cast(const void* x, int x_dtype, int64_t n, int out_e5m2, int mode,
                            int margin, float* scale, float* scale_inv, float* amax,
                            uint8_t* out, void* ws, hipStream_t s);

hipError_t launch_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 int out_e5m2, int mode, int margin, float* scale,
                                 float* scale_inv, float* amax, uint8_t* out_row,
                                 uint8_t* out_col, float* dbias, float* dbias_part, void* ws,
                                 hipStream_t s);

// Size of the static scratch of te_cast_transpose_dbias_noalloc (quant.hip), and its
// device address on the current device (first call on a device: hipGetSymbolAddress and
// a clear of the amax counters on stream s).
constexpr int64_t kStaticScratchBytes = int64_t{16} << 20;
hipError_t static_scratch(void** ptr, hipStream_t s);

hipError_t launch_layernorm_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, const void* gamma,
                                const void* beta, int param_dtype, float eps, int out_e5m2, int current,
                                int margin, float* scale, float* scale_inv, float* amax, uint8_t* out,
                                float* mu, float* rsigma, void* ws, hipStream_t s);

hipError_t launch_scale_update(float* hist, float* scale, float* scale_inv, int n, int hist_len,
                               int e5m2, int most_recent, int margin, hipStream_t s);

// dbias != nullptr: also the bias gradient dbias[c] = sum_r x[r, c] from the same pass,
// through fp32 tile partials in part [ceil(rows / 128), cols]
hipError_t launch_mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 int e5m2, uint8_t* out_row, uint8_t* scale_row,
                                 uint8_t* out_col, uint8_t* scale_col, hipStream_t s,
                                 float* dbias = nullptr, float* part = nullptr);
hipError_t launch_mx_quantize_panel(const void* x, int64_t rows, int64_t cols, int fp4, int e5m2,
                                    uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                    hipStream_t s);
// MXFP4 with the FP4 recipe steps (bf16, whole 128 x 128 tiles, panel-layout scales):
// rht: Hadamard transform of the column copy (sign_mask); sr: stochastic rounding (seed);
// two_d: 32 x 32 block scales (both copies).
hipError_t launch_mxfp4_recipe(const void* x, int64_t rows, int64_t cols, int rht, int sr, int two_d,
                               uint32_t sign_mask, uint64_t seed, uint8_t* out_row, uint8_t* scale_row,
                               uint8_t* out_col, uint8_t* scale_col, hipStream_t s);
hipError_t launch_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* out_row,
                                 uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col, hipStream_t s);

// ---- GEMM (gemm.hip) ----
struct GemmArgs {
  const void* a;
  const void* b;
  const void* a_scale;  // float* scale_inv (tensor) or uint8 E8M0 (MX) or null (bf16)
  const void* b_scale;
  const void* bias;
  void* d;
  int64_t m, n, k;       // elements
  int a_fmt, b_fmt;      // E4M3 / E5M2 / BF16 / E2M1 (MX only, both operands)
  int mx;                // 1: MX block-32 scales
  int mx_panel;          // 1: MX scales in the panel layout (k % 128 == 0)
  int bias_bf16;         // bias dtype: 0 f32, 1 bf16
  int d_bf16;            // output dtype: 0 f32, 1 bf16
  int accumulate;        // 1: fp32 D = fl32(D_old + result)
  int splits = 1;        // split-K: k splits (per-tensor FP8 / BF16 only)
  void* workspace = nullptr;  // split-K: [splits, m, n] fp32
  // fused epilogue (te_fp8_gemm_amax): amax of the output, optional FP8 output
  float* amax = nullptr;
  void* amax_ws = nullptr;
  const float* d_scale = nullptr;
  float* d_scale_inv = nullptr;
  int d_fp8 = 0;              // 0 none, 1 E4M3, 2 E5M2
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);

// Name of the kernel variant the last launch_gemm on this thread dispatched
// (for logging; see TE_LOG_LEVEL in api.cpp).
const char* last_gemm_variant();

}  // namespace te
