/*
 * te_mi355x.h -- C ABI of the MI355X (gfx950) per-tensor scaled FP8 linear-layer path.
 *
 * Pages cited (by title; sections are the pages' own headings):
 *   [TE-summary] "NVIDIA Transformer Engine - 大規模Transformer向け高速低精度学習"
 *   [TE-readme]  "transformerengine" (README summary)
 *   [FP8-intro]  "Introduction to FP8 training using Transformer Engine"
 *                (NVIDIA technical blog, Japanese edition)
 *   [LP-opt]     "How to Optimize Transformer-Based Models for Low-Precision Training"
 *                (NVIDIA technical blog, Japanese translation)
 *
 * [TE-readme] says the library carries a framework-agnostic C++ API so that
 * other deep-learning libraries can add FP8; this header is that API reduced to
 * the five operations of the FP8 linear layer.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates
 *     and owns every buffer, including the scaling state and every workspace.
 *     The library allocates no memory, keeps no pointer to the caller's buffers
 *     after a call returns and caches nothing between calls: its only state is
 *     a per-thread error string and the name of the last GEMM variant
 *     (te_gemm_variant), both diagnostics.
 *   - Amax workspace.  Calls that reduce an amax over a whole tensor inside one
 *     launch (te_amax_cast, te_cast_transpose, te_cast_transpose_dbias,
 *     te_layernorm_fp8, te_fp8_gemm_amax) keep the counters of that grid-wide
 *     reduction in a caller-owned device workspace of te_amax_workspace_bytes()
 *     bytes, 16-byte aligned, which must be all zero before its first use
 *     (e.g. cleared once at allocation).  Every launch that completes leaves it
 *     all zero again, so it can be reused without clearing.  Calls that may run
 *     at the same time (on different streams, or a captured graph replayed
 *     beside eager work) must use different workspaces; calls on one stream run
 *     one after another and may share one.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream).  There is no host synchronization inside.  Scale, amax
 *     and history values never leave the device.
 *   - Layout is row-major.  A matrix [R, C] has C contiguous elements per row.
 *   - Pointers must be 16-byte aligned (TE_ERR_ALIGN otherwise).
 *   - Arguments are validated on the host before any launch; a rejected call
 *     launches nothing, returns a te_status and sets te_get_last_error().  A
 *     launch failure returns TE_ERR_HIP.  No exception or abort crosses the ABI.
 *   - An unsupported combination returns TE_ERR_UNSUPPORTED; nothing falls back
 *     silently to another precision ([LP-opt] "実モデルにおける結果の解釈" warns
 *     that silent fallback hides itself as matching performance).
 *   - The first call on a device checks that it is gfx950 (TE_ERR_UNSUPPORTED
 *     otherwise).
 *   - Calls that write the same buffers must not overlap; calls on one stream
 *     are ordered by the stream.
 *
 * FP8 formats: E4M3 (bias 7, no infinities, max 448) and E5M2 (bias 15, max
 * 57344), per the FP8 paper that [TE-summary] "導入とリソース" points to.  The
 * cast rounds to nearest even and saturates (finite overflow and +-Inf map to
 * +-max; NaN maps to a NaN code).
 */
#ifndef TE_MI355X_H
#define TE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TE_OK = 0,
  TE_ERR_NULL = 1,        /* a required pointer is NULL */
  TE_ERR_SHAPE = 2,       /* a size is negative or breaks a divisibility rule */
  TE_ERR_DTYPE = 3,       /* a dtype is not allowed for that argument */
  TE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  TE_ERR_UNSUPPORTED = 5, /* valid request this library does not implement, or not gfx950 */
  TE_ERR_HIP = 6,         /* the HIP runtime reported an error (launch or device query) */
  TE_ERR_ARG = 7          /* an enum or scalar argument is out of range */
} te_status;

/* TE_E2M1: 4-bit MXFP4 elements, two per byte (element 2i in the low nibble). */
typedef enum { TE_F32 = 0, TE_BF16 = 1, TE_E4M3 = 2, TE_E5M2 = 3, TE_E8M0 = 4, TE_E2M1 = 5 } te_dtype;

/* [FP8-intro] "FP8 Training について": one scale per tensor, refreshed every step.
 * DELAYED: the scale comes from the amax history of earlier steps
 * ([FP8-intro] "Transformer Engine の使い方": DelayedScaling); CURRENT: from this
 * tensor's own amax ([LP-opt] "実モデルにおける結果の解釈", FP8 CurrentScaling).
 * CURRENT_FROM_AMAX: current scaling whose amax is already in *amax, produced by
 * the launch that wrote the tensor (te_fp8_gemm_amax), so the cast reads the
 * tensor once instead of twice. */
typedef enum { TE_SCALE_DELAYED = 0, TE_SCALE_CURRENT = 1, TE_SCALE_CURRENT_FROM_AMAX = 2 } te_scaling;

/* [FP8-intro] "Transformer Engine 統合済みライブラリの利用" (NeMo keys):
 * fp8_amax_compute_algo is 'max' or 'most_recent'. */
typedef enum { TE_AMAX_MAX = 0, TE_AMAX_MOST_RECENT = 1 } te_amax_algo;

/* TENSOR: one fp32 scale_inv per operand.  MX_BLOCK32: one E8M0 exponent per 32
 * consecutive elements along K (MXFP8, [TE-summary] "主な機能"). */
typedef enum { TE_GRAN_TENSOR = 0, TE_GRAN_MX_BLOCK32 = 1, TE_GRAN_MX_BLOCK32_PANEL = 2 } te_granularity;

/*
 * te_amax_cast -- amax reduction and scaled saturating cast of one tensor to FP8.
 *
 * Defines: [FP8-intro] "FP8 Training について" (per-tensor scaling factor, cast
 * to FP8 at compute time); [TE-summary] "主な機能" (amax tracking);
 * [LP-opt] "autocast モードの使用と事前量子化の比較" (inputs are quantized before
 * each GEMM in autocast mode).
 *
 *   x          [rows, cols] of x_dtype (TE_F32 or TE_BF16).
 *   out_dtype  TE_E4M3 (forward tensors) or TE_E5M2 (gradients) -- HYBRID.
 *   mode       TE_SCALE_DELAYED: reads *scale (set by te_scale_update).
 *              TE_SCALE_CURRENT: computes amax first, then
 *                *scale = fl32(fp8_max / amax) * 2^-margin (overflow -> FLT_MAX;
 *                amax 0 or non-finite -> 1.0), and casts with it (two passes
 *                over x: the amax must exist before the first element is cast).
 *              TE_SCALE_CURRENT_FROM_AMAX: as TE_SCALE_CURRENT with *amax read
 *                instead of computed (one pass over x).
 *   margin     >= 0; scale multiplier 2^-margin (CURRENT modes only; DELAYED
 *              applies its margin in te_scale_update).
 *   scale      [1] fp32.  DELAYED: read.  CURRENT modes: written.
 *   scale_inv  [1] fp32, written = fl32(1 / scale used).
 *   amax       [1] fp32, written = max_i |x_i| (overwritten, not accumulated;
 *              point it at slot 0 of the tensor's amax history for DELAYED);
 *              read-only for TE_SCALE_CURRENT_FROM_AMAX.
 *              A NaN input makes amax NaN (the max is taken over magnitude
 *              bit patterns, where NaN ranks above +Inf).
 *   out        [rows, cols] uint8 codes, out_i = satRNE(fl32(x_i * scale)).
 *              May be NULL: then only amax (and, for CURRENT, scale/scale_inv)
 *              is produced.
 *   amax_workspace  the amax workspace (see the conventions above); may be NULL
 *              for TE_SCALE_CURRENT_FROM_AMAX, which reduces nothing.
 * Any rows, cols >= 0 (0 elements: amax = 0 and, for CURRENT, scale = 1).
 */
te_status te_amax_cast(const void* x, int x_dtype, int64_t rows, int64_t cols,
                       int out_dtype, int mode, int margin,
                       float* scale, float* scale_inv, float* amax,
                       uint8_t* out, void* amax_workspace, void* stream);

/* Bytes of the amax workspace (8448; see the conventions above).  Host only. */
int64_t te_amax_workspace_bytes(void);

/*
 * te_cast_transpose -- te_amax_cast that also (or only) writes the byte transpose.
 *
 * Not named on the pages; needed because every GEMM here is "TN" (both
 * operands K-contiguous): Dgrad consumes W^T and Wgrad consumes X^T and dY^T
 * ([LP-opt] "autocast モードの使用と事前量子化の比較": Fprop, Dgrad and Wgrad are
 * separate GEMMs).
 *
 * Arguments as te_amax_cast (amax_workspace included), plus
 *   out_row  [rows, cols] uint8 or NULL.
 *   out_col  [cols, rows] uint8 or NULL; out_col[c, r] == out_row[r, c] byte for byte.
 * At least one of out_row / out_col must be non-NULL (unless rows * cols == 0).
 */
te_status te_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols,
                            int out_dtype, int mode, int margin,
                            float* scale, float* scale_inv, float* amax,
                            uint8_t* out_row, uint8_t* out_col, void* amax_workspace, void* stream);

/*
 * te_cast_transpose_dbias -- te_cast_transpose of an output gradient dY that also
 * returns its bias gradient, read in the same pass over dY.
 *
 * Defines: the backward of te.Linear(..., bias=True) ([FP8-intro] "Transformer
 * Engine の使い方"): for y = x W^T + b the bias gradient is the sum of dY over its
 * rows (tokens); reading it from the pass that casts dY saves a second read of dY.
 *
 * Arguments as te_cast_transpose, plus
 *   dbias      [cols] fp32, written: dbias[c] = sum_r x[r, c], summed in fp32 in a
 *              fixed order (within each 128-row tile, then over tiles in row
 *              order), so the result is reproducible run to run.  NULL only if
 *              cols == 0.
 *   workspace  device scratch of at least te_cast_transpose_dbias_workspace_bytes(
 *              rows, cols) bytes, 16-byte aligned, owned by the caller: the first
 *              te_amax_workspace_bytes() bytes are the amax workspace (all zero
 *              before the first use, left zero by every call, see the conventions
 *              above), the rest holds per-tile partial sums (contents on entry
 *              ignored).
 *   workspace_bytes  its size (TE_ERR_ARG if too small).
 * rows == 0 gives dbias = 0.
 */
te_status te_cast_transpose_dbias(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                  int out_dtype, int mode, int margin,
                                  float* scale, float* scale_inv, float* amax,
                                  uint8_t* out_row, uint8_t* out_col, float* dbias,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes te_cast_transpose_dbias needs for [rows, cols]:
 * te_amax_workspace_bytes() + ceil(rows / 128) * cols * 4 (host only, no GPU call);
 * -1 for negative sizes. */
int64_t te_cast_transpose_dbias_workspace_bytes(int64_t rows, int64_t cols);

/*
 * te_cast_transpose_dbias_noalloc -- te_cast_transpose_dbias for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and results as te_cast_transpose_dbias, but
 * no workspace argument: the amax counters and the per-tile partial sums live in a
 * static scratch array of the library (te_cast_transpose_dbias_noalloc_max_bytes(),
 * 16 MiB), one copy per GPU, held until the process ends.  The call allocates nothing.
 *   - Shapes whose te_cast_transpose_dbias_workspace_bytes(rows, cols) exceeds that
 *     maximum are rejected with TE_ERR_SHAPE (e.g. 15872 x 16384 needs 8.1 MB and fits;
 *     cols = 16384 fits up to 32640 rows).
 *   - Every call on a GPU shares that GPU's scratch: calls that may overlap in time on
 *     one GPU (different streams, a replayed graph beside eager calls) race and must be
 *     ordered by the caller.  Each completed call leaves the amax counters at zero; the
 *     first call on a device also enqueues a clear of them on its stream.
 */
te_status te_cast_transpose_dbias_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                          int out_dtype, int mode, int margin,
                                          float* scale, float* scale_inv, float* amax,
                                          uint8_t* out_row, uint8_t* out_col, float* dbias,
                                          void* stream);

/* Bytes of the static scratch of te_cast_transpose_dbias_noalloc (host only). */
int64_t te_cast_transpose_dbias_noalloc_max_bytes(void);

/*
 * te_layernorm_fp8 -- LayerNorm over the last axis, its output written directly as
 * FP8 codes with per-tensor scaling.
 *
 * Defines: te.LayerNorm, the drop-in for nn.LayerNorm(normalized_shape, eps) with
 * weight and bias ([FP8-intro] "Transformer Engine の使い方": module list;
 * "HuggingFace BERT を例にした Transformer Engine の適用": the conversion keeps eps,
 * weight and bias).  Its output is the input of the QKV and MLP-up GEMMs, so the
 * cast those GEMMs need is done in the normalization pass (one read of x instead of
 * two, no high-precision output).  Per row r:
 *   mu = mean_c x[r, c], var = mean_c (x[r, c] - mu)^2 (biased, as nn.LayerNorm),
 *   rsigma = 1 / sqrt(var + eps),
 *   y[r, c] = ((x[r, c] - mu) * rsigma) * gamma[c] + beta[c],
 *   out[r, c] = satRNE(fl32(y[r, c] * scale)),
 * each step an fp32 operation (sums in a fixed order: reproducible run to run).
 *
 *   x          [rows, cols] of x_dtype (TE_F32 or TE_BF16); cols % 16 == 0, cols > 0
 *              when rows > 0.
 *   gamma, beta  [cols] of param_dtype (TE_F32 or TE_BF16), 16-byte aligned.
 *   eps        >= 0.
 *   out_dtype, mode, margin, scale, scale_inv, amax  as te_amax_cast, with amax the
 *              max |y| (the tensor that is cast).  TE_SCALE_CURRENT reads x twice
 *              (statistics and amax, then the cast).
 *   out        [rows, cols] uint8 codes.
 *   mu, rsigma [rows] fp32, written (the backward's saved statistics), or NULL.
 *   amax_workspace  the amax workspace (required).
 * mode TE_SCALE_CURRENT_FROM_AMAX: TE_ERR_UNSUPPORTED (the amax is of y, which only
 * this call produces).
 */
te_status te_layernorm_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols,
                           const void* gamma, const void* beta, int param_dtype, float eps,
                           int out_dtype, int mode, int margin,
                           float* scale, float* scale_inv, float* amax,
                           uint8_t* out, float* mu, float* rsigma, void* amax_workspace,
                           void* stream);

/*
 * te_scale_update -- delayed-scaling update of n tensors of one FP8 format.
 *
 * Defines: [FP8-intro] "Transformer Engine の使い方" (DelayedScaling with
 * amax_history_len=16, amax_compute_algo="max"); [FP8-intro] "Transformer Engine
 * 統合済みライブラリの利用" (margin, update interval 1, 'max' or 'most_recent').
 *
 *   amax_history  [n, hist_len] fp32, slot 0 = newest (filled by te_amax_cast).
 *   scale, scale_inv  [n] fp32, read and written.
 * For each tensor t:  a = max(hist[t, :]) (TE_AMAX_MAX) or hist[t, 0]
 * (TE_AMAX_MOST_RECENT);  if a is finite and > 0: scale = fl32(fp8_max / a)
 * (overflow -> FLT_MAX) * 2^-margin, else scale unchanged;  scale_inv =
 * fl32(1/scale);  then the history rolls: hist[t, i] = hist[t, i-1] for i >= 1,
 * hist[t, 0] = 0.  fp8_dtype (TE_E4M3 / TE_E5M2) selects fp8_max.
 * n >= 0, 1 <= hist_len <= 4096.
 */
te_status te_scale_update(float* amax_history, float* scale, float* scale_inv,
                          int n, int hist_len, int fp8_dtype, int algo, int margin,
                          void* stream);

/*
 * te_fp8_gemm -- D[m, n] = A[m, k] . B[n, k]^T with a dequantizing epilogue.
 *
 * Defines: [FP8-intro] "FP8 Training について" (FP8 tensor-core GEMM, twice the
 * FLOPS of FP16/BF16); [LP-opt] "autocast モードの使用と事前量子化の比較" (Fprop,
 * Dgrad, Wgrad benchmarked separately); [FP8-intro] "Transformer Engine の使い方"
 * (te.Linear with bias).
 *
 *   a, b       A [m, k], B [n, k] row-major (k contiguous in both: "TN").
 *   a_dtype, b_dtype  TE_E4M3 / TE_E5M2 in any combination (HYBRID Dgrad and
 *              Wgrad use E5M2 x E4M3), or both TE_BF16 for the BF16 baseline.
 *   gran = TE_GRAN_TENSOR: a_scale, b_scale are float* [1] scale_inv values
 *              (NULL for BF16):  D = fl32(fl32(acc * a_scale) * b_scale) + bias.
 *   gran = TE_GRAN_MX_BLOCK32: a_scale uint8 E8M0 [m, k/32], b_scale uint8 E8M0
 *              [n, k/32] (row-major); element formats E4M3/E5M2;
 *              D = sum_blocks 2^(ea-127) 2^(eb-127) (block dot) + bias.  k % 32 == 0.
 *              MXFP4: a_dtype = b_dtype = TE_E2M1, a and b packed [m, k/2] and
 *              [n, k/2] bytes, same scale arrays, k % 256 == 0 ([LP-opt]
 *              "実モデルにおける結果の解釈": FP4 GEMMs against MXFP8 on the same
 *              shapes; the matrix core applies E8M0 scales per 32 elements).
 *   gran = TE_GRAN_MX_BLOCK32_PANEL: as TE_GRAN_MX_BLOCK32 with the same scale
 *              values in the panel layout (te_mx_scale_panel_bytes): rows in panels
 *              of 256; in a panel, the dwords (four block scales) of one 128-element
 *              group of k for the 256 rows are contiguous; byte of (row r, block b) =
 *              4 ((r / 256) (k / 128) + b / 4) 256 + 4 (r % 256) + b % 4.  a_scale
 *              and b_scale hold te_mx_scale_panel_bytes(m, k) and (n, k) bytes;
 *              padding rows are read and never used.  k % 128 == 0 (MXFP4:
 *              k % 256 == 0).  Same results as TE_GRAN_MX_BLOCK32, bit for bit; the
 *              GEMM loads a stage's scales as whole cache lines.
 *   acc        fp32 accumulation on the matrix cores.
 *   bias       [n] of bias_dtype (TE_F32 or TE_BF16, widened to fp32) or NULL.
 *   d          [m, n] of d_dtype (TE_BF16, rounded to nearest even, or TE_F32).
 * Shape rules: m >= 0; n % 16 == 0 and k % 16 == 0 ([FP8-intro] "HuggingFace BERT
 * を例にした Transformer Engine の適用": Linear dims must be multiples of 16 for
 * the tensor cores), k > 0 unless m == 0 or n == 0.
 */
te_status te_fp8_gemm(const void* a, int a_dtype, const void* a_scale,
                      const void* b, int b_dtype, const void* b_scale,
                      int gran, int64_t m, int64_t n, int64_t k,
                      const void* bias, int bias_dtype,
                      void* d, int d_dtype, void* stream);

/*
 * te_fp8_gemm_amax -- te_fp8_gemm (per-tensor FP8 or BF16 operands) whose epilogue also
 * reduces the amax of its output, and can write that output directly as FP8.
 *
 * Defines: [LP-opt] "実モデルにおける結果の解釈" (a per-tensor amax needs an extra
 * memory pass; Current scaling pays that pass on top of Delayed) and [FP8-intro] "FP8
 * Training について" (every tensor cast to FP8 has its own scale, the next layer's
 * input included): the GEMM that produces a tensor finds its amax while writing it,
 * so the next cast needs no amax pass (TE_SCALE_CURRENT_FROM_AMAX), or, with delayed
 * scaling, writes it as FP8 at once.
 *
 *   a, b, scales, m, n, k, bias  as te_fp8_gemm with gran = TE_GRAN_TENSOR.
 *   d          [m, n] of d_dtype: TE_BF16 or TE_F32 as te_fp8_gemm, or TE_E4M3 /
 *              TE_E5M2: uint8 codes satRNE(fl32(r * *d_scale)), r the fp32 result
 *              (scaled, bias added), rounded to nearest even and saturating as
 *              te_amax_cast does.
 *   d_scale    [1] fp32, read (FP8 d only, e.g. the tensor's delayed scale); else NULL.
 *   d_scale_inv [1] fp32, written 1 / *d_scale (FP8 d only); else NULL.
 *   amax       [1] fp32, written: max |D| over the stored values (bf16 / fp32), or over
 *              the fp32 results before the cast (FP8), as a separate cast of that
 *              result would record it; a NaN result makes it NaN; 0 for an empty D.
 *   amax_workspace  the amax workspace (see the conventions above).
 * Shape rules and errors as te_fp8_gemm; MX granularities: TE_ERR_UNSUPPORTED.
 */
te_status te_fp8_gemm_amax(const void* a, int a_dtype, const void* a_scale,
                           const void* b, int b_dtype, const void* b_scale,
                           int64_t m, int64_t n, int64_t k,
                           const void* bias, int bias_dtype,
                           void* d, int d_dtype, const float* d_scale, float* d_scale_inv,
                           float* amax, void* amax_workspace, void* stream);

/*
 * te_fp8_gemm_accumulate -- te_fp8_gemm that adds its result into an fp32 D:
 * D[i, j] = fl32(D_old[i, j] + r[i, j]), r the te_fp8_gemm result of the same
 * arguments (scaled, plus bias).
 *
 * Defines: Wgrad computed in FP8 ([FP8-intro] "統合済みライブラリの利用", the
 * fp8_wgrad key) and accumulated into the weight's fp32 gradient across
 * micro-batches, the main-gradient reading of a Wgrad whose output is fp32.
 *
 *   d          [m, n] fp32, read and written (the caller initialises it).
 * Every other argument, shape rule and error as te_fp8_gemm.  Calls on one D
 * must not overlap (each element is read, added to and written by one thread).
 */
te_status te_fp8_gemm_accumulate(const void* a, int a_dtype, const void* a_scale,
                                 const void* b, int b_dtype, const void* b_scale,
                                 int gran, int64_t m, int64_t n, int64_t k,
                                 const void* bias, int bias_dtype,
                                 float* d, void* stream);

/*
 * te_mxfp8_quantize -- MXFP8 block quantization, row-wise and/or column-wise.
 *
 * Defines: [TE-summary] "主な機能" and [TE-readme] (MXFP8 recipe); [LP-opt]
 * "autocast モードの使用と事前量子化の比較" (per-block scale computation and format
 * conversion are part of the autocast cost).  Block rule (OCP MX v1.0 reading):
 * for 32 consecutive elements, e = floor(log2(max|x|)) - emax_elem (8 for E4M3,
 * 15 for E5M2), clamped to [-127, 127]; scale code = e + 127 (127 for an all-zero
 * block); elements = satRNE(x * 2^-e).  Special blocks: an infinite max reads as
 * log2 = +inf, so the code is 254 (the clamp's top), the infinities saturate to
 * +-max and the finite elements go to 0; a block holding a NaN has a NaN max,
 * which is not > 0, so it keeps code 127 and its NaN elements stay NaN codes.
 * (MXFP4 differs on NaN blocks, see te_mxfp4_quantize: E2M1 has no NaN code, so
 * there the NaN travels in the scale, code 255.)
 *
 *   x          [rows, cols] of x_dtype (TE_F32 or TE_BF16).
 *   elem_dtype TE_E4M3 (or TE_E5M2).
 *   out_row    [rows, cols] uint8, blocks along cols; scale_row [rows, cols/32] E8M0.
 *   out_col    [cols, rows] uint8 = MXFP8 of x^T (blocks along rows, an
 *              independent quantization, not a transpose of out_row);
 *              scale_col [cols, rows/32] E8M0.
 * Either pair may be NULL (not both, unless x is empty).  Row pair needs
 * cols % 32 == 0; col pair needs rows % 32 == 0.
 */
te_status te_mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                            int elem_dtype, uint8_t* out_row, uint8_t* scale_row,
                            uint8_t* out_col, uint8_t* scale_col, void* stream);

/*
 * te_mxfp8_quantize_dbias -- te_mxfp8_quantize of dY that also returns its bias
 * gradient, read in the same pass over dY (the MXFP8 recipe's backward of a linear
 * layer with a bias).
 *
 * Defines: the backward of te.Linear(..., bias=True) ([FP8-intro] "Transformer
 * Engine の使い方") under the MXFP8 recipe ([TE-summary] "主な機能"): db[c] =
 * sum over rows r of x[r, c].
 *
 *   dbias      [cols] fp32, written: the sum in fp32 in the order of
 *              te_cast_transpose_dbias over the same input type (within each
 *              128-row tile, rows g, g + G, ... for each g < G, then the G group
 *              sums; then over tiles in row order), so both calls give the same bits
 *              and a run is reproducible.  NULL only if cols == 0.
 *   workspace  te_mxfp8_quantize_dbias_workspace_bytes(rows, cols) bytes of device
 *              memory, 16-byte aligned, owned by the caller: ceil(rows / 128) * cols
 *              fp32 partial sums, overwritten by every call (no initial contents
 *              needed).  Calls that may overlap need one workspace each.
 *   workspace_bytes  its size; TE_ERR_ARG if smaller than needed.
 * Every other argument, shape rule and error as te_mxfp8_quantize; rows == 0 gives
 * dbias = 0.
 */
int64_t te_mxfp8_quantize_dbias_workspace_bytes(int64_t rows, int64_t cols);
te_status te_mxfp8_quantize_dbias(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                  int elem_dtype, uint8_t* out_row, uint8_t* scale_row,
                                  uint8_t* out_col, uint8_t* scale_col, float* dbias,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * te_mxfp4_quantize -- MXFP4 block quantization (E2M1 elements, E8M0 per 32),
 * row-wise and/or column-wise.
 *
 * Defines: [LP-opt] "実モデルにおける結果の解釈" (FP4 block-scaled GEMMs compared
 * with MXFP8) and the MXFP8 block rule of te_mxfp8_quantize with 4-bit elements
 * (OCP MX v1.0 reading): for 32 consecutive elements, e = floor(log2(max|x|)) - 2,
 * clamped to [-127, 127] (127 for an infinite max), scale code e + 127 (127 for an
 * all-zero block); elements = E2M1 of x * 2^-e, rounded to nearest with ties to the
 * even mantissa and saturated at +-6, sign of zero kept.  A block holding a NaN gets
 * scale code 255 and is cast with e = 0, its NaN elements becoming +0.
 *
 *   x          [rows, cols] of x_dtype (TE_F32 or TE_BF16).
 *   out_row    [rows, cols/2] uint8, two codes per byte, blocks along cols;
 *              scale_row [rows, cols/32] E8M0.
 *   out_col    [cols, rows/2] uint8 = MXFP4 of x^T (an independent quantization
 *              with blocks along rows); scale_col [cols, rows/32] E8M0.
 * Either pair may be NULL (not both).  Row pair needs cols % 32 == 0; col pair
 * needs rows % 32 == 0.  x and the code outputs 16-byte aligned.
 */
te_status te_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                            uint8_t* out_row, uint8_t* scale_row,
                            uint8_t* out_col, uint8_t* scale_col, void* stream);

/*
 * te_fp8_gemm_splitk -- te_fp8_gemm (per-tensor FP8 or BF16 operands) with k split into
 * `splits` ranges of whole 128-byte stages, each range's fp32 sums written to a
 * workspace, then added in split order and put through the same epilogue
 * (fl32(fl32(acc * a_scale) * b_scale) + bias, bf16 or fp32).
 *
 * For GEMMs with few output tiles and a long k (the Wgrad and Dgrad GEMMs of small
 * layers, [LP-opt] "autocast モードの使用と事前量子化の比較": Fprop, Dgrad and Wgrad
 * have different aspect ratios): more workgroups than the 256 x 256 tiles give.
 *
 *   Arguments as te_fp8_gemm with gran = TE_GRAN_TENSOR, plus
 *   splits     1 .. min(64, ceil(k bytes / 128)); 1 is te_fp8_gemm.
 *   workspace  device, 16-byte aligned, >= te_fp8_gemm_splitk_workspace_bytes(m, n,
 *              splits) bytes, owned by the caller; contents on entry are ignored.
 * The sum is the same fp32 accumulation in a different order (deterministic: split
 * order fixed).  Other granularities or accumulation: TE_ERR_UNSUPPORTED.
 */
te_status te_fp8_gemm_splitk(const void* a, int a_dtype, const void* a_scale,
                             const void* b, int b_dtype, const void* b_scale,
                             int64_t m, int64_t n, int64_t k, const void* bias, int bias_dtype,
                             void* d, int d_dtype, int splits, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* Workspace bytes of te_fp8_gemm_splitk: splits * m * n * 4 (0 for splits == 1; -1 for
 * negative sizes or splits < 1).  Host only. */
int64_t te_fp8_gemm_splitk_workspace_bytes(int64_t m, int64_t n, int splits);

/*
 * te_mxfp8_quantize_panel / te_mxfp4_quantize_panel -- te_mxfp8_quantize /
 * te_mxfp4_quantize with the E8M0 scales written in the panel layout that
 * te_fp8_gemm reads with TE_GRAN_MX_BLOCK32_PANEL (same codes, same scale values).
 *
 * Defines: the MX block rule of te_mxfp8_quantize (te_mxfp4_quantize for E2M1);
 * the layout only reorders the scales (see te_fp8_gemm).
 *
 *   x          [rows, cols] TE_BF16 (other input types: TE_ERR_UNSUPPORTED).
 *   out_row, out_col  as in te_mxfp8_quantize / te_mxfp4_quantize.
 *   scale_row  te_mx_scale_panel_bytes(rows, cols) bytes: the scales of the row-wise
 *              copy (rows of cols elements).
 *   scale_col  te_mx_scale_panel_bytes(cols, rows) bytes: the scales of the
 *              column-wise copy (x^T: cols rows of rows elements).
 *   Padding rows of the last panel are not written.
 * rows % 128 == 0 and cols % 128 == 0 (TE_ERR_UNSUPPORTED otherwise); all pointers
 * 16-byte aligned.  Either pair may be NULL (not both).
 */
te_status te_mxfp8_quantize_panel(const void* x, int x_dtype, int64_t rows, int64_t cols, int elem_dtype,
                                  uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                  void* stream);
te_status te_mxfp4_quantize_panel(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                  uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                  void* stream);

/*
 * te_mxfp4_quantize_recipe -- MXFP4 quantization with the FP4 recipe's steps around it.
 *
 * Defines: [LP-opt] "実モデルにおける結果の解釈" (diagnosis "GEMM の速度向上 >> トレー
 * ニングの速度向上"): besides the FP4 GEMM, the recipe applies a random Hadamard
 * transform to the Wgrad inputs, stochastic rounding to gradients and 2D block scaling
 * to weights.  The scale rule is te_mxfp4_quantize's; scales go out in the panel layout
 * (as te_mxfp4_quantize_panel).
 *
 *   flags      TE_MX4_RHT: the column-wise copy (the Wgrad operand, blocks along the
 *                rows = tokens) is taken of y = (1/4) H16 diag(s) x, per 16 consecutive
 *                rows: H16 the Sylvester Hadamard matrix, s_j = -1 where bit j of
 *                rht_sign_mask is set (the same mask for both Wgrad operands of a step
 *                keeps dY^T X unchanged); the sum is formed by the fast transform's
 *                butterflies in fp64 and rounded once to fp32.
 *              TE_MX4_SR: E2M1 elements rounded stochastically: between neighbouring
 *                magnitudes lo <= a < hi (a the scaled magnitude, a >= 6 saturates),
 *                up iff r < 65536 (a - lo) / (hi - lo); r of element i (row-major index
 *                in the copy written) is 16-bit lane i % 16 of Philox4x64-10 with counter
 *                (i / 16, copy, 0, 0), copy 0 row-wise / 1 column-wise, key (sr_seed, 0);
 *                lane l = bits 16 (l % 4) .. of output word l / 4.
 *              TE_MX4_2D: one scale per 32 x 32 tile (weights); the column-wise copy
 *                is the transpose of the row-wise one (same codes), so a call that
 *                writes one copy (Fprop: row-wise; Dgrad: column-wise) and a call
 *                that writes the other agree; excludes RHT and SR.
 *   x          [rows, cols] TE_BF16, rows % 128 == 0 and cols % 128 == 0
 *              (TE_ERR_UNSUPPORTED otherwise).
 *   out_row / scale_row, out_col / scale_col  as te_mxfp4_quantize_panel; either pair
 *              may be NULL, not both (TE_MX4_RHT needs the column pair).
 */
enum { TE_MX4_RHT = 1, TE_MX4_SR = 2, TE_MX4_2D = 4 };
te_status te_mxfp4_quantize_recipe(const void* x, int x_dtype, int64_t rows, int64_t cols, int flags,
                                   uint32_t rht_sign_mask, uint64_t sr_seed,
                                   uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                   void* stream);

/* Bytes of E8M0 scales in the panel layout (see te_fp8_gemm) for a matrix of `rows`
 * rows and `cols` elements per row: ceil(rows / 256) * 256 * cols / 32.  Host only;
 * -1 if rows < 0 or cols is not a non-negative multiple of 128. */
int64_t te_mx_scale_panel_bytes(int64_t rows, int64_t cols);

/* Text of the last error on the calling thread ("" if none).  Host pointer owned
 * by the library, valid until the next call on this thread. */
const char* te_get_last_error(void);

/* Library version string (host, static). */
const char* te_version(void);

/* Name of the GEMM kernel variant the last te_fp8_gemm call on the calling thread
 * dispatched (e.g. "gemm4_fp8_e4m3_e4m3_256x256_pingpong"), or "none" before the
 * first call.  Host pointer to a static string.  Lets a caller check which matrix-core
 * path ran: [LP-opt] "実モデルにおける結果の解釈" warns that a silent fallback to
 * another precision shows up only as unchanged performance. */
const char* te_gemm_variant(void);

#ifdef __cplusplus
}
#endif

#endif /* TE_MI355X_H */
