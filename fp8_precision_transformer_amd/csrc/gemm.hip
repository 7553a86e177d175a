// GEMM kernels for gfx950 (CDNA4): D[m, n] = A[m, k] . B[n, k]^T ("TN").
//
// Pages: [FP8-intro] = "Introduction to FP8 training using Transformer Engine"
// (NVIDIA blog, Japanese edition), section "FP8 Training について": the FP8
// tensor-core GEMM has twice the FLOPS of FP16/BF16 and runs with per-tensor
// scales.  [LP-opt] = "How to Optimize Transformer-Based Models for Low-Precision
// Training", section "autocast モードの使用と事前量子化の比較": Fprop, Dgrad and
// Wgrad of each weight are separate GEMMs with different aspect ratios;
// [TE-summary] "主な機能": MXFP8 block scaling.
//
// One kernel template serves three operand kinds:
//   FP8  per-tensor scaled E4M3/E5M2 (any mix), v_mfma_f32_32x32x64_f8f6f4;
//        epilogue d = fl32(fl32(acc * sa_inv) * sb_inv) + bias;
//   MX   E4M3/E5M2 elements with one E8M0 exponent per 32 elements along k,
//        v_mfma_scale_f32_32x32x64_f8f6f4 (the matrix core applies the scales);
//   BF16 comparison GEMM, v_mfma_f32_32x32x16_bf16.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), each wave owns
// a 128 x 128 block = 4 x 4 MFMA tiles of 32 x 32 (256 fp32 accumulators per
// lane).  The k loop advances 128 bytes per stage (128 FP8 or 64 BF16 elements);
// A and B stages (32 KB each) are double-buffered in LDS (128 KB of the 160 KB).
// Global loads for stage t+1 are issued before the MFMAs of stage t, so their
// latency hides behind 32 MFMAs per wave.  LDS rows are 128 bytes = 8 chunks
// of 16 bytes stored at chunk ^ (row & 7), so the 32 rows a wave reads for one
// fragment hit distinct banks.  Workgroups are remapped so each of the 8 XCDs
// (own L2) runs a contiguous, row-grouped range of tiles.

#include "device_common.hpp"
#include "internal.hpp"

namespace te {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BKB = 128, NT = 256;
constexpr int kTileBytes = BM * BKB;  // one operand, one stage
constexpr int kGroupM = 8;            // tile rows per raster group

enum { KIND_FP8 = 0, KIND_MX = 1, KIND_BF16 = 2 };

struct Params {
  const uint8_t* a;
  const uint8_t* b;
  const void* a_scale;
  const void* b_scale;
  const void* bias;
  void* d;
  int M, N;          // rows of A / rows of B (= cols of D)
  int KB;            // bytes per operand row
  int KT;            // k stages
  int kblocks;       // MX: 32-element blocks per row (k / 32)
  int nbm, nbn;      // tile grid
  int bias_bf16, d_bf16;
};

template <int V>
using ic = std::integral_constant<int, V>;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ (row & 7)) << 4); }

template <int KIND, int AF, int BF>
__global__ __launch_bounds__(NT, 1) void k_gemm(Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];

  // ---- tile selection: per-XCD contiguous ranges, grouped raster within ----
  const int nb = p.nbm * p.nbn;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int lin = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int gspan = kGroupM * p.nbn;
  const int group = lin / gspan;
  const int first_m = group * kGroupM;
  const int gsz = (p.nbm - first_m) < kGroupM ? (p.nbm - first_m) : kGroupM;
  const int in_g = lin - group * gspan;
  const int tm = first_m + in_g % gsz;
  const int tn = in_g / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int lr = lane & 31, lk = lane >> 5;

  // ---- global -> register staging: each thread moves 8 chunks of 16 bytes per operand ----
  const int lrow = tid >> 3, lch = tid & 7;
  const uint8_t* a_blk = p.a + static_cast<int64_t>(m0) * p.KB;
  const uint8_t* b_blk = p.b + static_cast<int64_t>(n0) * p.KB;
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int ra = lrow + 32 * i, rb = lrow + 32 * i;
    ra = (m0 + ra < p.M) ? ra : (p.M - 1 - m0);  // clamp: rows past the end re-read the last row
    rb = (n0 + rb < p.N) ? rb : (p.N - 1 - n0);
    a_off[i] = static_cast<uint32_t>(ra) * static_cast<uint32_t>(p.KB) + lch * 16;
    b_off[i] = static_cast<uint32_t>(rb) * static_cast<uint32_t>(p.KB) + lch * 16;
  }
  v4u ra[8], rb[8];
  auto gload = [&](int kt) {
    const uint32_t kb = static_cast<uint32_t>(kt) * BKB;
    const bool in = (kb + lch * 16) < static_cast<uint32_t>(p.KB);  // k tail: zero-fill whole chunks
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = in ? *reinterpret_cast<const v4u*>(a_blk + a_off[i] + kb) : v4u{0, 0, 0, 0};
      rb[i] = in ? *reinterpret_cast<const v4u*>(b_blk + b_off[i] + kb) : v4u{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int stage) {
    uint8_t* sA = smem + stage * 2 * kTileBytes;
    uint8_t* sB = sA + kTileBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lrow + 32 * i;
      *reinterpret_cast<v4u*>(sA + swz(row, lch)) = ra[i];
      *reinterpret_cast<v4u*>(sB + swz(row, lch)) = rb[i];
    }
  };

  // ---- MX scales: one dword = the 4 E8M0 codes of one 128-element k stage ----
  uint32_t sa_cur[4] = {0, 0, 0, 0}, sb_cur[4] = {0, 0, 0, 0};
  uint32_t sa_nxt[4] = {0, 0, 0, 0}, sb_nxt[4] = {0, 0, 0, 0};
  auto scale_load = [&](int kt, uint32_t* sa, uint32_t* sb) {
    if constexpr (KIND == KIND_MX) {
      const uint8_t* as = static_cast<const uint8_t*>(p.a_scale);
      const uint8_t* bs = static_cast<const uint8_t*>(p.b_scale);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = m0 + wm + i * 32 + lr;
        r = r < p.M ? r : p.M - 1;
        int c = n0 + wn + i * 32 + lr;
        c = c < p.N ? c : p.N - 1;
        const int kb0 = kt * 4;
        if ((p.kblocks & 3) == 0) {
          sa[i] = *reinterpret_cast<const uint32_t*>(as + static_cast<int64_t>(r) * p.kblocks + kb0);
          sb[i] = *reinterpret_cast<const uint32_t*>(bs + static_cast<int64_t>(c) * p.kblocks + kb0);
        } else {
          uint32_t va = 0, vb = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int kbq = (kb0 + q < p.kblocks) ? kb0 + q : p.kblocks - 1;
            va |= static_cast<uint32_t>(as[static_cast<int64_t>(r) * p.kblocks + kbq]) << (8 * q);
            vb |= static_cast<uint32_t>(bs[static_cast<int64_t>(c) * p.kblocks + kbq]) << (8 * q);
          }
          sa[i] = va;
          sb[i] = vb;
        }
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{0};

  const int swk = lr & 7;  // (row & 7) of every row this lane reads

  auto compute = [&](int stage) {
    const uint8_t* sA = smem + stage * 2 * kTileBytes;
    const uint8_t* sB = sA + kTileBytes;
    if constexpr (KIND == KIND_BF16) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // four k groups of 16 elements (32 bytes)
        const int ch = g * 2 + lk;
        v8bf af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm + i * 32 + lr;
          af[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(sA + row * BKB + ((ch ^ swk) << 4)));
          const int col = wn + i * 32 + lr;
          bf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(sB + col * BKB + ((ch ^ swk) << 4)));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    } else {
      auto sub = [&](auto S) {  // 64-element k sub-step; lane holds 32 contiguous k
        constexpr int s = decltype(S)::value;
        const int c0 = s * 4 + lk * 2;
        v8i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm + i * 32 + lr;
          const v4u lo = *reinterpret_cast<const v4u*>(sA + row * BKB + ((c0 ^ swk) << 4));
          const v4u hi = *reinterpret_cast<const v4u*>(sA + row * BKB + (((c0 + 1) ^ swk) << 4));
          af[i] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          const int col = wn + i * 32 + lr;
          const v4u lo2 = *reinterpret_cast<const v4u*>(sB + col * BKB + ((c0 ^ swk) << 4));
          const v4u hi2 = *reinterpret_cast<const v4u*>(sB + col * BKB + (((c0 + 1) ^ swk) << 4));
          bf[i] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (KIND == KIND_MX) {
              // byte (2s + lk) of the stage's scale dword is this lane's 32-block
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  af[i], bf[j], acc[i][j], AF, BF, 2 * s, static_cast<int>(sa_cur[i] >> (8 * lk)),
                  2 * s, static_cast<int>(sb_cur[j] >> (8 * lk)));
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j],
                                                                         AF, BF, 0, 0, 0, 0);
            }
          }
      };
      sub(ic<0>{});
      sub(ic<1>{});
    }
  };

  // ---- main loop: one barrier per stage ----
  gload(0);
  scale_load(0, sa_cur, sb_cur);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < p.KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < p.KT;
    if (more) {
      gload(kt + 1);
      scale_load(kt + 1, sa_nxt, sb_nxt);
    }
    compute(cur);
    if (more) sstore(cur ^ 1);
    __syncthreads();
    if constexpr (KIND == KIND_MX) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_cur[i] = sa_nxt[i];
        sb_cur[i] = sb_nxt[i];
      }
    }
  }

  // ---- epilogue ----
  float sa = 1.0f, sb = 1.0f;
  if constexpr (KIND == KIND_FP8) {
    sa = *static_cast<const float*>(p.a_scale);
    sb = *static_cast<const float*>(p.b_scale);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn + j * 32 + lr;
    const bool col_ok = col < p.N;
    float bias_v = 0.0f;
    if (p.bias != nullptr && col_ok) {
      bias_v = p.bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p.bias)[col]) << 16)
                           : static_cast<const float*>(p.bias)[col];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
        float val = acc[i][j][v];
        if constexpr (KIND == KIND_FP8) val = __fmul_rn(__fmul_rn(val, sa), sb);
        if (p.bias != nullptr) val = __fadd_rn(val, bias_v);
        if (col_ok && row < p.M) {
          const int64_t o = static_cast<int64_t>(row) * p.N + col;
          if (p.d_bf16)
            static_cast<uint16_t*>(p.d)[o] = static_cast<uint16_t>(f32_to_bf16_bits(val));
          else
            static_cast<float*>(p.d)[o] = val;
        }
      }
    }
  }
}

thread_local const char* g_last_variant = "none";

template <int KIND, int AF, int BF>
hipError_t run(const Params& p, hipStream_t s, const char* name) {
  g_last_variant = name;
  const int nb = p.nbm * p.nbn;
  hipLaunchKernelGGL((k_gemm<KIND, AF, BF>), dim3(nb), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

const char* last_gemm_variant() { return g_last_variant; }

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.m == 0 || g.n == 0) return hipSuccess;
  Params p;
  p.a = static_cast<const uint8_t*>(g.a);
  p.b = static_cast<const uint8_t*>(g.b);
  p.a_scale = g.a_scale;
  p.b_scale = g.b_scale;
  p.bias = g.bias;
  p.d = g.d;
  p.M = static_cast<int>(g.m);
  p.N = static_cast<int>(g.n);
  const int esz = (g.a_fmt == BF16) ? 2 : 1;
  p.KB = static_cast<int>(g.k * esz);
  p.KT = (p.KB + BKB - 1) / BKB;
  p.kblocks = static_cast<int>(g.k / 32);
  p.nbm = static_cast<int>((g.m + BM - 1) / BM);
  p.nbn = static_cast<int>((g.n + BN - 1) / BN);
  p.bias_bf16 = g.bias_bf16;
  p.d_bf16 = g.d_bf16;
  // f8f6f4 format codes: 0 = E4M3, 1 = E5M2
  const int af = (g.a_fmt == E5M2) ? 1 : 0, bf = (g.b_fmt == E5M2) ? 1 : 0;
  if (g.a_fmt == BF16) return run<KIND_BF16, 0, 0>(p, s, "gemm_bf16_256x256x64");
  if (g.mx) {
    if (af == 0 && bf == 0) return run<KIND_MX, 0, 0>(p, s, "gemm_mx_e4m3_e4m3_256x256x128");
    if (af == 1 && bf == 0) return run<KIND_MX, 1, 0>(p, s, "gemm_mx_e5m2_e4m3_256x256x128");
    if (af == 0 && bf == 1) return run<KIND_MX, 0, 1>(p, s, "gemm_mx_e4m3_e5m2_256x256x128");
    return run<KIND_MX, 1, 1>(p, s, "gemm_mx_e5m2_e5m2_256x256x128");
  }
  if (af == 0 && bf == 0) return run<KIND_FP8, 0, 0>(p, s, "gemm_fp8_e4m3_e4m3_256x256x128");
  if (af == 1 && bf == 0) return run<KIND_FP8, 1, 0>(p, s, "gemm_fp8_e5m2_e4m3_256x256x128");
  if (af == 0 && bf == 1) return run<KIND_FP8, 0, 1>(p, s, "gemm_fp8_e4m3_e5m2_256x256x128");
  return run<KIND_FP8, 1, 1>(p, s, "gemm_fp8_e5m2_e5m2_256x256x128");
}

}  // namespace te
