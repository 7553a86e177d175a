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
// Operand kinds:
//   FP8  per-tensor scaled E4M3/E5M2 (any mix), v_mfma_f32_{16x16x128,32x32x64}_f8f6f4;
//        epilogue d = fl32(fl32(acc * sa_inv) * sb_inv) + bias;
//   MX   E4M3/E5M2 elements with one E8M0 exponent per 32 elements along k,
//        v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4 (the matrix core applies the scales);
//   MX4  E2M1 elements (two per byte) with one E8M0 exponent per 32, the same
//        scaled instruction with the FP4 operand format (MXFP4);
//   BF16 comparison GEMM, v_mfma_f32_32x32x16_bf16.
//
// Three kernels, all with a 256 x 256 output tile per workgroup and an XCD-aware
// tile order (each of the 8 XCDs, with its own L2, runs a contiguous, row-grouped
// range of tiles):
//   k_gemm1x one wave per SIMD on 16 x 16 x 128 MFMAs (see its header): per-tensor
//            FP8 with k a multiple of 128, and MXFP8 / MXFP4 with panel-layout scales;
//   k_gemm4  8 waves in two ping-pong groups on 32 x 32 MFMAs (see its header): BF16,
//            FP8 with the fused amax epilogue, split-K or ragged k, and MX GEMMs with
//            row-major scales and k a multiple of 128;
//   k_gemm   4 waves of 128 x 128, two-stage LDS pipeline with register
//            staging: MX GEMMs whose k is not a multiple of 128.

#include <map>
#include <mutex>
#include <string>
#include <type_traits>

#include "device_common.hpp"
#include "grid_amax.hpp"
#include "internal.hpp"

namespace te {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Two fp32 values to packed bf16 (x in the low half), round to nearest even, by the
// gfx950 packed convert (v_cvt_pk_bf16_f32); a NaN stays a NaN.
__device__ __forceinline__ unsigned bf16x2_rne(float x, float y) {
  const v2bf v = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
  return __builtin_bit_cast(unsigned, v);
}

constexpr int BM = 256, BN = 256, BKB = 128, NT = 256;
constexpr int kTileBytes = BM * BKB;  // one operand, one stage
constexpr int kGroupM = 8;            // tile rows per raster group

enum { KIND_FP8 = 0, KIND_MX = 1, KIND_BF16 = 2, KIND_MX4 = 3 };

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
  int accumulate;    // fp32 D only: D = fl32(D_old + result)
  int splits;        // k splits (split-K); 1 = the whole k per tile
  int partial;       // 1: write raw fp32 sums of this split to d + split * M * N (no scale, bias)
  float* partial_ws; // split-K: [splits, M, N] fp32 workspace
  // fused epilogue (k_gemm4<..., FUSED>): amax of the output and optional FP8 output
  float* amax;             // [1] written: max |D| (bf16 / fp32: as stored; FP8: before the cast)
  void* amax_ws;           // the caller's grid-amax workspace (AmaxWork)
  const float* d_scale;    // FP8 output: the scale of the cast
  float* d_scale_inv;      // FP8 output: written 1 / d_scale by block 0
  int d_fp8;               // 0: bf16 / fp32 output; 1: E4M3; 2: E5M2
};

template <int V>
using ic = std::integral_constant<int, V>;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BKB + ((chunk ^ (row & 7)) << 4); }

// ============================================================================
// Two-stage kernel (MX GEMMs with k not a multiple of 128): 4 waves (2 x 2), each
// owning a 128 x 128 block = 4 x 4 MFMA tiles of 32 x 32.  The k loop advances
// 128 bytes per stage; A and B stages (32 KB each) are double-buffered in LDS,
// rows of 8 chunks of 16 bytes stored at chunk ^ (row & 7).  Global loads for
// stage t+1 go through registers while the MFMAs of stage t run.  Scale dwords
// of a partial last k stage are assembled per byte.
// ============================================================================
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
      // 64-element k sub-step.  Operand layout of v_mfma_*_32x32x64_f8f6f4: lane l
      // (row l % 32, half h = l / 32) holds k = 16h + [0, 16) in VGPRs 0-3 and
      // k = 32 + 16h + [0, 16) in VGPRs 4-7; the 32-element scale block b is
      // k = [32b, 32b + 32) and takes its E8M0 scale from lane (row, b).
      auto sub = [&](auto S) {
        constexpr int s = decltype(S)::value;
        const int c_lo = s * 4 + lk, c_hi = s * 4 + 2 + lk;
        v8i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm + i * 32 + lr;
          const v4u lo = *reinterpret_cast<const v4u*>(sA + row * BKB + ((c_lo ^ swk) << 4));
          const v4u hi = *reinterpret_cast<const v4u*>(sA + row * BKB + ((c_hi ^ swk) << 4));
          af[i] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          const int col = wn + i * 32 + lr;
          const v4u lo2 = *reinterpret_cast<const v4u*>(sB + col * BKB + ((c_lo ^ swk) << 4));
          const v4u hi2 = *reinterpret_cast<const v4u*>(sB + col * BKB + ((c_hi ^ swk) << 4));
          bf[i] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (KIND == KIND_MX) {
              // lane (row, b) supplies block b of this sub-step: byte 2s + b of the stage dword
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
          else if (p.accumulate)
            static_cast<float*>(p.d)[o] = __fadd_rn(static_cast<float*>(p.d)[o], val);
          else
            static_cast<float*>(p.d)[o] = val;
        }
      }
    }
  }
}

// ============================================================================
// Direct-to-LDS loads: buffer_load_dwordx4 ... lds writes lane j's 16 bytes to
// M0 + 16 j, so any LDS swizzle is applied on the global side (the lane that
// lands at a physical chunk fetches the logical chunk mapped there).  Buffer
// offsets at or past num_records read as zero, which zero-fills rows past m or
// n and chunks past k.
// ============================================================================
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ void raw_buffer_load_lds(v4i rsrc, __attribute__((address_space(3))) uint32_t* lds,
                                    int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

__device__ int buffer_load_u32(v4i rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.i32");

__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = static_cast<int>(a & 0xffffffffu);
  r[1] = static_cast<int>(a >> 32);  // stride 0: raw byte-addressed buffer
  r[2] = static_cast<int>(bytes);    // num_records: offsets at or past it read as 0
  r[3] = 0x00020000;
  return r;
}

constexpr uint32_t kOOB = 0x80000000u;

// s_waitcnt immediate, gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4], lgkmcnt [11:8] = 0
constexpr int wait_vm_lgkm0(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4); }

// ============================================================================
// LDS layout of a 128-byte k stage: a 128-byte slice of each of the tile's 256 A
// rows and 256 B rows (64 KB), loaded as whole cache lines.  Two stage slots: A
// at [0, 64K), B at [64K, 128K), 32 KB each; rows of 8 chunks of 16 bytes stored
// at chunk ^ f(row), f(r) = (r & 7) ^ ((r >> 3) & 3), which keeps the 8- and
// 16-lane groups of a fragment read (one logical chunk, consecutive rows) on
// distinct banks.
// ============================================================================
constexpr int PK = 128;                  // k bytes per stage row
constexpr int kPairOp = BM * PK;         // 32 KB: one operand, one stage
constexpr int kPB = 2 * kPairOp;         // B stage slots start at 64 KB

__device__ __forceinline__ int f8(int row) { return (row & 7) ^ ((row >> 3) & 3); }

// ============================================================================
// Ping-pong pipeline: 8 waves, two per SIMD, in two groups of four.
//
// Each wave owns a 128 x 64 block of the 256 x 256 tile (waves 4 apart share a
// SIMD, the same 128 rows and neighbouring 64-column halves).  The groups
// alternate between a compute phase (16 FP8 MFMAs over one 128-byte k stage
// held in registers, about 1024 cycles) and a memory phase (the next stage's
// fragments from LDS, plus global->LDS loads of a later stage: A from group 0, B
// from group 1), so on every SIMD one wave keeps the matrix core busy while the
// other waits on LDS and memory.  Two barriers per stage keep the rhythm:
//
//   phase 2s   : group 0 computes stage s    | group 1 reads stage s
//   barrier X  : group 0 has waited for its loads of stage s+1 -> stage s+1
//                is visible; group 1 has its stage-s fragments
//   phase 2s+1 : group 0 reads stage s+1 and | group 1 computes stage s
//                loads A of stage s+2 into the
//                slot of stage s (read by both
//                groups before X)
//   barrier Y  : group 1 then reads stage s+1 and loads B of a later stage
//                into a slot both groups have finished reading
//
// A gets two phases (one stage) of latency, B three.  LDS: stage slots in the
// layout of the pair pipeline above (A [0, 64K), B from 64K, rows of 8 swizzled
// 16-byte chunks).  Correctness does not depend on which SIMD a wave lands on;
// only the overlap does.
// ============================================================================
constexpr int NT8 = 512;

// FUSED: the epilogue also reduces max |D| over the grid into *p.amax (the caller's
// workspace holds the counters) and can write D as FP8 codes with the scale *p.d_scale.
template <int KIND, int AF, int BF, bool PANEL = false, bool FUSED = false>
__global__ __launch_bounds__(NT8, 1) void k_gemm4(Params p) {
  constexpr bool MX4 = KIND == KIND_MX4;
  constexpr bool MX = KIND == KIND_MX || MX4;
  // PANEL (MX only): the E8M0 scales come in the panel layout, so every wave loads the
  // scales of its own rows straight into registers as whole lines, and LDS holds A in
  // two stage slots and B in three, as for FP8.
  constexpr bool RSC = MX && PANEL;
  // The two groups share the global->LDS loads, each in its own memory phases: group 0
  // loads A, group 1 loads B.  FP8/BF16 (SPLIT): A in two stage slots, B in three.  MX:
  // two slots each (group 0 also loads the scales), plus per stage slot the E8M0 block
  // scales of the stage's 128 bytes of each row: one dword (four blocks of 32 FP8
  // elements) per row of A (1 KB) and of B (1 KB); MXFP4 two dwords (eight blocks of 32
  // E2M1 elements), kept as four 1 KB arrays (A dword 0, A dword 1, B dword 0, B dword 1).
  constexpr bool SPLIT = !MX || PANEL;
  constexpr int kScOff = 2 * kPB, kScSlot = MX4 ? 4096 : 2048;
  constexpr int kLds = SPLIT ? kPB + 3 * kPairOp : 2 * kPB + 2 * kScSlot;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];

  const int nb = p.nbm * p.nbn;
  // split-K: blocks [z * nb, (z + 1) * nb) take k split z of every tile
  const int zsplit = static_cast<int>(blockIdx.x) / nb;
  const int bid = static_cast<int>(blockIdx.x) - zsplit * nb;
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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, q4 = wave & 3;
  const int wm = (q4 >> 1) * 128, wn = (q4 & 1) * 128 + grp * 64;
  const int lr = lane & 31, lk = lane >> 5;

  const int rows_a = (p.M - m0) < BM ? (p.M - m0) : BM;
  const int rows_b = (p.N - n0) < BN ? (p.N - n0) : BN;
  const v4i rsA = make_rsrc(p.a + static_cast<int64_t>(m0) * p.KB, static_cast<uint32_t>(rows_a) * p.KB);
  const v4i rsB = make_rsrc(p.b + static_cast<int64_t>(n0) * p.KB, static_cast<uint32_t>(rows_b) * p.KB);

  // global->LDS: wave q4 moves rows [64 q4, 64 q4 + 64) of A and/or of B, 8 rows
  // per instruction t (lane j: row 64 q4 + 8t + j/8, physical chunk j % 8, logical chunk
  // (j % 8) ^ f(row) = c0 ^ (t & 3) with c0 = (j % 8) ^ (j / 8))
  const int c0 = (lane & 7) ^ (lane >> 3);
  const uint32_t ld_base = static_cast<uint32_t>(q4 * 64 + (lane >> 3)) * static_cast<uint32_t>(p.KB);
  // MX scales (k % 128 == 0 here): stage st of row r is the dword at r * kblocks + 4 st
  // (MXFP4, k % 256 == 0: the two dwords at r * kblocks + 8 st); lane l of group-0 wave
  // q4 fetches row 64 q4 + l of A and of B (rows past m or n read 0)
  v4i rsSA = {0, 0, 0, 0}, rsSB = {0, 0, 0, 0};
  if constexpr (MX) {
    rsSA = make_rsrc(static_cast<const uint8_t*>(p.a_scale) + static_cast<int64_t>(m0) * p.kblocks,
                     static_cast<uint32_t>(rows_a) * p.kblocks);
    rsSB = make_rsrc(static_cast<const uint8_t*>(p.b_scale) + static_cast<int64_t>(n0) * p.kblocks,
                     static_cast<uint32_t>(rows_b) * p.kblocks);
  }
  const uint32_t sc_off = static_cast<uint32_t>(q4 * 64 + lane) * static_cast<uint32_t>(p.kblocks);
  // 128-byte k stages (a ragged end reads as zeros); split z takes stages
  // [z S_all / splits, (z + 1) S_all / splits) (MX: one split)
  const int S_all = (p.KB + PK - 1) / PK;
  const int s_begin = zsplit * S_all / p.splits;
  const int S = (zsplit + 1) * S_all / p.splits - s_begin;
  // PANEL scales: in the panel layout the dword of row r and 128-element group g is
  // dword ((r / 256) * G + g) * 256 + r % 256, G = k / 128; the tile's rows are one
  // panel (m0 and n0 are multiples of 256), so a stage's dwords of 64 consecutive rows
  // are 256 contiguous bytes.  Lane l holds A rows wm + l and wm + 64 + l (row groups
  // lk and 2 + lk of its fragments) and B row wn + l (group lk); the scales of the
  // other half-wave's row groups come by a lane swap when a stage is packed.  Two
  // stages (a window) are loaded at a time, one window ahead.  Rows past m or n read
  // the padding of the last panel: their outputs are never stored.
  constexpr int SDW = MX4 ? 2 : 1;  // scale dwords per row and stage
  constexpr int WDW = 2 * SDW;      // per row and window of two stages
  const uint32_t* scA0 = nullptr;
  const uint32_t* scA1 = nullptr;
  const uint32_t* scB = nullptr;
  if constexpr (RSC) {
    const int64_t G = p.kblocks / 4;
    scA0 = static_cast<const uint32_t*>(p.a_scale) + (static_cast<int64_t>(m0 / BM) * G) * 256 + wm + lane;
    scA1 = scA0 + 64;
    scB = static_cast<const uint32_t*>(p.b_scale) + (static_cast<int64_t>(n0 / BN) * G) * 256 + wn + lane;
  }
  uint32_t nA0[WDW], nA1[WDW], nB[WDW], cA0[WDW], cA1[WDW], cB[WDW];
  // Stage 2w exists; past the row's last stage the index is clamped to its last dword
  // (read, never used).  The loads are unconditional: a conditional one would make the
  // compiler wait on the register's earlier load, and so on every older load in flight.
  const int last_dw = S * SDW - 1;
  auto load_window = [&](int w) {
#pragma unroll
    for (int d = 0; d < WDW; ++d) {
      const int64_t i = static_cast<int64_t>(min(w * WDW + d, last_dw)) * 256;
      nA0[d] = scA0[i];
      nA1[d] = scA1[i];
      nB[d] = scB[i];
    }
  };
  auto issue_scales = [&](auto SLOT, int st) {
    constexpr int slot = decltype(SLOT)::value;
    if constexpr (MX) {
      const int sbase = kScOff + slot * kScSlot + q4 * 256;
      if constexpr (MX4) {
        const uint32_t so = sc_off + 8u * st;
        raw_buffer_load_lds(rsSA, (__attribute__((address_space(3))) uint32_t*)(smem + sbase), 4,
                            static_cast<int>(so), 0, 0, 0);
        raw_buffer_load_lds(rsSA, (__attribute__((address_space(3))) uint32_t*)(smem + sbase + 1024), 4,
                            static_cast<int>(so + 4u), 0, 0, 0);
        raw_buffer_load_lds(rsSB, (__attribute__((address_space(3))) uint32_t*)(smem + sbase + 2048), 4,
                            static_cast<int>(so), 0, 0, 0);
        raw_buffer_load_lds(rsSB, (__attribute__((address_space(3))) uint32_t*)(smem + sbase + 3072), 4,
                            static_cast<int>(so + 4u), 0, 0, 0);
      } else {
        raw_buffer_load_lds(rsSA, (__attribute__((address_space(3))) uint32_t*)(smem + sbase), 4,
                            static_cast<int>(sc_off + 4u * st), 0, 0, 0);
        raw_buffer_load_lds(rsSB, (__attribute__((address_space(3))) uint32_t*)(smem + sbase + 1024), 4,
                            static_cast<int>(sc_off + 4u * st), 0, 0, 0);
      }
    }
  };
  // one operand of one stage (8 loads per lane), into the slot at byte offset off_slot
  auto issue_op = [&](const v4i& rs, int off_slot, int st) {
    const uint32_t kb = static_cast<uint32_t>(s_begin + st) * PK;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t cb = static_cast<uint32_t>((c0 ^ (t & 3)) << 4);
      const uint32_t off = (kb + cb < static_cast<uint32_t>(p.KB))
                               ? ld_base + static_cast<uint32_t>(t * 8) * static_cast<uint32_t>(p.KB) + kb + cb
                               : kOOB;
      const int base = off_slot + (q4 * 64 + t * 8) * PK;
      raw_buffer_load_lds(rs, (__attribute__((address_space(3))) uint32_t*)(smem + base), 16,
                          static_cast<int>(off), 0, 0, 0);
    }
  };
  auto issue_a = [&](auto SLOT, int st) { issue_op(rsA, decltype(SLOT)::value * kPairOp, st); };
  auto issue_b = [&](int st) { issue_op(rsB, kPB + (st % 3) * kPairOp, st); };
  // MX: group 0 loads A and the scales of a stage, group 1 its B, both into slot st % 2
  auto issue_b2 = [&](auto SLOT, int st) { issue_op(rsB, kPB + decltype(SLOT)::value * kPairOp, st); };
  constexpr int kLoadsA = 8 + (MX4 ? 4 : 2);

  // A phase covers NH of the stage's k steps (two of 64 bytes for FP8, MX and BF16,
  // four of 32 bytes for MXFP4): both for FP8 and BF16; one for MX, whose scaled MFMA
  // needs a fresh accumulator tuple per instruction and so cannot also hold a whole
  // stage of fragments within 256 registers; two for MXFP4 (half-size fragments).
  constexpr int KSTEPS = MX4 ? 4 : 2;
  constexpr int NH = MX4 ? 2 : (MX ? 1 : 2);
  constexpr int PPS = KSTEPS / NH;  // phases per stage and group

  // fragments: A rows wm + 32 i + lr (i < 4), B rows wn + 32 j + lr (j < 2); k step h of
  // the stage uses logical chunks 4h + lk (low 16 bytes) and 4h + 2 + lk (high 16 bytes).
  // A row base wm + lr (a multiple of 128 bytes) or'd with the swizzled chunk: chunk
  // 4h + lk + 2x is (lk ^ f(lr)) ^ (4h + 2x), i.e. the address bits 6 and 5 flip
  const int fk = f8(lr);
  const int ra0 = (wm + lr) * PK + ((lk ^ fk) << 4);
  const int rb0 = kPB + (wn + lr) * PK + ((lk ^ fk) << 4);
  // MXFP4 fragments: k step h (64 elements, 32 bytes) of a row is logical chunk
  // 2h + lk, the 32 elements this lane supplies, so one 16-byte read; the matrix core
  // reads only the first four registers of an E2M1 operand.
  using Frag = std::conditional_t<MX4, v4u, v8i>;
  Frag fa[NH][4], fb[NH][2];
  // MX: this lane's block scales for the stage.  A lane supplies the scale of block
  // 2h + lk of its row for k step h; two row groups share a dword: byte 2h + g holds
  // row group 2p + g (A: dwords p = 0, 1; B: one dword for its two row groups).
  // MXFP4: one dword per row group, byte x4_sel(h) = block 2h + lk of the row.
  uint32_t sa2[2] = {0u, 0u}, sb1 = 0u;
  uint32_t sa4[4] = {0u, 0u, 0u, 0u}, sb4[2] = {0u, 0u};
  // read the fragments of part P (k steps P*NH ..) of stage st, whose A is in SLOT
  auto read_part = [&](auto SLOT, auto PART, int st) {
    constexpr int slot = decltype(SLOT)::value;
    constexpr int part = decltype(PART)::value;
    const int boff = (SPLIT ? st % 3 : slot) * kPairOp;
    if constexpr (RSC) {
      if constexpr (part == 0) {
        // stage parity = A slot: an even stage opens a window (its scales are in the
        // loaded window, which then becomes the current one), an odd stage closes it
        constexpr bool opens = slot == 0;
        uint32_t A0[SDW], A1[SDW], Bv[SDW];
#pragma unroll
        for (int d = 0; d < SDW; ++d) {
          A0[d] = opens ? nA0[d] : cA0[SDW + d];
          A1[d] = opens ? nA1[d] : cA1[SDW + d];
          Bv[d] = opens ? nB[d] : cB[SDW + d];
        }
        if constexpr (opens) {
#pragma unroll
          for (int d = 0; d < WDW; ++d) {
            cA0[d] = nA0[d];
            cA1[d] = nA1[d];
            cB[d] = nB[d];
          }
        }
        // row groups: the half-waves hold groups (0, 2) and (1, 3) of A, 0 and 1 of B;
        // v_permlane32_swap of a register with itself gives every lane the value of lane
        // l % 32 (lower half-wave) and of lane l % 32 + 32 (upper half-wave)
        uint32_t G4[4][SDW], H2[2][SDW];
#pragma unroll
        for (int d = 0; d < SDW; ++d) {
          const auto x0 = __builtin_amdgcn_permlane32_swap(A0[d], A0[d], false, false);
          const auto x1 = __builtin_amdgcn_permlane32_swap(A1[d], A1[d], false, false);
          const auto xb = __builtin_amdgcn_permlane32_swap(Bv[d], Bv[d], false, false);
          G4[0][d] = x0[0];
          G4[1][d] = x0[1];
          G4[2][d] = x1[0];
          G4[3][d] = x1[1];
          H2[0][d] = xb[0];
          H2[1][d] = xb[1];
        }
        // keep the bytes of this lane's blocks (lk, 2 + lk of each dword)
        auto pick = [&](uint32_t w0, uint32_t w1) {
          return ((w0 >> (8 * lk)) & 0x00ff00ffu) | (((w1 >> (8 * lk)) & 0x00ff00ffu) << 8);
        };
        if constexpr (MX4) {
          // dword 0 of a row holds blocks 0-3 of the stage, dword 1 blocks 4-7
#pragma unroll
          for (int i = 0; i < 4; ++i) sa4[i] = pick(G4[i][0], G4[i][SDW - 1]);
#pragma unroll
          for (int j = 0; j < 2; ++j) sb4[j] = pick(H2[j][0], H2[j][SDW - 1]);
        } else {
          sa2[0] = pick(G4[0][0], G4[1][0]);
          sa2[1] = pick(G4[2][0], G4[3][0]);
          sb1 = pick(H2[0][0], H2[1][0]);
        }
      }
    } else if constexpr (MX4) {
      if constexpr (part == 0) {
        // dword 0 of a row holds blocks 0-3 of the stage, dword 1 blocks 4-7; keep the
        // bytes of this lane's blocks: (b lk, b 2+lk, b 4+lk, b 6+lk) -> bytes (0, 2, 1, 3)
        const uint32_t* sc = reinterpret_cast<const uint32_t*>(smem + kScOff + slot * kScSlot);
        auto pack4 = [&](uint32_t d0, uint32_t d1) {
          return ((d0 >> (8 * lk)) & 0x00ff00ffu) | (((d1 >> (8 * lk)) & 0x00ff00ffu) << 8);
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) sa4[i] = pack4(sc[wm + 32 * i + lr], sc[256 + wm + 32 * i + lr]);
#pragma unroll
        for (int j = 0; j < 2; ++j) sb4[j] = pack4(sc[512 + wn + 32 * j + lr], sc[768 + wn + 32 * j + lr]);
      }
    } else if constexpr (MX) {
      if constexpr (part == 0) {
        const uint32_t* sc = reinterpret_cast<const uint32_t*>(smem + kScOff + slot * kScSlot);
        auto pack = [&](uint32_t w0, uint32_t w1) {
          return ((w0 >> (8 * lk)) & 0x00ff00ffu) | (((w1 >> (8 * lk)) & 0x00ff00ffu) << 8);
        };
        sa2[0] = pack(sc[wm + lr], sc[wm + 32 + lr]);
        sa2[1] = pack(sc[wm + 64 + lr], sc[wm + 96 + lr]);
        sb1 = pack(sc[256 + wn + lr], sc[256 + wn + 32 + lr]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int h = part * NH + hh;
      if constexpr (MX4) {
        const int ao = ra0 ^ (h << 5), bo = rb0 ^ (h << 5);  // logical chunk 2h + lk
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[hh][i] = *reinterpret_cast<const v4u*>(smem + ao + slot * kPairOp + i * 32 * PK);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[hh][j] = *reinterpret_cast<const v4u*>(smem + (bo + boff) + j * 32 * PK);
        continue;
      }
      const int alo = ra0 ^ (h << 6), ahi = ra0 ^ (h << 6) ^ 32;
      const int blo = rb0 ^ (h << 6), bhi = rb0 ^ (h << 6) ^ 32;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = slot * kPairOp + i * 32 * PK;
        const v4u lo = *reinterpret_cast<const v4u*>(smem + alo + o);
        const v4u hi = *reinterpret_cast<const v4u*>(smem + ahi + o);
        if constexpr (!MX4) fa[hh][i] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int o = j * 32 * PK;
        const v4u lo = *reinterpret_cast<const v4u*>(smem + (blo + boff) + o);
        const v4u hi = *reinterpret_cast<const v4u*>(smem + (bhi + boff) + o);
        if constexpr (!MX4) fb[hh][j] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{0};

  // MX MFMA for k step H, A row group I, B row group J: opsel picks byte 2H + (group & 1)
  // of the packed scale dwords
  auto mfma_mx = [&](auto H, auto I, auto J, const v8i& a, const v8i& b) {
    constexpr int h = decltype(H)::value, i = decltype(I)::value, j = decltype(J)::value;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        a, b, acc[i][j], AF, BF, 2 * h + (i & 1), static_cast<int>(sa2[i >> 1]), 2 * h + j, static_cast<int>(sb1));
  };
  // MXFP4 MFMA for k step h: E2M1 operands (format 4) in the low four registers
  auto mfma_x4 = [&](auto H, int i, int j, const v4u& a, const v4u& b) {
    constexpr int h = decltype(H)::value;
    constexpr int sel = ((h & 1) << 1) | (h >> 1);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        __builtin_bit_cast(v8i, __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3)),
        __builtin_bit_cast(v8i, __builtin_shufflevector(b, b, 0, 1, 2, 3, 0, 1, 2, 3)), acc[i][j], 4, 4, sel,
        static_cast<int>(sa4[i]), sel, static_cast<int>(sb4[j]));
  };
  auto compute_part = [&](auto PART) {
    constexpr int part = decltype(PART)::value;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      if constexpr (MX4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (hh == 0) mfma_x4(ic<part * NH>{}, i, j, fa[0][i], fb[0][j]);
            else mfma_x4(ic<part * NH + 1>{}, i, j, fa[1][i], fb[1][j]);
          }
      } else if constexpr (KIND == KIND_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const v8i a = fa[hh][i], b = fb[hh][j];
              const v8bf av = __builtin_bit_cast(v8bf, q ? __builtin_shufflevector(a, a, 4, 5, 6, 7)
                                                         : __builtin_shufflevector(a, a, 0, 1, 2, 3));
              const v8bf bv = __builtin_bit_cast(v8bf, q ? __builtin_shufflevector(b, b, 4, 5, 6, 7)
                                                         : __builtin_shufflevector(b, b, 0, 1, 2, 3));
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i][j], 0, 0, 0);
            }
      } else if constexpr (MX) {
        constexpr int h = part;  // NH == 1
        mfma_mx(ic<h>{}, ic<0>{}, ic<0>{}, fa[0][0], fb[0][0]);
        mfma_mx(ic<h>{}, ic<0>{}, ic<1>{}, fa[0][0], fb[0][1]);
        mfma_mx(ic<h>{}, ic<1>{}, ic<0>{}, fa[0][1], fb[0][0]);
        mfma_mx(ic<h>{}, ic<1>{}, ic<1>{}, fa[0][1], fb[0][1]);
        mfma_mx(ic<h>{}, ic<2>{}, ic<0>{}, fa[0][2], fb[0][0]);
        mfma_mx(ic<h>{}, ic<2>{}, ic<1>{}, fa[0][2], fb[0][1]);
        mfma_mx(ic<h>{}, ic<3>{}, ic<0>{}, fa[0][3], fb[0][0]);
        mfma_mx(ic<h>{}, ic<3>{}, ic<1>{}, fa[0][3], fb[0][1]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[hh][i], fb[hh][j], acc[i][j], AF, BF,
                                                                       0, 0, 0, 0);
      }
    }
  };

  const int T = S * PPS;  // phases per group

  // Both groups run the same loop body, compute part u | barrier | read part u+1 |
  // barrier, so compute and fragment reads are one code path; group 1 runs it one
  // phase behind group 0 (one extra barrier before its loop, matched by one after
  // group 0's).  Group 0 waits for its loads of the next stage at the end of a stage's
  // last part, and after the barrier loads A of the stage after that into the slot both
  // groups have finished reading.  Group 1 loads B: three slots deep for FP8/BF16; for
  // MX (two phases per stage) it waits for B of stage s+1 in the memory phase after
  // part 0 of stage s, and loads B of stage s+2 into the slot of stage s in the one
  // after the last part, when both groups have read that slot.
  if constexpr (SPLIT) {
    // group 0 loads A of stages 0 and 1, group 1 B of stages 0, 1 and (after the
    // prologue) 2; each waits for its stage-0 half (and, PANEL, the scales of stages 0
    // and 1, issued first) before the first barrier
    if constexpr (RSC) load_window(0);
    if (grp == 0) {
      issue_a(ic<0>{}, 0);
      if (S > 1) issue_a(ic<1>{}, 1);
    } else {
      issue_b(0);
      if (S > 1) issue_b(1);
    }
    if (S > 1) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(8));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  } else {
    if (grp == 0) {
      issue_scales(ic<0>{}, 0);
      issue_a(ic<0>{}, 0);
      if (S > 1) {
        issue_scales(ic<1>{}, 1);
        issue_a(ic<1>{}, 1);
      }
    } else {
      issue_b2(ic<0>{}, 0);
      if (S > 1) issue_b2(ic<1>{}, 1);
    }
    if (S > 1) {
      if (grp == 0) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kLoadsA));
      else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(8));
    } else {
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    }
  }
  __builtin_amdgcn_s_barrier();  // stage 0 visible
  read_part(ic<0>{}, ic<0>{}, 0);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
  __builtin_amdgcn_s_barrier();
  if (grp == 1) {
    if constexpr (SPLIT) {
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // B of stage 1 landed
      if (S > 2) issue_b(2);                         // its slot has never been used
    }
    __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_sched_barrier(0);

  // phase u = PPS * s + part; U = u mod 2 PPS fixes slot and part at compile time.
  // Group 0 at the end of a stage's last part waits for its loads of stage s+1 (A, or
  // everything without SPLIT) and after the barrier loads stage s+2 into the slot both
  // groups have finished reading.  Group 1 (SPLIT) in its memory phase after stage s
  // waits for B of stage s+2 and loads B of stage s+3 into the slot of stage s.
  auto iter = [&](auto U, int u) {
    constexpr int uu = decltype(U)::value;
    constexpr int slot = (uu / PPS) & 1, part = uu % PPS;
    constexpr bool last_part = part == PPS - 1;
    constexpr int nslot = last_part ? (slot ^ 1) : slot, npart = last_part ? 0 : part + 1;
    const int s = u / PPS;
    compute_part(ic<part>{});
    if constexpr (MX) {
      // pin the phase's scaled MFMAs here: left free, the optimizer gathers them across
      // phases and the live fragments overflow the register file
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    __builtin_amdgcn_sched_barrier(0);
    // PANEL: loads and waits do not depend on s (past the last stage they read zeros
    // into a free slot), so every path through the loop has the same loads in flight and
    // the compiler's waits for the scale registers count exactly the younger loads
    constexpr bool kUncond = RSC;
    if (last_part && grp == 0 && (kUncond || s + 1 < S)) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // stage s+1 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (u + 1 < T) read_part(ic<nslot>{}, ic<npart>{}, last_part ? s + 1 : s);
    if constexpr (SPLIT) {
      // PANEL: the first phase of a window (part 0 of an even stage) loads the next
      // window's scales; the part-0 read of its first stage comes three memory phases later
      if constexpr (RSC) {
        if (uu == 0) load_window(s / 2 + 1);
      }
      if (last_part && grp == 0 && (kUncond || s + 2 < S)) issue_a(ic<slot>{}, s + 2);  // the A slot of stage s is free
      if (last_part && grp == 1) {
        if (kUncond || s + 2 < S) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // B of stage s+2 landed
        if (kUncond || s + 3 < S) issue_b(s + 3);                                // into the B slot of stage s
      }
    } else {
      if (last_part && grp == 0 && s + 2 < S) {  // the slot of stage s is free
        issue_scales(ic<slot>{}, s + 2);
        issue_a(ic<slot>{}, s + 2);
      }
      if (grp == 1) {
        if (!last_part && s + 1 < S) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // B of stage s+1 landed
        if (last_part && s + 2 < S) issue_b2(ic<slot>{}, s + 2);                       // into the slot of stage s
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  int u = 0;
  for (; u + 2 * PPS - 1 < T; u += 2 * PPS) {
    iter(ic<0>{}, u);
    iter(ic<1>{}, u + 1);
    if constexpr (PPS == 2) {
      iter(ic<2>{}, u + 2);
      iter(ic<3>{}, u + 3);
    }
  }
  if (u < T) iter(ic<0>{}, u);
  if (u + 1 < T) iter(ic<1>{}, u + 1);
  if constexpr (PPS == 2) {
    if (u + 2 < T) iter(ic<2>{}, u + 2);
  }
  // PANEL: loads issued past the last stage still write LDS; drain them before the
  // epilogue stages the output there
  if constexpr (RSC) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  if (grp == 0) __builtin_amdgcn_s_barrier();

  // ---- epilogue: scale, bias, round; staged through LDS for full-row 16-byte stores ----
  // Each wave owns a 128 x 64 block, written in two passes of 64 rows through its own
  // 16 KB LDS region (64 rows x 64 floats): a half-wave writes 32 consecutive floats
  // of a row, then each lane reads 8 (bf16 out) or 4 (fp32 out) consecutive floats.
  float sa = 1.0f, sb = 1.0f;
  if constexpr (KIND == KIND_FP8) {
    sa = *static_cast<const float*>(p.a_scale);
    sb = *static_cast<const float*>(p.b_scale);
  }
  float bias_v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn + j * 32 + lr;
    bias_v[j] = 0.0f;
    if (p.bias != nullptr && col < p.N)
      bias_v[j] = p.bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p.bias)[col]) << 16)
                              : static_cast<const float*>(p.bias)[col];
  }
  constexpr int kEpPitch = 256;             // bytes per staged row (64 floats)
  constexpr int kEpRegion = 64 * kEpPitch;  // 16 KB per wave
  static_assert(8 * kEpRegion <= 2 * kPB, "epilogue staging must fit in the stage slots");
  float* ep = reinterpret_cast<float*>(smem + wave * kEpRegion);
  // FUSED: running max of |D| over this lane's stored outputs, as magnitude bits (NaN,
  // whose bits are largest, wins); FP8 output scale
  uint32_t mbits = 0u;
  float s_out = 1.0f;
  if constexpr (FUSED) {
    if (p.d_fp8) {
      s_out = *p.d_scale;
      if (blockIdx.x == 0 && tid == 0) *p.d_scale_inv = 1.0f / s_out;
    }
  }
  // every wave's last LDS reads finished before the final barrier of the k loop
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = pass * 2 + ii;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float val = acc[i][j][v];
          if (!p.partial) {
            if constexpr (KIND == KIND_FP8) val = __fmul_rn(__fmul_rn(val, sa), sb);
            if (p.bias != nullptr) val = __fadd_rn(val, bias_v[j]);
          }
          const int r = ii * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
          ep[r * (kEpPitch / 4) + j * 32 + lr] = val;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    __builtin_amdgcn_wave_barrier();
    const int row0 = m0 + wm + pass * 64;
    const int col0 = n0 + wn;
    // Output goes out with nontemporal stores: a tile round writes as much as the L2
    // holds, and cached stores would evict the operand panels the next k steps reuse.
    if (FUSED && p.d_fp8) {
      // FP8 codes of eight consecutive outputs per lane: satRNE(fl32(d * scale))
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = t * 8 + (lane >> 3);
        const int c = (lane & 7) * 8;
        const float4 lo = *reinterpret_cast<const float4*>(ep + r * (kEpPitch / 4) + c);
        const float4 hi = *reinterpret_cast<const float4*>(ep + r * (kEpPitch / 4) + c + 4);
        const int grow = row0 + r, gcol = col0 + c;
        if (grow < p.M && gcol < p.N) {
          const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
          for (int q = 0; q < 8; ++q) mbits = max(mbits, __float_as_uint(v[q]) & 0x7fffffffu);
          v2u o;
          if (p.d_fp8 == 2) {
            o[0] = quant4<true>(v[0], v[1], v[2], v[3], s_out);
            o[1] = quant4<true>(v[4], v[5], v[6], v[7], s_out);
          } else {
            o[0] = quant4<false>(v[0], v[1], v[2], v[3], s_out);
            o[1] = quant4<false>(v[4], v[5], v[6], v[7], s_out);
          }
          __builtin_nontemporal_store(
              o, reinterpret_cast<v2u*>(static_cast<uint8_t*>(p.d) + static_cast<int64_t>(grow) * p.N + gcol));
        }
      }
    } else if (p.d_bf16) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = t * 8 + (lane >> 3);
        const int c = (lane & 7) * 8;
        const float4 lo = *reinterpret_cast<const float4*>(ep + r * (kEpPitch / 4) + c);
        const float4 hi = *reinterpret_cast<const float4*>(ep + r * (kEpPitch / 4) + c + 4);
        const int grow = row0 + r, gcol = col0 + c;
        if (grow < p.M && gcol < p.N) {
          const v4u o = {bf16x2_rne(lo.x, lo.y), bf16x2_rne(lo.z, lo.w), bf16x2_rne(hi.x, hi.y),
                         bf16x2_rne(hi.z, hi.w)};
          if constexpr (FUSED) {  // the stored bf16 magnitudes, widened: max over both halves
#pragma unroll
            for (int q = 0; q < 4; ++q)
              mbits = max(mbits, max((o[q] << 16) & 0x7fffffffu, o[q] & 0x7fff0000u));
          }
          __builtin_nontemporal_store(
              o, reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.d) + static_cast<int64_t>(grow) * p.N + gcol));
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int r = t * 4 + (lane >> 4);
        const int c = (lane & 15) * 4;
        v4f v4 = *reinterpret_cast<const v4f*>(ep + r * (kEpPitch / 4) + c);
        const int grow = row0 + r, gcol = col0 + c;
        if (grow < p.M && gcol < p.N) {
          float* dbase = static_cast<float*>(p.d) + (p.partial ? static_cast<int64_t>(zsplit) * p.M * p.N : 0);
          v4f* dst = reinterpret_cast<v4f*>(dbase + static_cast<int64_t>(grow) * p.N + gcol);
          if (p.accumulate) {  // fp32 main-gradient accumulation: D = fl32(D_old + result)
            const v4f old = __builtin_nontemporal_load(dst);
#pragma unroll
            for (int q = 0; q < 4; ++q) v4[q] = __fadd_rn(old[q], v4[q]);
          }
          if constexpr (FUSED) {
#pragma unroll
            for (int q = 0; q < 4; ++q) mbits = max(mbits, __float_as_uint(v4[q]) & 0x7fffffffu);
          }
          __builtin_nontemporal_store(v4, dst);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    __builtin_amdgcn_wave_barrier();
  }
  if constexpr (FUSED) {
    // the third B stage slot [128 KB, 160 KB) is not used by the epilogue's staging
    grid_amax<NT8>(__uint_as_float(mbits), p.amax, static_cast<AmaxWork*>(p.amax_ws), false,
                   reinterpret_cast<uint32_t*>(smem + 2 * kPB));
  }
}

// Split-K reduction: D = epilogue(sum over splits of the fp32 partials, in split
// order), the epilogue of k_gemm4: fl32(fl32(acc * sa) * sb) for FP8, then + bias,
// then bf16 (round to nearest even) or fp32.  Four consecutive outputs per thread
// (n % 16 == 0, so a group never crosses a row).
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int splits, int64_t mn, int n,
                                                       const float* __restrict__ a_scale,
                                                       const float* __restrict__ b_scale, int fp8,
                                                       const void* __restrict__ bias, int bias_bf16,
                                                       void* __restrict__ d, int d_bf16) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  auto part = [&](int z) { return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(ws + static_cast<int64_t>(z) * mn + i)); };
  auto add = [&](v4f& x, const v4f& v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = __fadd_rn(x[q], v[q]);
  };
  v4f acc = part(0);
  int z = 1;
  // four loads in flight per step, added in split order
  for (; z + 3 < splits; z += 4) {
    const v4f v0 = part(z), v1 = part(z + 1), v2 = part(z + 2), v3 = part(z + 3);
    add(acc, v0);
    add(acc, v1);
    add(acc, v2);
    add(acc, v3);
  }
  for (; z < splits; ++z) add(acc, part(z));
  const float sa = fp8 ? *a_scale : 1.0f, sb = fp8 ? *b_scale : 1.0f;
  const int col = static_cast<int>(i % n);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float val = acc[q];
    if (fp8) val = __fmul_rn(__fmul_rn(val, sa), sb);
    if (bias != nullptr)
      val = __fadd_rn(val, bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col + q]) << 16)
                                     : static_cast<const float*>(bias)[col + q]);
    acc[q] = val;
  }
  if (d_bf16) {
    const uint2 o = {bf16x2_rne(acc[0], acc[1]), bf16x2_rne(acc[2], acc[3])};
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(d) + i) = o;
  } else {
    *reinterpret_cast<v4f*>(static_cast<float*>(d) + i) = acc;
  }
}

thread_local const char* g_last_variant = "none";

// "<name>_splitk" for a variant name (stable pointers: the names are few and fixed)
const char* splitk_name(const char* name) {
  static std::mutex mu;
  static std::map<std::string, std::string> names;
  std::lock_guard<std::mutex> lock(mu);
  auto it = names.find(name);
  if (it == names.end()) it = names.emplace(name, std::string(name) + "_splitk").first;
  return it->second.c_str();
}

// ============================================================================
// One wave per SIMD with 16 x 16 x 128 MFMAs (per-tensor FP8 with k % 128 == 0; MXFP8
// and MXFP4 with panel-layout scales).
// With operands that change from one instruction to the next, as in a GEMM, the
// 16 x 16 x 128 FP8 instruction sustains about a tenth more FLOP/s than the 32 x 32 x 64
// one: both run below the published rate at the clocks the device holds under that
// load, the larger one further below (k_peak_rand in peak.hip: 4290 against 3900
// TFLOP/s with register operands only).  The outputs are bit-identical to k_gemm4's:
// every output sums the same products in the same k order.
// Four waves (2 x 2) each own a 128 x 128 block of the 256 x 256 tile, 8 x 8 MFMA
// tiles of 16 x 16, whose 64 accumulators (256 registers) live in AGPRs beside 256
// VGPRs.  One instruction takes a whole 128-byte stage of k for FP8 (64 MFMAs per stage
// over 8 + 8 fragments); an E2M1 stage holds 256 elements, two k steps of 128.  The
// operand with more rows (R) is read whole into registers during the stage before the
// one that uses it (two register sets); the other (T) is read one 16-row group ahead of
// the 8 MFMAs that use the group.
// Stage slots: R three -- its slot of stage s is free once stage s has been read into
// registers, so R loads run two stages ahead; T two -- T's slot of stage s is read all
// through stage s, so it is refilled in two parts: groups 0-2 of each wave's 128 rows
// (read before the stage's barrier) with stage s + 2 at that barrier, groups 3-7 (read
// after it) with stage s + 1 at the next one.  One barrier per stage, after its first
// two groups of MFMAs: before it every wave has read T's groups 0-2 of stage s, and R
// and T groups 0-2 of stage s + 1 and T groups 3-7 of stage s have landed; after it
// the wave reads R of stage s + 1 and the rest of T, and issues the loads of T groups
// 3-7 of s + 1, T groups 0-2 of s + 2 and R of s + 3, in that order, so that only R's
// are still in flight at the next barrier.  Each slot part is its own LDS array, so the
// compiler can tell the loads into one from the reads of another and adds no wait.
// Past the last stage the loads are sent out of range: they fetch nothing and fill
// slots that are never read again, so every iteration has the same shape.
// ============================================================================
template <int KIND, int AF, int BF, int DEEP>
__global__ __launch_bounds__(256, 1) void k_gemm1x(Params p) {
  constexpr bool MX4 = KIND == KIND_MX4;           // E2M1 elements: two 128-element k steps per stage
  constexpr bool MX = KIND == KIND_MX || MX4;      // E8M0 block scales, panel layout
  constexpr int KS = MX4 ? 2 : 1;                  // MFMA k steps per 128-byte stage
  constexpr bool RA = DEEP == 1;        // R is A (A has at least as many rows as B)
  __shared__ __attribute__((aligned(1024))) uint8_t sR0[kPairOp];
  __shared__ __attribute__((aligned(1024))) uint8_t sR1[kPairOp];
  __shared__ __attribute__((aligned(1024))) uint8_t sR2[kPairOp];
  // T slots in two arrays each: the rows of groups 0-2 of both 128-row halves (96 rows)
  // and of groups 3-7 (160 rows), so that the compiler can tell the loads into one part
  // from the reads of the other
  constexpr int kTa = 96 * PK, kTb = 160 * PK;
  __shared__ __attribute__((aligned(1024))) uint8_t sT0a[kTa];
  __shared__ __attribute__((aligned(1024))) uint8_t sT1a[kTa];
  __shared__ __attribute__((aligned(1024))) uint8_t sT0b[kTb];
  __shared__ __attribute__((aligned(1024))) uint8_t sT1b[kTb];
  auto slotR = [&](int slot) { return slot == 0 ? sR0 : slot == 1 ? sR1 : sR2; };
  auto slotTa = [&](int slot) { return slot == 0 ? sT0a : sT1a; };
  auto slotTb = [&](int slot) { return slot == 0 ? sT0b : sT1b; };
  const int nb = p.nbm * p.nbn;
  const int bid = static_cast<int>(blockIdx.x);
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
  // per-tensor scale_inv values, read once at the start (scalar loads; the kernel never
  // writes them)
  float sa = 1.0f, sb = 1.0f;
  if constexpr (!MX) {
    sa = *(const __attribute__((address_space(4))) float*)(reinterpret_cast<uintptr_t>(p.a_scale));
    sb = *(const __attribute__((address_space(4))) float*)(reinterpret_cast<uintptr_t>(p.b_scale));
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int l16 = lane & 15, lq = lane >> 4;
  const int rows_a = (p.M - m0) < BM ? (p.M - m0) : BM;
  const int rows_b = (p.N - n0) < BN ? (p.N - n0) : BN;
  const v4i rsA = make_rsrc(p.a + static_cast<int64_t>(m0) * p.KB, static_cast<uint32_t>(rows_a) * p.KB);
  const v4i rsB = make_rsrc(p.b + static_cast<int64_t>(n0) * p.KB, static_cast<uint32_t>(rows_b) * p.KB);
  const v4i rsR = RA ? rsA : rsB;
  const v4i rsT = RA ? rsB : rsA;
  const int S = (p.KB + PK - 1) / PK;
  // global->LDS: one instruction moves 8 rows (1 KB) from row rb; lane l lands at row
  // rb + (l >> 3), physical chunk l & 7, and fetches the logical chunk stored there.  In
  // this kernel's slots logical chunk c of row r sits at c ^ ((r >> 1) & 7): the two rows
  // of a 256-byte LDS line share the swizzle, which keeps a fragment read (16 rows x 4
  // chunks) free of bank conflicts; the swizzle of the other kernels (c ^ (r & 7) ^
  // ((r >> 3) & 3)) spent half of the LDS cycles here in conflicts
  auto voff_of = [&](int gb, int lb) {  // global row base, LDS row base (multiples of 8)
    return static_cast<uint32_t>(gb + (lane >> 3)) * static_cast<uint32_t>(p.KB) +
           static_cast<uint32_t>(((lane & 7) ^ (((lb + (lane >> 3)) >> 1) & 7)) << 4);
  };
  // R: wave w moves rows [64 w, 64 w + 64).  T: the 8-row units of groups 0-2 of both
  // 128-row halves (part 1: 12 units, 3 per wave; LDS rows 48 h + 16 g + ...) and of
  // groups 3-7 (part 2: 20 units, 5 per wave; LDS rows 80 h + 16 (g - 3) + ...); the
  // global row of an LDS row is 128 h + 16 g + ...
  uint32_t voR[8], voT1[3], voT2[5];
  int rbT1[3], rbT2[5];
#pragma unroll
  for (int t = 0; t < 8; ++t) voR[t] = voff_of(wave * 64 + t * 8, wave * 64 + t * 8);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const int q = wave * 3 + t, h = q / 6, r = q % 6;
    rbT1[t] = 48 * h + 16 * (r >> 1) + 8 * (r & 1);
    voT1[t] = voff_of(128 * h + 16 * (r >> 1) + 8 * (r & 1), rbT1[t]);
  }
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const int q = wave * 5 + t, h = q / 10, r = q % 10;
    rbT2[t] = 80 * h + 16 * (r >> 1) + 8 * (r & 1);
    voT2[t] = voff_of(128 * h + 16 * (3 + (r >> 1)) + 8 * (r & 1), rbT2[t]);
  }
  auto ld = [&](const v4i& rs, uint8_t* slot, int rb, uint32_t vo, int st) {
    // past the last stage: an offset beyond the buffer's range, so the load fetches
    // nothing (it writes zeros into a slot that is never read again)
    const uint32_t kb = __builtin_amdgcn_readfirstlane(st < S ? static_cast<uint32_t>(st) * PK : 0x40000000u);
    raw_buffer_load_lds(rs, (__attribute__((address_space(3))) uint32_t*)(slot + rb * PK), 16,
                        static_cast<int>(vo + kb), 0, 0, 0);
  };
  // load k (0 .. 15) of the set issued after stage s's barrier: T part 2 of stage s + 1,
  // T part 1 of stage s + 2, R of stage s + 3
  auto load_k = [&](int k, int ts, int rs, int s) {
    if (k < 5) ld(rsT, slotTb(ts ^ 1), rbT2[k], voT2[k], s + 1);
    else if (k < 8) ld(rsT, slotTa(ts), rbT1[k - 5], voT1[k - 5], s + 2);
    else ld(rsR, slotR(rs), wave * 64 + (k - 8) * 8, voR[k - 8], s + 3);
  };
  // fragments: lane l reads row 16 g + (l & 15) of the wave's 128, logical chunks l >> 4
  // (low 16 bytes) and 4 + (l >> 4) (high): the k order of the matrix instruction, so the
  // products are grouped and summed exactly as by the 32 x 32 x 64 instruction (outputs
  // bit-identical to the other FP8 kernels').  The offsets of even and odd groups are
  // computed alike (16 rows move the swizzle by 8), the group adds 16 g rows.  (T: group
  // g < 3 is LDS row 48 h + 16 g + (l & 15) of part 1, group g >= 3 row 80 h + 16 (g - 3)
  // + (l & 15) of part 2, h the wave's half of T's rows)
  const int th = (RA ? wn : wm) >> 7;
  int oR[2][2], oTa[2][2], oTb[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int rR = (RA ? wm : wn) + 16 * par + l16, rA = 48 * th + 16 * par + l16, rB = 80 * th + 16 * par + l16;
      oR[par][hh] = ((RA ? wm : wn) + l16) * PK + (((4 * hh + lq) ^ ((rR >> 1) & 7)) << 4);
      oTa[par][hh] = (48 * th + l16) * PK + (((4 * hh + lq) ^ ((rA >> 1) & 7)) << 4);
      oTb[par][hh] = (80 * th + l16) * PK + (((4 * hh + lq) ^ ((rB >> 1) & 7)) << 4);
    }
  // E2M1 k step h of a group: logical chunk 4 h + (l >> 4), one 16-byte read (the
  // instruction reads four registers of an E2M1 operand: the lane group's 32-element block)
  using Frag = std::conditional_t<MX4, v4u, v8i>;
  auto rd = [&](const uint8_t* slot, const int (&o)[2][2], int g) {
    const v4u lo = *reinterpret_cast<const v4u*>(slot + o[g & 1][0] + g * 16 * PK);
    const v4u hi = *reinterpret_cast<const v4u*>(slot + o[g & 1][1] + g * 16 * PK);
    return __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto rdF = [&](const uint8_t* slot, const int (&o)[2][2], int g, int h) -> Frag {
    if constexpr (MX4) return *reinterpret_cast<const v4u*>(slot + o[g & 1][h] + g * 16 * PK);
    else return rd(slot, o, g);
  };
  // T group g (k step h) of T slot ts
  auto rdT = [&](int ts, int g, int h) {
    return g < 3 ? rdF(slotTa(ts), oTa, g, h) : rdF(slotTb(ts), oTb, g - 3, h);
  };
  // MX: a lane's fragment data is 32-element block l >> 4 of its row's stage, so its scale
  // is byte l >> 4 of the row's dword in the panel layout (dword ((r / 256) G + g) 256 +
  // r % 256 for row r and 128-element group g; G = k / 128, one group per stage).  Per
  // operand and stage a lane loads the dwords of rows 16 (2 (l >> 4) + h) + (l & 15),
  // h = 0, 1, of the wave's 128 (two loads: the wave reads its 128 rows once), two stages
  // ahead; the bytes reach the lanes that need them through a transpose over the lane
  // groups (below), the stage before they are used.  (16 byte loads per stage instead
  // kept the address unit busy, 7% slower; a fetch through ds_bpermute, 11%.)  Buffers
  // over the tile's panel: stages past the last read 0.
  const v4i rsSR = make_rsrc(MX ? static_cast<const uint8_t*>(RA ? p.a_scale : p.b_scale) +
                                      static_cast<int64_t>((RA ? m0 : n0) / 256) * S * KS * 1024
                                : nullptr,
                             MX ? static_cast<uint32_t>(S * KS) * 1024u : 0u);
  const v4i rsST = make_rsrc(MX ? static_cast<const uint8_t*>(RA ? p.b_scale : p.a_scale) +
                                      static_cast<int64_t>((RA ? n0 : m0) / 256) * S * KS * 1024
                                : nullptr,
                             MX ? static_cast<uint32_t>(S * KS) * 1024u : 0u);
  const int scR = 4 * ((RA ? wm : wn) + 32 * lq + l16), scT = 4 * ((RA ? wn : wm) + 32 * lq + l16);
  // The lanes of group q hold the dwords of groups 2q and 2q + 1 (rows 16 (2q + h) + (l &
  // 15)); byte d of each is the scale lane group d needs: a 4 x 4 transpose of 2-byte items
  // over the lane groups, done with the two half-wave swaps (no LDS traffic)
  const bool odd = (lq & 1) != 0;
  const uint32_t selK = odd ? 0x07060302u : 0x05040100u;  // keep this group's items
  const uint32_t selS = odd ? 0x05040100u : 0x07060302u;  // send the partner's
  const uint32_t sel0 = odd ? 0x01000504u : 0x05040100u;  // groups 0-3 in source order
  const uint32_t sel1 = odd ? 0x03020706u : 0x07060302u;  // groups 4-7
  // packed scales: byte g & 3 of dword g >> 2 is the scale of group g
  // (E2M1: a stage holds two 128-element groups, k step h reads group 2 st + h)
  uint32_t rawR[2][KS][2], rawT[2][KS][2], Rsc[2][KS][2], Tsc[2][KS][2];  // raw: two stages in flight
  auto load_raw = [&](uint32_t (&dst)[KS][2], const v4i& rs, int off, int st) {
#pragma unroll
    for (int h = 0; h < KS; ++h) {
      const int so = __builtin_amdgcn_readfirstlane((st * KS + h) * 1024);
      dst[h][0] = static_cast<uint32_t>(buffer_load_u32(rs, off, so, 0));
      dst[h][1] = static_cast<uint32_t>(buffer_load_u32(rs, off + 64, so, 0));
    }
  };
  auto xpose1 = [&](uint32_t (&dst)[2], const uint32_t (&raw)[2]) {
    // items for destinations 0, 1 (A) and 2, 3 (B): (group 2q, group 2q + 1) byte pairs
    const uint32_t A = __builtin_amdgcn_perm(raw[1], raw[0], 0x05010400u);
    const uint32_t B = __builtin_amdgcn_perm(raw[1], raw[0], 0x07030602u);
    // half-waves: lanes 0-31 end with the items for destinations 0, 1, lanes 32-63 with
    // those for 2, 3 (P: source q or q - 2, Q: source q + 2 or q)
    const auto pq = __builtin_amdgcn_permlane32_swap(A, B, false, false);
    const uint32_t P = pq[0], Q = pq[1];
    // rows of 16 lanes in pairs: the even row keeps the lower destination's items and
    // sends the upper's, the odd row the other way round
    const uint32_t K = __builtin_amdgcn_perm(Q, P, selK);
    const uint32_t S2 = __builtin_amdgcn_perm(Q, P, selS);
    const auto xy = __builtin_amdgcn_permlane16_swap(S2, S2, false, false);
    const uint32_t R = odd ? xy[0] : xy[1];
    dst[0] = __builtin_amdgcn_perm(R, K, sel0);
    dst[1] = __builtin_amdgcn_perm(R, K, sel1);
  };
  auto xpose = [&](uint32_t (&dst)[KS][2], const uint32_t (&raw)[KS][2]) {
#pragma unroll
    for (int h = 0; h < KS; ++h) xpose1(dst[h], raw[h]);
  };
  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  Frag Rf[2][8][KS], Tf[2][KS];

  // prologue: T of stage 0 (both parts), R of stage 0, T part 1 of stage 1, R of stages
  // 1 and 2; then stage 0's R and first T group into registers
#pragma unroll
  for (int t = 0; t < 3; ++t) ld(rsT, sT0a, rbT1[t], voT1[t], 0);
#pragma unroll
  for (int t = 0; t < 5; ++t) ld(rsT, sT0b, rbT2[t], voT2[t], 0);
#pragma unroll
  for (int t = 0; t < 8; ++t) ld(rsR, sR0, wave * 64 + t * 8, voR[t], 0);
#pragma unroll
  for (int t = 0; t < 3; ++t) ld(rsT, sT1a, rbT1[t], voT1[t], 1);
#pragma unroll
  for (int t = 0; t < 8; ++t) ld(rsR, sR1, wave * 64 + t * 8, voR[t], 1);
#pragma unroll
  for (int t = 0; t < 8; ++t) ld(rsR, sR2, wave * 64 + t * 8, voR[t], 2);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 + 8 + 8));  // stage 0 landed
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int h = 0; h < KS; ++h) Rf[0][g][h] = rdF(sR0, oR, g, h);
#pragma unroll
  for (int h = 0; h < KS; ++h) Tf[0][h] = rdT(0, 0, h);
  if constexpr (MX) {
    load_raw(rawR[0], rsSR, scR, 0);
    load_raw(rawT[0], rsST, scT, 0);
    load_raw(rawR[1], rsSR, scR, 1);
    load_raw(rawT[1], rsST, scT, 1);
    xpose(Rsc[0], rawR[0]);
    xpose(Tsc[0], rawT[0]);
  }
  __builtin_amdgcn_sched_barrier(0);

  // one group of 8 MFMAs (T group t against R's 8), each followed by its share of the
  // fragment reads and global->LDS loads; the order is pinned (scheduling barriers).  The
  // MFMAs are written as instructions with the accumulator bound to AGPRs: through the
  // builtin, the register allocator spread the 64 four-register accumulators over both
  // register files and moved them back and forth (hundreds of spills and copies per
  // stage).  The compiler still counts the LDS waits for the operands it reads.
  // scaled: the scale of A is byte IA of sca, of B byte IB of scb (op_sel bit 0 and
  // op_sel_hi bit 0 give A's byte, bit 1 of each B's)
  auto mfma16s = [&](auto IA, auto IB, v4f& c, const Frag& a, const Frag& b, uint32_t sca, uint32_t scb) {
    constexpr int ia = decltype(IA)::value, ib = decltype(IB)::value;
#if defined(__HIP_DEVICE_COMPILE__)  // device pass only: the host pass cannot type the AGPR operands
#define TE_MFS(A0, B0, A1, B1, FMT)                                                                       \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #A0 "," #B0         \
               ",0] op_sel_hi:[" #A1 "," #B1 ",0]" FMT                                                  \
               : "+a"(c)                                                                                \
               : "v"(a), "v"(b), "v"(sca), "v"(scb))
#define TE_MFS_F(A0, B0, A1, B1)                                   \
  if constexpr (MX4) TE_MFS(A0, B0, A1, B1, " cbsz:4 blgp:4");     \
  else if constexpr (AF == 0 && BF == 0) TE_MFS(A0, B0, A1, B1, ""); \
  else if constexpr (AF == 1 && BF == 0) TE_MFS(A0, B0, A1, B1, " cbsz:1"); \
  else if constexpr (AF == 0 && BF == 1) TE_MFS(A0, B0, A1, B1, " blgp:1"); \
  else TE_MFS(A0, B0, A1, B1, " cbsz:1 blgp:1");
    if constexpr (ia == 0 && ib == 0) { TE_MFS_F(0, 0, 0, 0) }
    else if constexpr (ia == 1 && ib == 0) { TE_MFS_F(1, 0, 0, 0) }
    else if constexpr (ia == 2 && ib == 0) { TE_MFS_F(0, 0, 1, 0) }
    else if constexpr (ia == 3 && ib == 0) { TE_MFS_F(1, 0, 1, 0) }
    else if constexpr (ia == 0 && ib == 1) { TE_MFS_F(0, 1, 0, 0) }
    else if constexpr (ia == 1 && ib == 1) { TE_MFS_F(1, 1, 0, 0) }
    else if constexpr (ia == 2 && ib == 1) { TE_MFS_F(0, 1, 1, 0) }
    else if constexpr (ia == 3 && ib == 1) { TE_MFS_F(1, 1, 1, 0) }
    else if constexpr (ia == 0 && ib == 2) { TE_MFS_F(0, 0, 0, 1) }
    else if constexpr (ia == 1 && ib == 2) { TE_MFS_F(1, 0, 0, 1) }
    else if constexpr (ia == 2 && ib == 2) { TE_MFS_F(0, 0, 1, 1) }
    else if constexpr (ia == 3 && ib == 2) { TE_MFS_F(1, 0, 1, 1) }
    else if constexpr (ia == 0 && ib == 3) { TE_MFS_F(0, 1, 0, 1) }
    else if constexpr (ia == 1 && ib == 3) { TE_MFS_F(1, 1, 0, 1) }
    else if constexpr (ia == 2 && ib == 3) { TE_MFS_F(0, 1, 1, 1) }
    else { TE_MFS_F(1, 1, 1, 1) }
#undef TE_MFS_F
#undef TE_MFS
#endif
  };
  auto mfma16 = [&](v4f& c, const Frag& a, const Frag& b) {
#if defined(__HIP_DEVICE_COMPILE__)  // device pass only: the host pass cannot type the AGPR operands
    if constexpr (AF == 0 && BF == 0)
      asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else if constexpr (AF == 1 && BF == 0)
      asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1" : "+a"(c) : "v"(a), "v"(b));
    else if constexpr (AF == 0 && BF == 1)
      asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 blgp:1" : "+a"(c) : "v"(a), "v"(b));
    else
      asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(c) : "v"(a), "v"(b));
#endif
  };
  auto group8 = [&](auto U, auto TT, int s) {
    constexpr int u = decltype(U)::value, t = decltype(TT)::value;
    constexpr int pr = u & 1;                     // R register set of stage s
    constexpr int ts = u & 1;                     // T slot of stage s
    constexpr int rs = u % 3, rs1 = (u + 1) % 3;  // R slots of stages s, s + 1
    constexpr int k0 = t < 2 ? 0 : t < 6 ? 3 * (t - 2) : 12 + 2 * (t - 6);
    constexpr int nld = t < 2 ? 0 : t < 6 ? 3 : 2;
    auto mf = [&](auto QQ) {
      constexpr int q = decltype(QQ)::value, r = q & 7, h = q >> 3;
      if constexpr (MX) {
        if constexpr (RA)
          mfma16s(ic<r & 3>{}, ic<t & 3>{}, acc[r][t], Rf[pr][r][h], Tf[t & 1][h], Rsc[pr][h][r >> 2],
                  Tsc[u & 1][h][t >> 2]);
        else
          mfma16s(ic<t & 3>{}, ic<r & 3>{}, acc[t][r], Tf[t & 1][h], Rf[pr][r][h], Tsc[u & 1][h][t >> 2],
                  Rsc[pr][h][r >> 2]);
      } else {
        if constexpr (RA) mfma16(acc[r][t], Rf[pr][r][0], Tf[t & 1][0]);
        else mfma16(acc[t][r], Tf[t & 1][0], Rf[pr][r][0]);
      }
    };
    // MFMA 0 (and 1: E2M1) with the next T fragment; MFMAs 1-2 (2-5: E2M1) with R of
    // stage s + 1 (groups 2-5); the loads after MFMAs 3 .. (6 ..: E2M1)
    constexpr int q_ld = MX4 ? 6 : 3;
    auto step = [&](auto QQ) {
      constexpr int q = decltype(QQ)::value;
      mf(QQ);
      if constexpr (q < KS) {
        if constexpr (t < 7) Tf[(t + 1) & 1][q] = rdT(ts, t + 1, q);
        else Tf[0][q] = rdT(ts ^ 1, 0, q);
      }
      if constexpr (t >= 2 && t <= 5) {
        if constexpr (q >= 1 && q < 1 + 2 * KS) {
          constexpr int i = q - 1, g = 2 * (t - 2) + i / KS, h = i % KS;
          Rf[pr ^ 1][g][h] = rdF(slotR(rs1), oR, g, h);
        }
      }
      if (q >= q_ld && q - q_ld < nld) load_k(k0 + q - q_ld, ts, rs, s);
      if constexpr (MX) {
        // scales: raw dwords of stage s + 2 in groups 0 (R) and 1 (T), those of stage s + 1
        // transposed into the packed set in groups 6 and 7
        if constexpr (t == 0) {
          if (q == 2) load_raw(rawR[u & 1], rsSR, scR, s + 2);
        }
        if constexpr (t == 1) {
          if (q == 2) load_raw(rawT[u & 1], rsST, scT, s + 2);
        }
        if constexpr (t == 6) {
          if (q == 6) xpose(Rsc[pr ^ 1], rawR[(u + 1) & 1]);
        }
        if constexpr (t == 7) {
          if (q == 6) xpose(Tsc[(u + 1) & 1], rawT[(u + 1) & 1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    step(ic<0>{});
    step(ic<1>{});
    step(ic<2>{});
    step(ic<3>{});
    step(ic<4>{});
    step(ic<5>{});
    step(ic<6>{});
    step(ic<7>{});
    if constexpr (KS == 2) {
      step(ic<8>{});
      step(ic<9>{});
      step(ic<10>{});
      step(ic<11>{});
      step(ic<12>{});
      step(ic<13>{});
      step(ic<14>{});
      step(ic<15>{});
    }
    if constexpr (t == 1) {
      // T groups 0-2 of stage s read by this wave; stage s + 1's R and T groups 0-2 and
      // stage s's T groups 3-7 landed (only the R loads of the last barrier in flight, and
      // MX: the four scale loads of this stage's first two groups, issued after them)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(MX ? 8 + 4 * KS : 8));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto iter = [&](auto U, int s) {
    group8(U, ic<0>{}, s);
    group8(U, ic<1>{}, s);
    group8(U, ic<2>{}, s);
    group8(U, ic<3>{}, s);
    group8(U, ic<4>{}, s);
    group8(U, ic<5>{}, s);
    group8(U, ic<6>{}, s);
    group8(U, ic<7>{}, s);
  };
  int s = 0;
  for (; s + 6 <= S; s += 6) {
    iter(ic<0>{}, s);
    iter(ic<1>{}, s + 1);
    iter(ic<2>{}, s + 2);
    iter(ic<3>{}, s + 3);
    iter(ic<4>{}, s + 4);
    iter(ic<5>{}, s + 5);
  }
  if (s < S) iter(ic<0>{}, s);
  if (s + 1 < S) iter(ic<1>{}, s + 1);
  if (s + 2 < S) iter(ic<2>{}, s + 2);
  if (s + 3 < S) iter(ic<3>{}, s + 3);
  if (s + 4 < S) iter(ic<4>{}, s + 4);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));  // loads past the last stage still write LDS
  __builtin_amdgcn_s_barrier();
  // the MFMAs are written as instructions, so the compiler does not count the wait states
  // between the last one and the first read of its accumulators: 32 here, more than the
  // instruction needs
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7");
  asm volatile("s_nop 7");
  asm volatile("s_nop 7");
  asm volatile("s_nop 7");
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue: scale, bias, round; staged through LDS, 64 x 64 floats per pass ----
  // a 16 x 16 tile's lane holds column l & 15 and rows 4 (l >> 4) .. + 3; staged rows
  // are 68 floats apart, so the four lane groups' rows land on different banks
  constexpr int kEp = 68;
  float* ep = reinterpret_cast<float*>(wave == 0 ? sR0 : wave == 1 ? sR1 : wave == 2 ? sR2 : sT0b);
  // the bias of this lane's eight columns, fetched together (one memory latency)
  float bias8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  if (p.bias != nullptr) {
    // columns past n read column n - 1 (every load issued unconditionally) and take 0
    uint32_t raw[8];
    if (p.bias_bf16) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int col = min(n0 + wn + q * 16 + l16, p.N - 1);
        raw[q] = static_cast<uint32_t>(static_cast<const uint16_t*>(p.bias)[col]) << 16;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int col = min(n0 + wn + q * 16 + l16, p.N - 1);
        raw[q] = static_cast<const uint32_t*>(p.bias)[col];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) bias8[q] = n0 + wn + q * 16 + l16 < p.N ? __uint_as_float(raw[q]) : 0.0f;
  }
  // the bias add is decided once per launch, not per element
  auto epilogue = [&](auto HB) {
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              float val = acc[4 * pr + ii][4 * pc + jj][v];
              if constexpr (!MX) val = __fmul_rn(__fmul_rn(val, sa), sb);
              if constexpr (decltype(HB)::value != 0) val = __fadd_rn(val, bias8[4 * pc + jj]);
              ep[(16 * ii + 4 * lq + v) * kEp + 16 * jj + l16] = val;
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
        __builtin_amdgcn_wave_barrier();
        const int row0 = m0 + wm + pr * 64;
        const int col0 = n0 + wn + pc * 64;
        if (p.d_bf16) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int r = t * 8 + (lane >> 3);
            const int c = (lane & 7) * 8;
            const float4 lo = *reinterpret_cast<const float4*>(ep + r * kEp + c);
            const float4 hi = *reinterpret_cast<const float4*>(ep + r * kEp + c + 4);
            const int grow = row0 + r, gcol = col0 + c;
            if (grow < p.M && gcol < p.N) {
              const v4u o = {bf16x2_rne(lo.x, lo.y), bf16x2_rne(lo.z, lo.w), bf16x2_rne(hi.x, hi.y),
                             bf16x2_rne(hi.z, hi.w)};
              __builtin_nontemporal_store(
                  o, reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.d) + static_cast<int64_t>(grow) * p.N + gcol));
            }
          }
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const int r = t * 4 + (lane >> 4);
            const int c = (lane & 15) * 4;
            v4f v4 = *reinterpret_cast<const v4f*>(ep + r * kEp + c);
            const int grow = row0 + r, gcol = col0 + c;
            if (grow < p.M && gcol < p.N) {
              v4f* dst = reinterpret_cast<v4f*>(static_cast<float*>(p.d) + static_cast<int64_t>(grow) * p.N + gcol);
              if (p.accumulate) {
                const v4f old = __builtin_nontemporal_load(dst);
#pragma unroll
                for (int q = 0; q < 4; ++q) v4[q] = __fadd_rn(old[q], v4[q]);
              }
              __builtin_nontemporal_store(v4, dst);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
        __builtin_amdgcn_wave_barrier();
      }
    }
  };
  if (p.bias != nullptr) epilogue(ic<1>{});
  else epilogue(ic<0>{});
}

template <int KIND, int AF, int BF, bool PANEL = false, bool FUSED = false>
hipError_t run(Params p, hipStream_t s, const char* name) {
  g_last_variant = name;
  const int nb = p.nbm * p.nbn;
  if (p.splits > 1) {
    // split-K (per-tensor FP8 and BF16 only): partial sums of every split into the
    // workspace, then the reduction with the epilogue
    g_last_variant = splitk_name(name);
    Params q = p;
    q.d = q.partial_ws;
    q.d_bf16 = 0;
    q.accumulate = 0;
    q.bias = nullptr;
    q.partial = 1;
    hipLaunchKernelGGL((k_gemm4<KIND, AF, BF>), dim3(nb * p.splits), dim3(NT8), 0, s, q);
    const int64_t mn = static_cast<int64_t>(p.M) * p.N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3(static_cast<unsigned>((mn / 4 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(p.partial_ws), p.splits, mn, p.N,
                       static_cast<const float*>(p.a_scale), static_cast<const float*>(p.b_scale),
                       KIND == KIND_FP8 ? 1 : 0, p.bias, p.bias_bf16, p.d, p.d_bf16);
    return hipGetLastError();
  }
  if (KIND == KIND_MX && !PANEL && (p.kblocks & 3) != 0) {
    // a k that is not a multiple of 128 leaves a partial scale dword per stage: the
    // two-stage kernel fills it per byte
    g_last_variant = "gemm_mx_256x256_twostage";
    hipLaunchKernelGGL((k_gemm<KIND_MX, AF, BF>), dim3(nb), dim3(NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_gemm4<KIND, AF, BF, PANEL, FUSED>), dim3(nb), dim3(NT8), 0, s, p);
  }
  return hipGetLastError();
}

// the one-wave kernel: per-tensor FP8 (k % 128 == 0) or MXFP8 / MXFP4 with panel
// scales, one k split, bf16 / fp32 output (with accumulation); the operand with more
// rows gets the deeper stage ring
template <int KIND, int AF, int BF>
hipError_t run_1w(Params p, hipStream_t s, const char* name_a, const char* name_b) {
  static_assert(KIND == KIND_FP8 || KIND == KIND_MX || KIND == KIND_MX4, "FP8, MXFP8 or MXFP4");
  const int nb = p.nbm * p.nbn;
  if (p.M >= p.N) {
    g_last_variant = name_a;
    hipLaunchKernelGGL((k_gemm1x<KIND, AF, BF, 1>), dim3(nb), dim3(256), 0, s, p);
  } else {
    g_last_variant = name_b;
    hipLaunchKernelGGL((k_gemm1x<KIND, AF, BF, 2>), dim3(nb), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

// empty output with the fused epilogue: amax = 0, and the FP8 output's scale_inv
__global__ void k_gemm_amax_empty(float* amax, const float* d_scale, float* d_scale_inv) {
  *amax = 0.0f;
  if (d_scale != nullptr) *d_scale_inv = 1.0f / *d_scale;
}

}  // namespace

const char* last_gemm_variant() { return g_last_variant; }

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.m == 0 || g.n == 0) {
    if (g.amax != nullptr) {
      hipLaunchKernelGGL(k_gemm_amax_empty, dim3(1), dim3(1), 0, s, g.amax, g.d_fp8 ? g.d_scale : nullptr,
                         g.d_scale_inv);
      return hipGetLastError();
    }
    return hipSuccess;
  }
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
  p.KB = static_cast<int>(g.a_fmt == E2M1 ? g.k / 2 : g.k * esz);
  p.KT = (p.KB + BKB - 1) / BKB;
  p.kblocks = static_cast<int>(g.k / 32);
  p.nbm = static_cast<int>((g.m + BM - 1) / BM);
  p.nbn = static_cast<int>((g.n + BN - 1) / BN);
  p.bias_bf16 = g.bias_bf16;
  p.d_bf16 = g.d_bf16;
  p.accumulate = g.accumulate;
  p.splits = g.splits > 1 ? g.splits : 1;
  p.partial = 0;
  p.partial_ws = static_cast<float*>(g.workspace);
  p.amax = g.amax;
  p.amax_ws = g.amax_ws;
  p.d_scale = g.d_scale;
  p.d_scale_inv = g.d_scale_inv;
  p.d_fp8 = g.d_fp8;
  // f8f6f4 format codes: 0 = E4M3, 1 = E5M2
  const int af = (g.a_fmt == E5M2) ? 1 : 0, bf = (g.b_fmt == E5M2) ? 1 : 0;
  if (g.amax != nullptr) {  // fused amax epilogue (per-tensor FP8 and BF16, no split-K; checked by the caller)
    if (g.a_fmt == BF16) return run<KIND_BF16, 0, 0, false, true>(p, s, "gemm4_bf16_256x256_pingpong_amax");
    if (af == 0 && bf == 0) return run<KIND_FP8, 0, 0, false, true>(p, s, "gemm4_fp8_e4m3_e4m3_256x256_pingpong_amax");
    if (af == 1 && bf == 0) return run<KIND_FP8, 1, 0, false, true>(p, s, "gemm4_fp8_e5m2_e4m3_256x256_pingpong_amax");
    if (af == 0 && bf == 1) return run<KIND_FP8, 0, 1, false, true>(p, s, "gemm4_fp8_e4m3_e5m2_256x256_pingpong_amax");
    return run<KIND_FP8, 1, 1, false, true>(p, s, "gemm4_fp8_e5m2_e5m2_256x256_pingpong_amax");
  }
  if (g.a_fmt == BF16) return run<KIND_BF16, 0, 0>(p, s, "gemm4_bf16_256x256_pingpong");
  if (g.a_fmt != E2M1 && p.splits == 1 && ((g.mx && g.mx_panel) || (!g.mx && p.KB % PK == 0))) {
    if (g.mx) {
      if (af == 0 && bf == 0)
        return run_1w<KIND_MX, 0, 0>(p, s, "gemm1w_mx_e4m3_e4m3_256x256_panel_mfma16_deepA",
                                      "gemm1w_mx_e4m3_e4m3_256x256_panel_mfma16_deepB");
      if (af == 1 && bf == 0)
        return run_1w<KIND_MX, 1, 0>(p, s, "gemm1w_mx_e5m2_e4m3_256x256_panel_mfma16_deepA",
                                      "gemm1w_mx_e5m2_e4m3_256x256_panel_mfma16_deepB");
      if (af == 0 && bf == 1)
        return run_1w<KIND_MX, 0, 1>(p, s, "gemm1w_mx_e4m3_e5m2_256x256_panel_mfma16_deepA",
                                      "gemm1w_mx_e4m3_e5m2_256x256_panel_mfma16_deepB");
      return run_1w<KIND_MX, 1, 1>(p, s, "gemm1w_mx_e5m2_e5m2_256x256_panel_mfma16_deepA",
                                      "gemm1w_mx_e5m2_e5m2_256x256_panel_mfma16_deepB");
    }
    if (af == 0 && bf == 0)
      return run_1w<KIND_FP8, 0, 0>(p, s, "gemm1w_fp8_e4m3_e4m3_256x256_mfma16_deepA",
                                       "gemm1w_fp8_e4m3_e4m3_256x256_mfma16_deepB");
    if (af == 1 && bf == 0)
      return run_1w<KIND_FP8, 1, 0>(p, s, "gemm1w_fp8_e5m2_e4m3_256x256_mfma16_deepA",
                                       "gemm1w_fp8_e5m2_e4m3_256x256_mfma16_deepB");
    if (af == 0 && bf == 1)
      return run_1w<KIND_FP8, 0, 1>(p, s, "gemm1w_fp8_e4m3_e5m2_256x256_mfma16_deepA",
                                       "gemm1w_fp8_e4m3_e5m2_256x256_mfma16_deepB");
    return run_1w<KIND_FP8, 1, 1>(p, s, "gemm1w_fp8_e5m2_e5m2_256x256_mfma16_deepA",
                                       "gemm1w_fp8_e5m2_e5m2_256x256_mfma16_deepB");
  }
  if (g.a_fmt == E2M1) {
    if (g.mx_panel)
      return run_1w<KIND_MX4, 4, 4>(p, s, "gemm1w_mxfp4_e2m1_e2m1_256x256_panel_mfma16_deepA",
                                    "gemm1w_mxfp4_e2m1_e2m1_256x256_panel_mfma16_deepB");
    return run<KIND_MX4, 4, 4>(p, s, "gemm4_mxfp4_e2m1_e2m1_256x256_pingpong");
  }
  if (g.mx && g.mx_panel) {
    if (af == 0 && bf == 0) return run<KIND_MX, 0, 0, true>(p, s, "gemm4_mx_e4m3_e4m3_256x256_pingpong_panel");
    if (af == 1 && bf == 0) return run<KIND_MX, 1, 0, true>(p, s, "gemm4_mx_e5m2_e4m3_256x256_pingpong_panel");
    if (af == 0 && bf == 1) return run<KIND_MX, 0, 1, true>(p, s, "gemm4_mx_e4m3_e5m2_256x256_pingpong_panel");
    return run<KIND_MX, 1, 1, true>(p, s, "gemm4_mx_e5m2_e5m2_256x256_pingpong_panel");
  }
  if (g.mx) {
    if (af == 0 && bf == 0) return run<KIND_MX, 0, 0>(p, s, "gemm4_mx_e4m3_e4m3_256x256_pingpong");
    if (af == 1 && bf == 0) return run<KIND_MX, 1, 0>(p, s, "gemm4_mx_e5m2_e4m3_256x256_pingpong");
    if (af == 0 && bf == 1) return run<KIND_MX, 0, 1>(p, s, "gemm4_mx_e4m3_e5m2_256x256_pingpong");
    return run<KIND_MX, 1, 1>(p, s, "gemm4_mx_e5m2_e5m2_256x256_pingpong");
  }
  if (af == 0 && bf == 0) return run<KIND_FP8, 0, 0>(p, s, "gemm4_fp8_e4m3_e4m3_256x256_pingpong");
  if (af == 1 && bf == 0) return run<KIND_FP8, 1, 0>(p, s, "gemm4_fp8_e5m2_e4m3_256x256_pingpong");
  if (af == 0 && bf == 1) return run<KIND_FP8, 0, 1>(p, s, "gemm4_fp8_e4m3_e5m2_256x256_pingpong");
  return run<KIND_FP8, 1, 1>(p, s, "gemm4_fp8_e5m2_e5m2_256x256_pingpong");
}

}  // namespace te
