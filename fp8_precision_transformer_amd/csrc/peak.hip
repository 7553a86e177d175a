// Measurement probes, built into libte_peak.so and driven by microbench.py:
//  - k_peak: MFMA-only throughput with register operands, no memory traffic in the
//    loop: the sustained FP8 (32x32x64 f8f6f4), BF16 (32x32x16), MXFP8 and MXFP4
//    (block-scaled 32x32x64 with the scales in registers) matrix-core rates under the
//    clocks the device actually runs, as a ceiling beside the published peak;
//  - k_peak_rand: the FP8 rate when the operands change from one instruction to the
//    next, as in a GEMM (eight register sets of random E4M3 codes), for the 32x32x64 and
//    the 16x16x128 instruction: the chip holds lower clocks under that load, and the two
//    shapes do not slow down alike;
//  - k_copy: a plain 16-byte-per-lane device copy of known size, the reference that
//    HBM byte counters (FETCH_SIZE, WRITE_SIZE) are calibrated against, and the
//    practical streaming rate (read + write) a memory-bound kernel can reach;
//  - k_read: a read-only stream (xor-reduce of every 16-byte word), the practical
//    read rate;
//  - k_stream: the streaming ceiling study: copy (read 1 : write 1), cast-shaped
//    (16 bytes read, 8 written per lane and chunk: the bf16 -> FP8 byte ratio),
//    read-only and write-only streams, with U chunks per lane in flight, cached or
//    nontemporal loads (NTL) and stores (NTS), over grid sizes chosen by the caller.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// KIND 0: FP8 (the scaled instruction with constant zero scales, which the compiler emits
// as the plain v_mfma_f32_32x32x64_f8f6f4), 1: BF16, 2: MXFP8 (v_mfma_scale with E8M0
// scales in registers), 3: MXFP4 (E2M1 operands, scales in registers)
template <int KIND>
__global__ __launch_bounds__(256, 1) void k_peak(const int* seed, float* out, int iters) {
  constexpr bool BF16 = KIND == 1;
  const int t = threadIdx.x + seed[0];
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (t * 131 + i * 7) & 0x3f3f3f3f;
    b[i] = (t * 17 + i * 3) & 0x3f3f3f3f;
  }
  const int sc = 0x7f7f7f7f ^ (seed[0] & 1);  // E8M0 unit scales, not known at compile time
  v16f acc[16];
  for (int i = 0; i < 16; ++i) acc[i] = v16f{0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (BF16) {
        const v8bf av = __builtin_bit_cast(v8bf, __builtin_shufflevector(a, a, 0, 1, 2, 3));
        const v8bf bv = __builtin_bit_cast(v8bf, __builtin_shufflevector(b, b, 0, 1, 2, 3));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
      } else if constexpr (KIND == 2) {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, sc, 1, sc);
      } else if constexpr (KIND == 3) {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 4, 4, 0, sc, 1, sc);
      } else {
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 0, 0, 0);
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i)
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ inline uint32_t mix32(uint32_t x) {  // an integer hash, for operand codes only
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// SHAPE 0: 32x32x64 (16 accumulators of 16), 1: 16x16x128 (64 accumulators of 4); one
// wave per SIMD, 256 accumulator registers either way; every instruction takes one of 8
// random A sets against a B set that rotates with it; codes without NaN (bit 3 clear)
template <int SHAPE>
__global__ __launch_bounds__(256, 1) void k_peak_rand(const int* seed, float* out, int iters) {
  const uint32_t t = threadIdx.x + 256u * blockIdx.x + static_cast<uint32_t>(seed[0]);
  v8i A[8], B[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      A[s][j] = static_cast<int>(mix32(t * 64u + s * 8u + j + 1u) & 0xF7F7F7F7u);
      B[s][j] = static_cast<int>(mix32(t * 64u + s * 8u + j + 0x9e3779b9u) & 0xF7F7F7F7u);
    }
  float r = 0.0f;
  if constexpr (SHAPE == 0) {
    v16f acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v16f{0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[s], B[(s + i) & 7], acc[i], 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) r += acc[i][j];
  } else {
    v4f acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          acc[(s & 1) * 32 + i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              A[s], B[(s + i) & 7], acc[(s & 1) * 32 + i], 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) r += acc[i][j];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// kind: 0 FP8, 1 BF16, 2 MXFP8, 3 MXFP4 (see k_peak); 4 FP8 32x32x64 and 5 FP8 16x16x128
// with changing random operands (k_peak_rand; 8 x 16 and 8 x 32 instructions per
// iteration, the same FLOP)
extern "C" int te_peak_launch(int kind, int blocks, int iters, const int* seed, float* out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (kind) {
    case 0: hipLaunchKernelGGL((k_peak<0>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 1: hipLaunchKernelGGL((k_peak<1>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 2: hipLaunchKernelGGL((k_peak<2>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 3: hipLaunchKernelGGL((k_peak<3>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 4: hipLaunchKernelGGL((k_peak_rand<0>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    case 5: hipLaunchKernelGGL((k_peak_rand<1>), dim3(blocks), dim3(256), 0, st, seed, out, iters); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// grid-stride copy of n16 16-byte words
__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ src, uint32_t* __restrict__ out, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keeps the loads live; out[0] is written only when the fold hits this value
  if (acc == 0x9e3779b9u) out[0] = acc;
}

// grid <= 0 picks min(ceil(n16 / 256), 4096) blocks.
extern "C" int te_copy_launch(const void* src, void* dst, int64_t n16, int grid, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  int64_t g = grid > 0 ? grid : (n16 + 255) / 256;
  if (grid <= 0 && g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_copy, dim3(static_cast<unsigned>(g)), dim3(256), 0, st, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int te_read_launch(const void* src, void* out4, int64_t n16, int grid, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  int64_t g = grid > 0 ? grid : (n16 + 255) / 256;
  if (grid <= 0 && g > 4096) g = 4096;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(k_read, dim3(static_cast<unsigned>(g)), dim3(256), 0, st, static_cast<const uint4*>(src),
                     static_cast<uint32_t*>(out4), n16);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// KIND 0: copy, 1: cast-shaped (8 output bytes per 16 input bytes), 2: read-only,
// 3: write-only.  Lane chunk u of an iteration is 16-byte word base + u * stride, so
// every load and store instruction covers a contiguous 4 KB per block.
template <int KIND, int U, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void k_stream(const v4u* __restrict__ src, void* __restrict__ dst, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; base < n16; base += stride * U) {
    v4u v[U];
    if constexpr (KIND != 3) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * stride;
        if (i < n16) v[u] = NTL ? __builtin_nontemporal_load(src + i) : src[i];
        else v[u] = v4u{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + u * stride;
      if (i >= n16) continue;
      if constexpr (KIND == 0) {
        if (NTS) __builtin_nontemporal_store(v[u], static_cast<v4u*>(dst) + i);
        else static_cast<v4u*>(dst)[i] = v[u];
      } else if constexpr (KIND == 1) {
        const v2u o = {__builtin_amdgcn_perm(v[u].y, v[u].x, 0x07050301u),
                       __builtin_amdgcn_perm(v[u].w, v[u].z, 0x07050301u)};
        if (NTS) __builtin_nontemporal_store(o, static_cast<v2u*>(dst) + i);
        else static_cast<v2u*>(dst)[i] = o;
      } else if constexpr (KIND == 2) {
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      } else {
        const v4u o = {static_cast<uint32_t>(i), 1u, 2u, 3u};
        if (NTS) __builtin_nontemporal_store(o, static_cast<v4u*>(dst) + i);
        else static_cast<v4u*>(dst)[i] = o;
      }
    }
  }
  if constexpr (KIND == 2) {
    if (acc == 0x9e3779b9u) static_cast<uint32_t*>(dst)[0] = acc;
  }
}

template <int KIND, int U>
static void stream_launch(int nt, const void* src, void* dst, int64_t n16, int grid, hipStream_t st) {
  const auto* s4 = static_cast<const v4u*>(src);
  switch (nt & 3) {
    case 0: hipLaunchKernelGGL((k_stream<KIND, U, false, false>), dim3(grid), dim3(256), 0, st, s4, dst, n16); break;
    case 1: hipLaunchKernelGGL((k_stream<KIND, U, true, false>), dim3(grid), dim3(256), 0, st, s4, dst, n16); break;
    case 2: hipLaunchKernelGGL((k_stream<KIND, U, false, true>), dim3(grid), dim3(256), 0, st, s4, dst, n16); break;
    default: hipLaunchKernelGGL((k_stream<KIND, U, true, true>), dim3(grid), dim3(256), 0, st, s4, dst, n16); break;
  }
}

template <int KIND>
static int stream_u(int u, int nt, const void* src, void* dst, int64_t n16, int grid, hipStream_t st) {
  switch (u) {
    case 1: stream_launch<KIND, 1>(nt, src, dst, n16, grid, st); break;
    case 2: stream_launch<KIND, 2>(nt, src, dst, n16, grid, st); break;
    case 4: stream_launch<KIND, 4>(nt, src, dst, n16, grid, st); break;
    case 8: stream_launch<KIND, 8>(nt, src, dst, n16, grid, st); break;
    default: return 1;
  }
  return 0;
}

// kind 0..3 as k_stream; u in {1, 2, 4, 8}; nt: bit 0 nontemporal loads, bit 1
// nontemporal stores; grid >= 1 blocks of 256 lanes.  dst holds
// n16 16-byte words (copy, write-only), n16 8-byte words (cast-shaped) or 4 bytes
// (read-only).
extern "C" int te_stream_launch(int kind, int u, int nt, const void* src, void* dst, int64_t n16, int grid,
                                void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid < 1) return 1;
  int bad = 1;
  switch (kind) {
    case 0: bad = stream_u<0>(u, nt, src, dst, n16, grid, st); break;
    case 1: bad = stream_u<1>(u, nt, src, dst, n16, grid, st); break;
    case 2: bad = stream_u<2>(u, nt, src, dst, n16, grid, st); break;
    case 3: bad = stream_u<3>(u, nt, src, dst, n16, grid, st); break;
    default: return 1;
  }
  return bad || hipGetLastError() != hipSuccess ? 1 : 0;
}
