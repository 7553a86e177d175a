// Quantizer kernels for gfx950: amax + scaled FP8 cast, fused cast + transpose,
// delayed-scaling update, MXFP8 block quantization.
//
// Pages: [FP8-intro] = "Introduction to FP8 training using Transformer Engine"
// (NVIDIA blog, Japanese edition); [LP-opt] = "How to Optimize Transformer-Based
// Models for Low-Precision Training" (NVIDIA blog, Japanese translation);
// [TE-summary] = "NVIDIA Transformer Engine - 大規模Transformer向け高速低精度学習".
//
// All of these are HBM-bound streaming kernels: each element is read once (twice
// for current scaling, whose amax must exist before the first cast) and written
// once per output layout.  Loads and stores are 16 bytes per lane.

#include "device_common.hpp"
#include "internal.hpp"

namespace te {
namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------------------
// element loads
// ----------------------------------------------------------------------------
template <typename T>
struct In;

template <>
struct In<uint16_t> {  // bf16 bits
  static __device__ __forceinline__ void load16(const uint16_t* p, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
};

template <>
struct In<float> {
  static __device__ __forceinline__ void load16(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = a.x;
      v[4 * i + 1] = a.y;
      v[4 * i + 2] = a.z;
      v[4 * i + 3] = a.w;
    }
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
};

// ----------------------------------------------------------------------------
// prologue: zero amax; for delayed scaling also publish scale_inv = 1/scale
// ----------------------------------------------------------------------------
__global__ void k_prologue(float* amax, const float* scale, float* scale_inv, int delayed) {
  *amax = 0.0f;
  if (delayed) *scale_inv = 1.0f / *scale;
}

// Finalize current scaling without a cast: scale and scale_inv from amax.
__global__ void k_current_scale(const float* amax, float* scale, float* scale_inv, float fp8_max,
                                int margin) {
  const float s = scale_from_amax(*amax, fp8_max, margin, 1.0f);
  *scale = s;
  *scale_inv = 1.0f / s;
}

// ----------------------------------------------------------------------------
// flat amax / cast.  MODE 0: amax + cast with *scale (delayed).  MODE 1: amax
// only.  MODE 2: cast with the current scale derived from *amax (block 0 also
// publishes scale and scale_inv).
// ----------------------------------------------------------------------------
template <typename T, bool E5M2, int MODE>
__global__ __launch_bounds__(kThreads) void k_amax_cast(const T* __restrict__ x, int64_t n,
                                                        float* __restrict__ scale,
                                                        float* __restrict__ scale_inv,
                                                        float* __restrict__ amax,
                                                        uint8_t* __restrict__ out, int margin) {
  constexpr bool kAmax = MODE != 2;
  constexpr bool kCast = MODE != 1;
  float s = 1.0f;
  if constexpr (MODE == 0) s = *scale;
  if constexpr (MODE == 2) {
    s = scale_from_amax(*amax, Fp8Traits<E5M2>::max, margin, 1.0f);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *scale = s;
      *scale_inv = 1.0f / s;
    }
  }
  float m = 0.0f;
  const int64_t nv = n >> 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < nv; i += stride) {
    float v[16];
    In<T>::load16(x + i * 16, v);
    if constexpr (kAmax) {
#pragma unroll
      for (int j = 0; j < 16; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
    }
    if constexpr (kCast) {
      uint4 q;
      q.x = quant4<E5M2>(v[0], v[1], v[2], v[3], s);
      q.y = quant4<E5M2>(v[4], v[5], v[6], v[7], s);
      q.z = quant4<E5M2>(v[8], v[9], v[10], v[11], s);
      q.w = quant4<E5M2>(v[12], v[13], v[14], v[15], s);
      *reinterpret_cast<uint4*>(out + i * 16) = q;
    }
  }
  if (blockIdx.x == 0) {  // tail of fewer than 16 elements
    const int64_t t = nv * 16 + threadIdx.x;
    if (t < n) {
      const float v = In<T>::load1(x + t);
      if constexpr (kAmax) m = __builtin_fmaxf(m, __builtin_fabsf(v));
      if constexpr (kCast) out[t] = static_cast<uint8_t>(quant4<E5M2>(v, 0.f, 0.f, 0.f, s) & 0xffu);
    }
  }
  if constexpr (kAmax) block_amax_atomic(m, amax);
}

// ----------------------------------------------------------------------------
// cast + transpose over 128 x 64 tiles.  MODE 0: amax + cast with *scale.
// MODE 2: cast with the current scale from *amax.  The FP8 bytes of the tile go
// through LDS; each wave then gathers 32 rows of 64 columns and writes them as
// 32-byte runs of out_col.
// ----------------------------------------------------------------------------
constexpr int kTR = 128, kTC = 64, kPitch = kTC + 4;

template <typename T>
__device__ __forceinline__ bool rows_vec_ok(int64_t cols) {
  return (cols % (16 / sizeof(T))) == 0;  // every row starts 16-byte aligned
}

template <typename T, bool E5M2, int MODE>
__global__ __launch_bounds__(kThreads) void k_cast_transpose(
    const T* __restrict__ x, int64_t R, int64_t C, float* __restrict__ scale,
    float* __restrict__ scale_inv, float* __restrict__ amax, uint8_t* __restrict__ out_row,
    uint8_t* __restrict__ out_col, int margin) {
  __shared__ uint32_t tile[kTR * kPitch / 4];
  uint8_t* tb = reinterpret_cast<uint8_t*>(tile);

  float s = 1.0f;
  if constexpr (MODE == 0) s = *scale;
  if constexpr (MODE == 2) {
    s = scale_from_amax(*amax, Fp8Traits<E5M2>::max, margin, 1.0f);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      *scale = s;
      *scale_inv = 1.0f / s;
    }
  }
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTR;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTC;
  const int t = threadIdx.x;
  const int lr = t >> 1, lc = (t & 1) * 32;
  const int64_t r = r0 + lr;
  const bool full = (r0 + kTR <= R) && (c0 + kTC <= C);

  float v[32];
  if (full && rows_vec_ok<T>(C)) {
    const T* p = x + r * C + c0 + lc;
    In<T>::load16(p, v);
    In<T>::load16(p + 16, v + 16);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int64_t c = c0 + lc + j;
      v[j] = (r < R && c < C) ? In<T>::load1(x + r * C + c) : 0.0f;
    }
  }
  float m = 0.0f;
  if constexpr (MODE == 0) {
#pragma unroll
    for (int j = 0; j < 32; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
  }
  uint32_t q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = quant4<E5M2>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], s);

  if (out_row != nullptr) {
    if (full && (C % 16) == 0) {
      uint4* o = reinterpret_cast<uint4*>(out_row + r * C + c0 + lc);
      o[0] = make_uint4(q[0], q[1], q[2], q[3]);
      o[1] = make_uint4(q[4], q[5], q[6], q[7]);
    } else if (r < R) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int64_t c = c0 + lc + j;
        if (c < C) out_row[r * C + c] = static_cast<uint8_t>(q[j >> 2] >> (8 * (j & 3)));
      }
    }
  }
  if (out_col != nullptr) {
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[(lr * kPitch + lc) / 4 + j] = q[j];
    __syncthreads();
    const int oc = t & 63, seg = t >> 6;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int rr = seg * 32 + 4 * j;
      w[j] = static_cast<uint32_t>(tb[(rr + 0) * kPitch + oc]) |
             (static_cast<uint32_t>(tb[(rr + 1) * kPitch + oc]) << 8) |
             (static_cast<uint32_t>(tb[(rr + 2) * kPitch + oc]) << 16) |
             (static_cast<uint32_t>(tb[(rr + 3) * kPitch + oc]) << 24);
    }
    const int64_t c = c0 + oc;
    const int64_t rb = r0 + seg * 32;
    if (c < C) {
      if (full && (R % 16) == 0) {
        uint4* o = reinterpret_cast<uint4*>(out_col + c * R + rb);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (rb + j < R) out_col[c * R + rb + j] = static_cast<uint8_t>(w[j >> 2] >> (8 * (j & 3)));
      }
    }
  }
  if constexpr (MODE == 0) block_amax_atomic(m, amax);
}

// ----------------------------------------------------------------------------
// delayed-scaling update, one thread per tensor
// ----------------------------------------------------------------------------
__global__ void k_scale_update(float* __restrict__ hist, float* __restrict__ scale,
                               float* __restrict__ scale_inv, int n, int L, float fp8_max,
                               int most_recent, int margin) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  float* h = hist + static_cast<int64_t>(t) * L;
  float a = h[0];
  if (!most_recent) {
    for (int i = 1; i < L; ++i) {
      const float hi = h[i];
      a = (hi > a || hi != hi) ? hi : a;  // NaN propagates, as a plain max does
      if (a != a) break;
    }
  }
  const float s = scale_from_amax(a, fp8_max, margin, scale[t]);
  scale[t] = s;
  scale_inv[t] = 1.0f / s;
  for (int i = L - 1; i >= 1; --i) h[i] = h[i - 1];
  h[0] = 0.0f;
}

// ----------------------------------------------------------------------------
// MXFP8: 128 x 64 tiles.  Row-wise: each thread owns one 32-element block of a
// row.  Column-wise: the tile goes through LDS as fp32; each thread owns one
// 32-row block of one column.
// ----------------------------------------------------------------------------
template <bool E5M2>
__device__ __forceinline__ int mx_exponent(float am) {
  if (!(am > 0.0f)) return 0;  // all-zero block -> 2^0 (code 127)
  const uint32_t u = __float_as_uint(am);
  const int E = static_cast<int>((u >> 23) & 0xffu);
  const int fl = E ? E - 127 : (31 - __clz(static_cast<int>(u & 0x7fffffu))) - 149;
  int e = fl - Fp8Traits<E5M2>::emax_elem;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

template <bool E5M2>
__device__ __forceinline__ void mx_block32(const float* v, uint32_t* q, uint8_t* code) {
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am = __builtin_fmaxf(am, __builtin_fabsf(v[j]));
  const int e = mx_exponent<E5M2>(am);
  *code = static_cast<uint8_t>(e + 127);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    q[j] = cvt4<E5M2>(saturate<E5M2>(__builtin_ldexpf(v[4 * j], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 1], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 2], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 3], -e)));
}

constexpr int kMxPitch = kTC + 1;  // floats

template <typename T, bool E5M2>
__global__ __launch_bounds__(kThreads) void k_mxfp8(const T* __restrict__ x, int64_t R, int64_t C,
                                                    uint8_t* __restrict__ out_row,
                                                    uint8_t* __restrict__ scale_row,
                                                    uint8_t* __restrict__ out_col,
                                                    uint8_t* __restrict__ scale_col) {
  __shared__ float tile[kTR * kMxPitch];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTR;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTC;
  const int t = threadIdx.x;
  const int lr = t >> 1, lc = (t & 1) * 32;
  const int64_t r = r0 + lr;
  const bool full = (r0 + kTR <= R) && (c0 + kTC <= C);

  float v[32];
  if (full && rows_vec_ok<T>(C)) {
    const T* p = x + r * C + c0 + lc;
    In<T>::load16(p, v);
    In<T>::load16(p + 16, v + 16);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int64_t c = c0 + lc + j;
      v[j] = (r < R && c < C) ? In<T>::load1(x + r * C + c) : 0.0f;
    }
  }
  // row-wise copy: the block is inside the matrix iff its first column is (cols % 32 == 0)
  if (out_row != nullptr && r < R && c0 + lc < C) {
    uint32_t q[8];
    uint8_t code;
    mx_block32<E5M2>(v, q, &code);
    uint4* o = reinterpret_cast<uint4*>(out_row + r * C + c0 + lc);
    o[0] = make_uint4(q[0], q[1], q[2], q[3]);
    o[1] = make_uint4(q[4], q[5], q[6], q[7]);
    scale_row[r * (C / 32) + (c0 + lc) / 32] = code;
  }
  if (out_col != nullptr) {
#pragma unroll
    for (int j = 0; j < 32; ++j) tile[lr * kMxPitch + lc + j] = v[j];
    __syncthreads();
    const int oc = t & 63, seg = t >> 6;
    const int64_t c = c0 + oc;
    const int64_t rb = r0 + seg * 32;
    if (c < C && rb < R) {
      float w[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) w[j] = tile[(seg * 32 + j) * kMxPitch + oc];
      uint32_t q[8];
      uint8_t code;
      mx_block32<E5M2>(w, q, &code);
      if ((R % 16) == 0) {
        uint4* o = reinterpret_cast<uint4*>(out_col + c * R + rb);
        o[0] = make_uint4(q[0], q[1], q[2], q[3]);
        o[1] = make_uint4(q[4], q[5], q[6], q[7]);
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) out_col[c * R + rb + j] = static_cast<uint8_t>(q[j >> 2] >> (8 * (j & 3)));
      }
      scale_col[c * (R / 32) + rb / 32] = code;
    }
  }
}

int flat_grid(int64_t nv) {
  int64_t g = (nv + kThreads - 1) / kThreads;
  if (g < 1) g = 1;
  if (g > 2048) g = 2048;  // 8 resident blocks per CU on 256 CUs; grid-stride beyond that
  return static_cast<int>(g);
}

template <typename T, bool E5M2>
hipError_t amax_cast_t(const T* x, int64_t n, int current, int margin, float* scale,
                       float* scale_inv, float* amax, uint8_t* out, hipStream_t st) {
  const int g = flat_grid(n >> 4);
  hipLaunchKernelGGL(k_prologue, dim3(1), dim3(1), 0, st, amax, scale, scale_inv, current ? 0 : 1);
  if (!current) {
    if (out)
      hipLaunchKernelGGL((k_amax_cast<T, E5M2, 0>), dim3(g), dim3(kThreads), 0, st, x, n, scale,
                         scale_inv, amax, out, margin);
    else
      hipLaunchKernelGGL((k_amax_cast<T, E5M2, 1>), dim3(g), dim3(kThreads), 0, st, x, n, scale,
                         scale_inv, amax, out, margin);
  } else {
    hipLaunchKernelGGL((k_amax_cast<T, E5M2, 1>), dim3(g), dim3(kThreads), 0, st, x, n, scale,
                       scale_inv, amax, out, margin);
    if (out)
      hipLaunchKernelGGL((k_amax_cast<T, E5M2, 2>), dim3(g), dim3(kThreads), 0, st, x, n, scale,
                         scale_inv, amax, out, margin);
    else
      hipLaunchKernelGGL(k_current_scale, dim3(1), dim3(1), 0, st, amax, scale, scale_inv,
                         Fp8Traits<E5M2>::max, margin);
  }
  return hipGetLastError();
}

template <typename T, bool E5M2>
hipError_t cast_transpose_t(const T* x, int64_t R, int64_t C, int current, int margin,
                            float* scale, float* scale_inv, float* amax, uint8_t* out_row,
                            uint8_t* out_col, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((C + kTC - 1) / kTC), static_cast<unsigned>((R + kTR - 1) / kTR));
  hipLaunchKernelGGL(k_prologue, dim3(1), dim3(1), 0, st, amax, scale, scale_inv, current ? 0 : 1);
  if (R == 0 || C == 0) {
    if (current)
      hipLaunchKernelGGL(k_current_scale, dim3(1), dim3(1), 0, st, amax, scale, scale_inv,
                         Fp8Traits<E5M2>::max, margin);
    return hipGetLastError();
  }
  if (!current) {
    hipLaunchKernelGGL((k_cast_transpose<T, E5M2, 0>), grid, dim3(kThreads), 0, st, x, R, C, scale,
                       scale_inv, amax, out_row, out_col, margin);
  } else {
    const int g = flat_grid((R * C) >> 4);
    hipLaunchKernelGGL((k_amax_cast<T, E5M2, 1>), dim3(g), dim3(kThreads), 0, st, x, R * C, scale,
                       scale_inv, amax, nullptr, margin);
    hipLaunchKernelGGL((k_cast_transpose<T, E5M2, 2>), grid, dim3(kThreads), 0, st, x, R, C, scale,
                       scale_inv, amax, out_row, out_col, margin);
  }
  return hipGetLastError();
}

template <typename T, bool E5M2>
hipError_t mxfp8_t(const T* x, int64_t R, int64_t C, uint8_t* out_row, uint8_t* scale_row,
                   uint8_t* out_col, uint8_t* scale_col, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((C + kTC - 1) / kTC), static_cast<unsigned>((R + kTR - 1) / kTR));
  hipLaunchKernelGGL((k_mxfp8<T, E5M2>), grid, dim3(kThreads), 0, st, x, R, C, out_row, scale_row,
                     out_col, scale_col);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_amax_cast(const void* x, int x_dtype, int64_t n, int out_e5m2, int current,
                            int margin, float* scale, float* scale_inv, float* amax, uint8_t* out,
                            hipStream_t s) {
  if (x_dtype == BF16)
    return out_e5m2 ? amax_cast_t<uint16_t, true>(static_cast<const uint16_t*>(x), n, current, margin, scale, scale_inv, amax, out, s)
                    : amax_cast_t<uint16_t, false>(static_cast<const uint16_t*>(x), n, current, margin, scale, scale_inv, amax, out, s);
  return out_e5m2 ? amax_cast_t<float, true>(static_cast<const float*>(x), n, current, margin, scale, scale_inv, amax, out, s)
                  : amax_cast_t<float, false>(static_cast<const float*>(x), n, current, margin, scale, scale_inv, amax, out, s);
}

hipError_t launch_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 int out_e5m2, int current, int margin, float* scale,
                                 float* scale_inv, float* amax, uint8_t* out_row,
                                 uint8_t* out_col, hipStream_t s) {
  if (x_dtype == BF16)
    return out_e5m2 ? cast_transpose_t<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, current, margin, scale, scale_inv, amax, out_row, out_col, s)
                    : cast_transpose_t<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, current, margin, scale, scale_inv, amax, out_row, out_col, s);
  return out_e5m2 ? cast_transpose_t<float, true>(static_cast<const float*>(x), rows, cols, current, margin, scale, scale_inv, amax, out_row, out_col, s)
                  : cast_transpose_t<float, false>(static_cast<const float*>(x), rows, cols, current, margin, scale, scale_inv, amax, out_row, out_col, s);
}

hipError_t launch_scale_update(float* hist, float* scale, float* scale_inv, int n, int hist_len,
                               int e5m2, int most_recent, int margin, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int bs = 256;
  hipLaunchKernelGGL(k_scale_update, dim3((n + bs - 1) / bs), dim3(bs), 0, s, hist, scale, scale_inv,
                     n, hist_len, e5m2 ? kE5M2Max : kE4M3Max, most_recent, margin);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int e5m2,
                                 uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col,
                                 uint8_t* scale_col, hipStream_t s) {
  if (x_dtype == BF16)
    return e5m2 ? mxfp8_t<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s)
                : mxfp8_t<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s);
  return e5m2 ? mxfp8_t<float, true>(static_cast<const float*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s)
              : mxfp8_t<float, false>(static_cast<const float*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s);
}

}  // namespace te
