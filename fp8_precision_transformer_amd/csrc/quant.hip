// Quantizer kernels for gfx950: amax + scaled FP8 cast, fused cast + transpose (with
// the bias gradient of the tensor as an option), delayed-scaling update, MXFP8 and
// MXFP4 block quantization, LayerNorm written straight as FP8.
//
// Pages: [FP8-intro] = "Introduction to FP8 training using Transformer Engine"
// (NVIDIA blog, Japanese edition); [LP-opt] = "How to Optimize Transformer-Based
// Models for Low-Precision Training" (NVIDIA blog, Japanese translation);
// [TE-summary] = "NVIDIA Transformer Engine - 大規模Transformer向け高速低精度学習".
//
// All of these are HBM-bound streaming kernels: each element is read once (twice
// for current scaling, whose amax must exist before the first cast) and written
// once per output layout.  Loads and stores are 16 bytes per lane.

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "grid_amax.hpp"
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
// empty input: amax = 0; for delayed scaling also publish scale_inv = 1/scale
// ----------------------------------------------------------------------------
__global__ void k_prologue(float* amax, const float* scale, float* scale_inv, int delayed) {
  *amax = 0.0f;
  if (delayed) *scale_inv = 1.0f / *scale;
}

// flags of the quantizing kernels (the grid-wide amax itself is in grid_amax.hpp)
constexpr int kAccAmax = 1;     // *amax = max(*amax, amax of this launch)
constexpr int kPublishInv = 2;  // block 0 writes scale_inv = 1 / scale (delayed scaling)

// grid_amax for the 256-thread quantizer blocks
__device__ __forceinline__ void grid_amax_q(float v, float* amax, AmaxWork* w, bool acc) {
  __shared__ uint32_t red[kThreads / 64];
  grid_amax<kThreads>(v, amax, w, acc, red);
}

// Finalize current scaling without a cast: scale and scale_inv from amax.
__global__ void k_current_scale(const float* amax, float* scale, float* scale_inv, float fp8_max,
                                int margin) {
  const float s = scale_from_amax(*amax, fp8_max, margin, 1.0f);
  *scale = s;
  *scale_inv = 1.0f / s;
}

// ----------------------------------------------------------------------------
// flat amax / cast over 16-element chunks, persistent blocks, two chunks per
// lane in flight.  MODE 0: amax + cast with *scale (delayed).  MODE 1: amax
// only.  MODE 2: cast with the current scale derived from *amax (block 0 also
// publishes scale and scale_inv); chunks are visited last-to-first so the tail
// of the input, read last by the amax pass, is reused from the last-level cache.
// ----------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u, float* v);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& u, float* v) {
  v[0] = __uint_as_float(u.x);
  v[1] = __uint_as_float(u.y);
  v[2] = __uint_as_float(u.z);
  v[3] = __uint_as_float(u.w);
}

template <typename T>
__device__ __forceinline__ uint32_t raw_bits(const T* p);
template <>
__device__ __forceinline__ uint32_t raw_bits<uint16_t>(const uint16_t* p) { return *p; }
template <>
__device__ __forceinline__ uint32_t raw_bits<float>(const float* p) { return __float_as_uint(*p); }

// Running max of |x| over raw input words, kept as magnitude bits: for
// non-negative floats the bit patterns order as the values do, so an unsigned
// max is the float max, and a NaN (bits above +inf) wins, as in a plain max.
// bf16: two 16-bit magnitudes per word, combined with a packed 16-bit max.
template <typename T>
__device__ __forceinline__ uint32_t absmax_bits(uint32_t m, const uint4& u);
template <>
__device__ __forceinline__ uint32_t absmax_bits<uint16_t>(uint32_t m, const uint4& u) {
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  v2u16 a = __builtin_bit_cast(v2u16, m);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2u16 b = __builtin_bit_cast(v2u16, w[i] & 0x7fff7fffu);
    a = __builtin_elementwise_max(a, b);
  }
  return __builtin_bit_cast(uint32_t, a);
}
template <>
__device__ __forceinline__ uint32_t absmax_bits<float>(uint32_t m, const uint4& u) {
  m = max(m, u.x & 0x7fffffffu);
  m = max(m, u.y & 0x7fffffffu);
  m = max(m, u.z & 0x7fffffffu);
  m = max(m, u.w & 0x7fffffffu);
  return m;
}
// the float value of a running max from absmax_bits
template <typename T>
__device__ __forceinline__ float absmax_value(uint32_t m) {
  if constexpr (sizeof(T) == 2) return __uint_as_float(max(m & 0xffffu, m >> 16) << 16);
  else return __uint_as_float(m);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Streaming input: read with nontemporal loads (the input is not read again after the
// pass; the FP8 output, stored cached, is what the next GEMM reads from the last-level
// cache).  A 16-byte word of input.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const v4u v = __builtin_nontemporal_load(static_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Raw buffer access: offsets at or past num_records load zeros and drop stores, so
// optional outputs, lanes past a row end and rows past the last one need no branch.
// Branch-free loads and stores let the compiler count the memory operations in flight
// exactly; behind a branch it falls back to waiting for all of them.
typedef int bv4i __attribute__((ext_vector_type(4)));
typedef int bv2i __attribute__((ext_vector_type(2)));
__device__ bv4i buffer_load4(bv4i rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ void buffer_store2(bv2i data, bv4i rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.store.v2i32");
__device__ void buffer_store1(int data, bv4i rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.store.i32");
__device__ void buffer_store4(bv4i data, bv4i rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.store.v4i32");
__device__ __forceinline__ bv4i buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  bv4i r;
  r[0] = static_cast<int>(a & 0xffffffffu);
  r[1] = static_cast<int>(a >> 32);  // stride 0: raw byte-addressed buffer
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;
  return r;
}

// Flat amax + cast: one 16-byte word per lane and load instruction (a wave covers 1 KB
// contiguous), kFlatU words per lane in flight; the word's EW elements go out as EW
// bytes.  The cast passes (MODE 0, 2) stream the input; the amax-only pass of current
// scaling (MODE 1) reads it cached, so that the cast pass after it finds the end of the
// input in the last-level cache (MODE 2 visits the words last to first).
constexpr int kFlatU = 2;
template <typename T, bool E5M2, int MODE>
__global__ __launch_bounds__(kThreads) void k_amax_cast(const T* __restrict__ x, int64_t n,
                                                        float* __restrict__ scale,
                                                        float* __restrict__ scale_inv,
                                                        float* __restrict__ amax,
                                                        uint8_t* __restrict__ out, int margin,
                                                        AmaxWork* __restrict__ work, int flags) {
  constexpr bool kAmax = MODE != 2;
  constexpr bool kCast = MODE != 1;
  constexpr int U = kFlatU;
  float s = 1.0f;
  if constexpr (MODE == 0) s = *scale;
  if constexpr (MODE != 2) {
    if ((flags & kPublishInv) && blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = 1.0f / *scale;
  }
  if constexpr (MODE == 2) {
    s = scale_from_amax(*amax, Fp8Traits<E5M2>::max, margin, 1.0f);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *scale = s;
      *scale_inv = 1.0f / s;
    }
  }
  constexpr int EW = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte word
  uint32_t m = 0u;  // running max of |x| as magnitude bits
  const uint4* xw = reinterpret_cast<const uint4*>(x);
  const int64_t nw = n / EW;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  auto at = [&](int64_t i) { return MODE == 2 ? nw - 1 - i : i; };
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < nw; b += stride * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = b + u * stride;
      if (i < nw) raw[u] = MODE == 1 ? xw[at(i)] : load_stream(xw + at(i));
      else raw[u] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = b + u * stride;
      if (i >= nw) break;
      if constexpr (kAmax) m = absmax_bits<T>(m, raw[u]);
      if constexpr (kCast) {
        float v[EW];
        unpack16<T>(raw[u], v);
        if constexpr (EW == 8) {
          const v2u q = {quant4<E5M2>(v[0], v[1], v[2], v[3], s), quant4<E5M2>(v[4], v[5], v[6], v[7], s)};
          *reinterpret_cast<v2u*>(out + at(i) * 8) = q;
        } else {
          *reinterpret_cast<uint32_t*>(out + at(i) * 4) = quant4<E5M2>(v[0], v[1], v[2], v[3], s);
        }
      }
    }
  }
  if (blockIdx.x == 0) {  // tail of fewer than EW elements
    const int64_t t = nw * EW + threadIdx.x;
    if (t < n) {
      const uint32_t bits = raw_bits<T>(x + t);
      if constexpr (kAmax) m = absmax_bits<T>(m, make_uint4(bits, 0u, 0u, 0u));
      if constexpr (kCast) {
        const float v = sizeof(T) == 2 ? __uint_as_float(bits << 16) : __uint_as_float(bits);
        out[t] = static_cast<uint8_t>(quant4<E5M2>(v, 0.f, 0.f, 0.f, s) & 0xffu);
      }
    }
  }
  if constexpr (kAmax) grid_amax_q(absmax_value<T>(m), amax, work, (flags & kAccAmax) != 0);
}

// ----------------------------------------------------------------------------
// cast + transpose, persistent blocks over 128 x 128 tiles.  MODE 0: amax +
// cast with *scale.  MODE 2: cast with the current scale from *amax, tiles
// visited last-to-first so that the end of the input, read last by the amax
// pass, is still in the last-level cache when it is read again.
//
// Loads: 16 bytes per lane, a tile row is 256 (bf16) or 512 (fp32) contiguous
// bytes.  Row-wise FP8 output: 8 or 4 bytes per lane, 128-byte rows.  The tile's
// FP8 bytes go through LDS (pitch 132 bytes); for the transposed output each
// lane reads a 16 x 4 byte block as 16 dwords, transposes it with byte permutes
// and writes four 16-byte column runs; 8 consecutive lanes complete one
// 128-byte line of out_col.  The next tile's loads, into the second of two register
// sets, are issued before the current tile's transposed stores, so each block keeps a
// tile in flight.  Whole tiles load and store through buffer descriptors with no
// branch (an absent next tile or output copy is an empty buffer), so the compiler
// counts the operations in flight exactly instead of waiting for all of them.  A
// request for the row-wise copy alone (no dbias) is the flat cast.
// ----------------------------------------------------------------------------
constexpr int kCT = 128;             // tile edge
constexpr int kCTPitch = kCT + 4;    // LDS bytes per tile row

template <typename T>
struct CTMap {
  static constexpr int E = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte load
  static constexpr int LPR = kCT / E;                          // lanes per tile row
  static constexpr int RPP = kThreads / LPR;                   // tile rows per pass
  static constexpr int NP = kCT / RPP;                         // passes per tile
};

// Whole tiles take the vector path when rows and columns are vector-aligned and
// every offset inside a tile fits in 31 bits.
template <typename T>
__host__ __device__ __forceinline__ bool ct_vec_ok(int64_t R, int64_t C) {
  constexpr int64_t E = 16 / static_cast<int64_t>(sizeof(T));
  return (C % E) == 0 && (R % 16) == 0 && C * kCT * static_cast<int64_t>(sizeof(T)) < (int64_t{1} << 31) &&
         R * kCT < (int64_t{1} << 31);
}

// FAST = true: the whole tiles, 16-byte loads, vector stores, 32-bit offsets
// inside a tile (the host checks that they fit).  FAST = false: the ragged
// right column and bottom row of tiles (or every tile when rows or columns are
// not vector-aligned), with element loads and byte stores under bounds checks.
template <typename T, bool E5M2, int MODE, bool FAST, bool DBIAS = false>
__global__ __launch_bounds__(kThreads) void k_cast_transpose(
    const T* __restrict__ x, int64_t R, int64_t C, float* __restrict__ scale,
    float* __restrict__ scale_inv, float* __restrict__ amax, uint8_t* __restrict__ out_row,
    uint8_t* __restrict__ out_col, int margin, AmaxWork* __restrict__ work, int flags,
    float* __restrict__ dbias_part) {
  using M = CTMap<T>;
  constexpr int E = M::E, NP = M::NP, RPP = M::RPP;
  constexpr int kBits = 8 * static_cast<int>(sizeof(T));
  __shared__ uint32_t lds[kCT * kCTPitch / 4];
  // DBIAS: per tile, column sums of the tile's rows, reduced over the lanes of one
  // column through LDS: red[tile row group][column]
  __shared__ float red[DBIAS ? RPP * kCT : 1];

  float s = 1.0f;
  if constexpr (MODE == 0) {
    s = *scale;
    if ((flags & kPublishInv) && blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = 1.0f / s;
  }
  if constexpr (MODE == 2) {
    s = scale_from_amax(*amax, Fp8Traits<E5M2>::max, margin, 1.0f);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *scale = s;
      *scale_inv = 1.0f / s;
    }
  }
  const int64_t ntc = (C + kCT - 1) / kCT, ntr = (R + kCT - 1) / kCT;
  const int64_t nfc = C / kCT, nfr = R / kCT;  // whole tiles
  const bool vec_ok = ct_vec_ok<T>(R, C);
  const int64_t ntiles = FAST ? nfr * nfc : (vec_ok ? ntr * ntc - nfr * nfc : ntr * ntc);
  const int t = threadIdx.x;
  const int prow = t / M::LPR, pcol = (t % M::LPR) * E;  // load / row-output position in a pass
  const int cg = t >> 3, rg = t & 7;                     // transposed output: columns 4cg.., rows 16rg..
  const uint32_t ld_off = static_cast<uint32_t>((prow * C + pcol) * static_cast<int64_t>(sizeof(T)));
  const uint32_t ld_pass = static_cast<uint32_t>(RPP * C * static_cast<int64_t>(sizeof(T)));
  const uint32_t ro_off = static_cast<uint32_t>(prow * C + pcol);
  const uint32_t ro_pass = static_cast<uint32_t>(RPP * C);
  const uint32_t co_off = static_cast<uint32_t>(4 * cg * R + 16 * rg);
  const uint32_t co_col = static_cast<uint32_t>(R);
  uint32_t m = 0u;  // running max of |x| as magnitude bits

  auto origin = [&](int64_t i, int64_t& r0, int64_t& c0) {
    if (FAST) {
      const int64_t tile = MODE == 2 ? ntiles - 1 - i : i;
      r0 = (tile / nfc) * kCT;
      c0 = (tile % nfc) * kCT;
    } else if (!vec_ok) {
      r0 = (i / ntc) * kCT;
      c0 = (i % ntc) * kCT;
    } else if (i < nfr * (ntc - nfc)) {  // right column of ragged tiles
      r0 = (i / (ntc - nfc)) * kCT;
      c0 = (nfc + i % (ntc - nfc)) * kCT;
    } else {  // bottom row
      const int64_t j = i - nfr * (ntc - nfc);
      r0 = (nfr + j / ntc) * kCT;
      c0 = (j % ntc) * kCT;
    }
    return FAST;
  };
  // FAST: one 16-byte load per pass; otherwise element loads with bounds checks
  // (outside the matrix reads as 0), packed into the same raw words.
  // the tile's bytes of x from its first element ((kCT - 1) C + kCT elements)
  const uint32_t tile_x_bytes = static_cast<uint32_t>(((kCT - 1) * C + kCT) * static_cast<int64_t>(sizeof(T)));
  auto load1 = [&](int p, int64_t r0, int64_t c0, bool valid = true) {
    if constexpr (FAST) {  // an absent tile (valid false): an empty buffer, zeros, nothing fetched
      const bv4i rs = buf_rsrc(x + (valid ? r0 * C + c0 : 0), valid ? tile_x_bytes : 0u);
      const bv4i v = buffer_load4(rs, static_cast<int>(ld_off + p * ld_pass), 0, 2);
      return make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                        static_cast<uint32_t>(v[3]));
    } else {
      const int64_t r = r0 + p * RPP + prow;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int64_t c = c0 + pcol + j;
        const uint32_t b = (r < R && c < C) ? raw_bits<T>(x + r * C + c) : 0u;
        w[(j * kBits) / 32] |= b << ((j * kBits) % 32);
      }
      return make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  // The tile's registers are reloaded with the next tile as soon as they are consumed:
  // pass by pass without the transposed copy, after all passes with it (the transposed
  // stores then run with the next tile's loads in flight).
  // raw: this tile's registers; nxt: the next tile's (two sets, alternating, so the loads
  // of the next tile land in registers the current tile does not use)
  auto process = [&](uint4 (&raw)[NP], uint4 (&nxt)[NP], int64_t r0, int64_t c0, bool has1, int64_t r1,
                     int64_t c1) {
    __syncthreads();  // the previous tile's LDS reads are done
    // the tile's rows of the row copy ((kCT - 1) C + kCT bytes from its first byte)
    const bv4i rs_row = buf_rsrc(out_row != nullptr ? out_row + r0 * C + c0 : nullptr,
                                 out_row != nullptr ? static_cast<uint32_t>((kCT - 1) * C + kCT) : 0u);
    float cs[E];  // DBIAS: this lane's column sums over its rows of the tile (rows past R read 0)
#pragma unroll
    for (int j = 0; j < E; ++j) cs[j] = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int lr = p * RPP + prow;
      float v[E];
      unpack16<T>(raw[p], v);
      if constexpr (DBIAS) {
#pragma unroll
        for (int j = 0; j < E; ++j) cs[j] = __fadd_rn(cs[j], v[j]);
      }
      if constexpr (MODE == 0) m = absmax_bits<T>(m, raw[p]);
      uint32_t q[E / 4];
#pragma unroll
      for (int j = 0; j < E / 4; ++j) {
        q[j] = quant4<E5M2>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], s);
        lds[(lr * kCTPitch + pcol) / 4 + j] = q[j];
      }
      if constexpr (FAST) {  // no row copy: an empty buffer, the stores are dropped
        if constexpr (E == 8) {
          const bv2i qq = {static_cast<int>(q[0]), static_cast<int>(q[1])};
          buffer_store2(qq, rs_row, static_cast<int>(ro_off + p * ro_pass), 0, 0);
        } else {
          buffer_store1(static_cast<int>(q[0]), rs_row, static_cast<int>(ro_off + p * ro_pass), 0, 0);
        }
      } else if (out_row != nullptr) {
        if (r0 + lr < R) {
          uint8_t* o = out_row + (r0 + lr) * C + c0 + pcol;
#pragma unroll
          for (int j = 0; j < E; ++j)
            if (c0 + pcol + j < C) o[j] = static_cast<uint8_t>(q[j >> 2] >> (8 * (j & 3)));
        }
      }
    }
    if constexpr (DBIAS) {
      // tile column sums, rows in a fixed order (lane passes, then lane groups), so the
      // result does not depend on scheduling; one partial per (tile row, column)
#pragma unroll
      for (int j = 0; j < E; ++j) red[prow * kCT + pcol + j] = cs[j];
      __syncthreads();
      if (t < kCT && c0 + t < C) {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < RPP; ++g) acc = __fadd_rn(acc, red[g * kCT + t]);
        dbias_part[(r0 / kCT) * C + c0 + t] = acc;
      }
    }
    // the next tile's loads, in flight during the transposed stores.  FAST: loads and
    // stores without branches (an absent next tile or output is an empty buffer), so the
    // compiler counts the operations in flight exactly
    if constexpr (FAST) {
#pragma unroll
      for (int p = 0; p < NP; ++p) nxt[p] = load1(p, r1, c1, has1);
    } else {
      if (has1) {
#pragma unroll
        for (int p = 0; p < NP; ++p) nxt[p] = load1(p, r1, c1);
      }
      if (out_col == nullptr) return;
    }
    __syncthreads();
    uint32_t d[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) d[k] = lds[((16 * rg + k) * kCTPitch) / 4 + cg];
    // w[i][j]: column 4cg + i, rows 16rg + 4j .. 16rg + 4j + 3 (row-minor bytes)
    uint32_t w[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d0 = d[4 * j], d1 = d[4 * j + 1], d2 = d[4 * j + 2], d3 = d[4 * j + 3];
      const uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);  // d0.b0 d1.b0 d0.b1 d1.b1
      const uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);  // d0.b2 d1.b2 d0.b3 d1.b3
      const uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
      w[0][j] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      w[1][j] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      w[2][j] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      w[3][j] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
    if constexpr (FAST) {  // the tile's columns of the column copy ((kCT - 1) R + kCT bytes)
      const bv4i rs_col = buf_rsrc(out_col != nullptr ? out_col + c0 * R + r0 : nullptr,
                                   out_col != nullptr ? static_cast<uint32_t>((kCT - 1) * R + kCT) : 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bv4i ww = {static_cast<int>(w[i][0]), static_cast<int>(w[i][1]), static_cast<int>(w[i][2]),
                         static_cast<int>(w[i][3])};
        buffer_store4(ww, rs_col, static_cast<int>(co_off + i * co_col), 0, 0);
      }
    } else {
      const int64_t rb = r0 + 16 * rg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + 4 * cg + i;
        if (c < C) {
          uint8_t* o = out_col + c * R + rb;
#pragma unroll
          for (int k = 0; k < 16; ++k)
            if (rb + k < R) o[k] = static_cast<uint8_t>(w[i][k >> 2] >> (8 * (k & 3)));
        }
      }
    }
  };

  int64_t i = blockIdx.x;
  if (i < ntiles) {
    uint4 ra[NP], rb[NP];
    int64_t r0, c0;
    origin(i, r0, c0);
#pragma unroll
    for (int p = 0; p < NP; ++p) ra[p] = load1(p, r0, c0);
    if constexpr (FAST) {
      // four dropped stores: every later tile's loads are followed by the four transposed
      // stores, so the loop is entered with the same operations in flight either way
      const bv4i none = buf_rsrc(nullptr, 0u);
      const bv4i zero = {0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) buffer_store4(zero, none, 16 * k, 0, 0);
    }
    auto step = [&](uint4 (&cur)[NP], uint4 (&nxt)[NP]) {  // false after the last tile
      const int64_t i1 = i + gridDim.x;
      const bool has1 = i1 < ntiles;
      int64_t r1 = 0, c1 = 0;
      if (has1) origin(i1, r1, c1);
      process(cur, nxt, r0, c0, has1, r1, c1);
      i = i1;
      r0 = r1;
      c0 = c1;
      return has1;
    };
    while (step(ra, rb) && step(rb, ra)) {
    }
  }
  if constexpr (MODE == 0) grid_amax_q(absmax_value<T>(m), amax, work, (flags & kAccAmax) != 0);
}

// dbias[c] = sum over tile rows of the partial column sums (0 when R == 0), in a fixed
// order: a block takes 64 columns; thread (q, c) sums tile rows q, q + 4, q + 8, ... in
// four interleaved accumulators (four loads in flight), then the four accumulators and
// the four quarters q are added in index order.
constexpr int kDbCols = 64;
__global__ __launch_bounds__(256) void k_dbias_reduce(const float* __restrict__ part, int64_t ntr, int64_t C,
                                                      float* __restrict__ dbias) {
  __shared__ float red[4][kDbCols];
  const int q = threadIdx.x / kDbCols, cl = threadIdx.x % kDbCols;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kDbCols + cl;
  float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (c < C) {
    int64_t r = q;
    for (; r + 12 < ntr; r += 16) {
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = __fadd_rn(a[u], part[(r + 4 * u) * C + c]);
    }
    for (int u = 0; r < ntr; r += 4, ++u) a[u & 3] = __fadd_rn(a[u & 3], part[r * C + c]);
  }
  red[q][cl] = __fadd_rn(__fadd_rn(a[0], a[1]), __fadd_rn(a[2], a[3]));
  __syncthreads();
  if (q == 0 && c < C)
    dbias[c] = __fadd_rn(__fadd_rn(red[0][cl], red[1][cl]), __fadd_rn(red[2][cl], red[3][cl]));
}

// ----------------------------------------------------------------------------
// LayerNorm over the last axis with the output written as FP8 codes (te.LayerNorm,
// whose output feeds the QKV and MLP-up GEMMs, fused with the cast of that output):
//   mu = mean_c x, var = mean_c (x - mu)^2, rsigma = 1 / sqrt(var + eps),
//   y = ((x - mu) * rsigma) * gamma + beta,  q = satRNE(fl32(y * scale)),
// every operation a separately rounded fp32 operation.  One wave per row (a block
// holds four rows, persistent over row groups): lane l takes the 16-byte chunks
// l, l + 64, ... of the row.  Rows of up to NREG chunks per lane (two for rows of up
// to 128 chunks, else kLnReg: 4096 bf16 / 2048 fp32 columns) stay in registers, and
// the wave loads its next row while it works on the current one; gamma and beta then
// sit in LDS, staged once per block (register use allows two blocks per CU).
// Wider rows are re-read from cache for the second and third pass.  Sums run per
// lane over four partial sums in chunk order (one per element slot j mod 4), then
// over the wave by an xor butterfly (every lane ends with the same bits), so a run is
// reproducible and no block barrier is needed in the row loop.  MODE 0: delayed
// scaling (amax of y + cast in one launch); MODE 1: current scaling's first pass
// (statistics, amax of y); MODE 2: its cast pass with the scale from *amax.
// ----------------------------------------------------------------------------
constexpr int kLnReg = 8;
constexpr int kLnParamBytes = 16384;  // gamma or beta staged in LDS (4096 fp32 values)

template <typename P, int EV>
__device__ __forceinline__ void load_params(const P* p, int64_t c, float* out) {
  if constexpr (sizeof(P) == 4) {
#pragma unroll
    for (int k = 0; k < EV / 4; ++k) {
      const float4 f = *reinterpret_cast<const float4*>(p + c + 4 * k);
      out[4 * k] = f.x;
      out[4 * k + 1] = f.y;
      out[4 * k + 2] = f.z;
      out[4 * k + 3] = f.w;
    }
  } else if constexpr (EV == 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + c);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(w[i]);
      out[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(p + c);
    out[0] = bf16_lo(u.x);
    out[1] = bf16_hi(u.x);
    out[2] = bf16_lo(u.y);
    out[3] = bf16_hi(u.y);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __fadd_rn(v, __shfl_xor(v, off, 64));
  return v;
}

template <typename T, typename P, bool E5M2, int MODE, int NREG>
__global__ __launch_bounds__(kThreads) void k_layernorm(const T* __restrict__ x, int64_t R, int64_t C,
                                                        const P* __restrict__ gamma, const P* __restrict__ beta,
                                                        float eps, float* __restrict__ scale,
                                                        float* __restrict__ scale_inv, float* __restrict__ amax,
                                                        uint8_t* __restrict__ out, float* __restrict__ mu_out,
                                                        float* __restrict__ rs_out, int margin,
                                                        AmaxWork* __restrict__ work, int flags) {
  constexpr int EV = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  constexpr int kWaves = kThreads / 64;
  // gamma at [0, kLnParamBytes), beta at [kLnParamBytes, 2 kLnParamBytes)
  __shared__ uint4 prm[2 * kLnParamBytes / 16];
  const int t = threadIdx.x, lane = t & 63, wid = __builtin_amdgcn_readfirstlane(t >> 6);
  float s = 1.0f;
  if constexpr (MODE == 0) {
    s = *scale;
    if ((flags & kPublishInv) && blockIdx.x == 0 && t == 0) *scale_inv = 1.0f / s;
  }
  if constexpr (MODE == 2) {
    s = scale_from_amax(*amax, Fp8Traits<E5M2>::max, margin, 1.0f);
    if (blockIdx.x == 0 && t == 0) {
      *scale = s;
      *scale_inv = 1.0f / s;
    }
  }
  const int64_t nch = C / EV;
  const int64_t pbytes = C * static_cast<int64_t>(sizeof(P));
  // register path: the row fits NREG chunks per lane, gamma and beta fit LDS, and the
  // statistics' byte offsets (4 row) fit the buffer offsets (below 2^31)
  const bool fast = nch <= 64 * NREG && pbytes <= kLnParamBytes && R < (int64_t{1} << 29);
  const float inv_c = 1.0f / static_cast<float>(C);
  uint32_t m = 0u;  // running max of |y| as magnitude bits
  const uint8_t* gl = reinterpret_cast<const uint8_t*>(prm);
  const uint8_t* bl = gl + kLnParamBytes;

  // y and its code for one chunk: g, b the chunk's gamma and beta
  auto out_vals = [&](const float (&v)[EV], const float (&g)[EV], const float (&b)[EV], float mean, float rs,
                      int64_t row, int64_t ch) {
    float y[EV];
#pragma unroll
    for (int j = 0; j < EV; ++j) {
      y[j] = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(v[j], mean), rs), g[j]), b[j]);
      if constexpr (MODE != 2) m = max(m, __float_as_uint(y[j]) & 0x7fffffffu);
    }
    if constexpr (MODE != 1) {
      uint8_t* o = out + row * C + ch * EV;
      if constexpr (EV == 8)
        *reinterpret_cast<uint2*>(o) = make_uint2(quant4<E5M2>(y[0], y[1], y[2], y[3], s),
                                                  quant4<E5M2>(y[4], y[5], y[6], y[7], s));
      else
        *reinterpret_cast<uint32_t*>(o) = quant4<E5M2>(y[0], y[1], y[2], y[3], s);
    }
  };
  auto stats_out = [&](int64_t row, float mean, float rs) {
    if (MODE != 2 && lane == 0) {
      if (mu_out != nullptr) mu_out[row] = mean;
      if (rs_out != nullptr) rs_out[row] = rs;
    }
  };

  if (fast) {
    const int n16 = static_cast<int>(pbytes / 16);
    for (int i = t; i < n16; i += kThreads) {
      prm[i] = reinterpret_cast<const uint4*>(gamma)[i];
      prm[kLnParamBytes / 16 + i] = reinterpret_cast<const uint4*>(beta)[i];
    }
    __syncthreads();
    // EV parameters of chunk ch from LDS
    auto lds_params = [&](const uint8_t* base, int64_t ch, float (&o)[EV]) {
      constexpr int PB = EV * static_cast<int>(sizeof(P));  // 8, 16 or 32 bytes
      const uint8_t* p = base + ch * PB;
      if constexpr (sizeof(P) == 4) {
#pragma unroll
        for (int k = 0; k < EV / 4; ++k) {
          const uint4 u = reinterpret_cast<const uint4*>(p)[k];
          o[4 * k] = __uint_as_float(u.x);
          o[4 * k + 1] = __uint_as_float(u.y);
          o[4 * k + 2] = __uint_as_float(u.z);
          o[4 * k + 3] = __uint_as_float(u.w);
        }
      } else if constexpr (EV == 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = bf16_lo(w[i]);
          o[2 * i + 1] = bf16_hi(w[i]);
        }
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        o[0] = bf16_lo(u.x);
        o[1] = bf16_hi(u.x);
        o[2] = bf16_lo(u.y);
        o[3] = bf16_hi(u.y);
      }
    };
    const uint32_t xrow_bytes = static_cast<uint32_t>(C * static_cast<int64_t>(sizeof(T)));
    // a row past the last one: an empty buffer (every load reads zeros, nothing fetched)
    auto load_row = [&](int64_t row, uint4 (&reg)[NREG]) {
      const bool ok = row < R;
      const bv4i rs = buf_rsrc(x + (ok ? row : 0) * C, ok ? xrow_bytes : 0u);
#pragma unroll
      for (int k = 0; k < NREG; ++k) {
        const bv4i v = buffer_load4(rs, (lane + 64 * k) * 16, 0, MODE == 1 ? 0 : 2);
        reg[k] = make_uint4(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), static_cast<uint32_t>(v[2]),
                            static_cast<uint32_t>(v[3]));
      }
    };
    const bv4i rs_mu = buf_rsrc(mu_out, mu_out != nullptr && MODE != 2 ? static_cast<uint32_t>(R * 4) : 0u);
    const bv4i rs_rs = buf_rsrc(rs_out, rs_out != nullptr && MODE != 2 ? static_cast<uint32_t>(R * 4) : 0u);
    auto process = [&](int64_t row, const uint4 (&reg)[NREG]) {
      // chunks past the row end hold zeros: they add +0 to the sums (no branch)
      float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < NREG; ++k) {
        float v[EV];
        unpack16<T>(reg[k], v);
#pragma unroll
        for (int j = 0; j < EV; ++j) a4[j & 3] = __fadd_rn(a4[j & 3], v[j]);
      }
      const float mean = __fmul_rn(wave_sum(__fadd_rn(__fadd_rn(a4[0], a4[1]), __fadd_rn(a4[2], a4[3]))), inv_c);
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[q] = 0.0f;
#pragma unroll
      for (int k = 0; k < NREG; ++k) {
        const bool in_row = lane + 64 * k < nch;
        float v[EV];
        unpack16<T>(reg[k], v);
#pragma unroll
        for (int j = 0; j < EV; ++j) {
          const float d = __fsub_rn(v[j], mean);
          a4[j & 3] = __fadd_rn(a4[j & 3], in_row ? __fmul_rn(d, d) : 0.0f);
        }
      }
      const float var = __fmul_rn(wave_sum(__fadd_rn(__fadd_rn(a4[0], a4[1]), __fadd_rn(a4[2], a4[3]))), inv_c);
      const float rs = 1.0f / __fsqrt_rn(__fadd_rn(var, eps));
      // lane 0 writes the row statistics; the other lanes' offsets are out of range
      const int soff = lane == 0 ? static_cast<int>(row * 4) : static_cast<int>(0x80000000u);
      buffer_store1(__float_as_int(mean), rs_mu, soff, 0, 0);
      buffer_store1(__float_as_int(rs), rs_rs, soff, 0, 0);
      const bv4i rs_out_row = buf_rsrc(out + row * C, MODE != 1 ? static_cast<uint32_t>(C) : 0u);
#pragma unroll
      for (int k = 0; k < NREG; ++k) {
        const int64_t ch = lane + 64 * k;
        const bool in_row = ch < nch;  // lanes past the row end: parameters of chunk 0, store dropped
        float v[EV], g[EV], b[EV], y[EV];
        unpack16<T>(reg[k], v);
        lds_params(gl, in_row ? ch : 0, g);
        lds_params(bl, in_row ? ch : 0, b);
#pragma unroll
        for (int j = 0; j < EV; ++j) {
          y[j] = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(v[j], mean), rs), g[j]), b[j]);
          if constexpr (MODE != 2) m = in_row ? max(m, __float_as_uint(y[j]) & 0x7fffffffu) : m;
        }
        const int off = static_cast<int>(ch * EV);  // >= C past the row end: dropped
        if constexpr (EV == 8) {
          const bv2i q = {static_cast<int>(quant4<E5M2>(y[0], y[1], y[2], y[3], s)),
                            static_cast<int>(quant4<E5M2>(y[4], y[5], y[6], y[7], s))};
          buffer_store2(q, rs_out_row, off, 0, 0);
        } else {
          buffer_store1(static_cast<int>(quant4<E5M2>(y[0], y[1], y[2], y[3], s)), rs_out_row, off, 0, 0);
        }
      }
    };
    // two register sets: the next row is in flight while the current one is worked on
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
    int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wid;
    uint4 ra[NREG], rb[NREG];
    load_row(row, ra);
    while (row < R) {
      int64_t nx = row + stride;
      load_row(nx, rb);
      process(row, ra);
      row = nx;
      if (row >= R) break;
      nx = row + stride;
      load_row(nx, ra);
      process(row, rb);
      row = nx;
    }
  } else {
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wid; row < R;
         row += static_cast<int64_t>(gridDim.x) * kWaves) {
      const T* xr = x + row * C;
      auto load = [&](int64_t ch) { return *reinterpret_cast<const uint4*>(xr + ch * EV); };
      float a4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int64_t ch = lane; ch < nch; ch += 64) {
        float v[EV];
        unpack16<T>(load(ch), v);
#pragma unroll
        for (int j = 0; j < EV; ++j) a4[j & 3] = __fadd_rn(a4[j & 3], v[j]);
      }
      const float mean = __fmul_rn(wave_sum(__fadd_rn(__fadd_rn(a4[0], a4[1]), __fadd_rn(a4[2], a4[3]))), inv_c);
#pragma unroll
      for (int q = 0; q < 4; ++q) a4[q] = 0.0f;
      for (int64_t ch = lane; ch < nch; ch += 64) {
        float v[EV];
        unpack16<T>(load(ch), v);
#pragma unroll
        for (int j = 0; j < EV; ++j) {
          const float d = __fsub_rn(v[j], mean);
          a4[j & 3] = __fadd_rn(a4[j & 3], __fmul_rn(d, d));
        }
      }
      const float var = __fmul_rn(wave_sum(__fadd_rn(__fadd_rn(a4[0], a4[1]), __fadd_rn(a4[2], a4[3]))), inv_c);
      const float rs = 1.0f / __fsqrt_rn(__fadd_rn(var, eps));
      stats_out(row, mean, rs);
      for (int64_t ch = lane; ch < nch; ch += 64) {
        float v[EV], g[EV], b[EV];
        unpack16<T>(load(ch), v);
        load_params<P, EV>(gamma, ch * EV, g);
        load_params<P, EV>(beta, ch * EV, b);
        out_vals(v, g, b, mean, rs, row, ch);
      }
    }
  }
  if constexpr (MODE != 2) grid_amax_q(__uint_as_float(m), amax, work, (flags & kAccAmax) != 0);
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
  if (E == 255) return 127;  // infinite amax: log2 = +inf, clamped (code 254)
  const int fl = E ? E - 127 : (31 - __clz(static_cast<int>(u & 0x7fffffu))) - 149;
  int e = fl - Fp8Traits<E5M2>::emax_elem;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

template <bool E5M2>
__device__ __forceinline__ void mx_block32(const float* v, uint32_t* q, uint8_t* code) {
  uint32_t mb = 0u;  // block amax as magnitude bits: a NaN wins, as in a plain max
#pragma unroll
  for (int j = 0; j < 32; ++j) mb = max(mb, __float_as_uint(v[j]) & 0x7fffffffu);
  const int e = mx_exponent<E5M2>(__uint_as_float(mb));
  *code = static_cast<uint8_t>(e + 127);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    q[j] = cvt4<E5M2>(saturate<E5M2>(__builtin_ldexpf(v[4 * j], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 1], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 2], -e)),
                      saturate<E5M2>(__builtin_ldexpf(v[4 * j + 3], -e)));
}

constexpr int kTR = 128, kTC = 64;  // MXFP8 tile
constexpr int kMxPitch = kTC + 1;   // floats

template <typename T>
__device__ __forceinline__ bool rows_vec_ok(int64_t cols) {
  return (cols % (16 / sizeof(T))) == 0;  // every row starts 16-byte aligned
}

template <typename T, bool E5M2, bool DBIAS = false>
__global__ __launch_bounds__(kThreads) void k_mxfp8(const T* __restrict__ x, int64_t R, int64_t C,
                                                    uint8_t* __restrict__ out_row,
                                                    uint8_t* __restrict__ scale_row,
                                                    uint8_t* __restrict__ out_col,
                                                    uint8_t* __restrict__ scale_col,
                                                    float* __restrict__ dbias_part) {
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
  if (out_col != nullptr || DBIAS) {
#pragma unroll
    for (int j = 0; j < 32; ++j) tile[lr * kMxPitch + lc + j] = v[j];
    __syncthreads();
  }
  if constexpr (DBIAS) {
    // the tile's column sums in the order of the cast-transpose pass over the same
    // input type: rows g, g + G, ... summed for each g < G (G = its rows per pass),
    // then the G group sums in order (rows past R read 0)
    constexpr int G = CTMap<T>::RPP, NQ = CTMap<T>::NP;
    static_assert(G * NQ == kTR, "a tile row group per pass");
    if (t < kTC && c0 + t < C) {
      float acc = 0.0f;
      for (int g = 0; g < G; ++g) {
        float sg = 0.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) sg = __fadd_rn(sg, tile[(G * q + g) * kMxPitch + t]);
        acc = __fadd_rn(acc, sg);
      }
      dbias_part[static_cast<int64_t>(blockIdx.y) * C + c0 + t] = acc;
    }
  }
  if (out_col != nullptr) {
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

// ----------------------------------------------------------------------------
// MXFP4: E2M1 elements with one E8M0 exponent per 32 elements, two codes per byte
// (element 2i in the low nibble).  Block exponent e = floor(log2 amax) - 2 (4 is the
// largest E2M1 power of two), clamped to [-127, 127], 127 for an infinite amax; a
// block holding a NaN takes scale code 255 and is cast with e = 0 (E2M1 has no NaN
// code: a NaN element becomes +0).  Elements round to nearest, ties to the even
// mantissa, and saturate at 6.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = __builtin_fabsf(y);
  // midpoints between the magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; on a midpoint the
  // neighbour with the even mantissa (0, 1, 2, 4) wins, hence > or >=
  const uint32_t c = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                     static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                     static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                     static_cast<uint32_t>(a > 5.0f);
  const uint32_t neg = (__float_as_uint(y) >> 31) & static_cast<uint32_t>(a == a);  // NaN -> +0
  return c | (neg << 3);
}

// exponent of a block whose amax magnitude bits are mb (finite or infinite)
__device__ __forceinline__ int mx4_exponent(uint32_t mb) {
  if (mb == 0u) return 0;
  if (mb >= 0x7f800000u) return 127;
  const int E = static_cast<int>(mb >> 23);
  const int fl = E ? E - 127 : (31 - __clz(static_cast<int>(mb))) - 149;
  const int e = fl - 2;
  return e < -127 ? -127 : e;
}

// Eight values (already scaled by 2^-e) -> one dword of codes, value j in nibble j.
// The gfx950 conversion rounds to nearest even, saturates at 6 and keeps the sign of
// zero exactly as e2m1_code does, but turns a NaN into +-6: blocks holding a NaN take
// e2m1_code instead.
__device__ __forceinline__ uint32_t e2m1_pack8(const float* w) {
  uint32_t d = 0u;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, w[0], w[1], 1.0f, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, w[2], w[3], 1.0f, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, w[4], w[5], 1.0f, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, w[6], w[7], 1.0f, 3);
  return d;
}

__device__ __forceinline__ uint32_t e2m1_pack8_slow(const float* w) {
  uint32_t d = 0u;
#pragma unroll
  for (int n = 0; n < 8; ++n) d |= e2m1_code(w[n]) << (4 * n);
  return d;
}

// 32 values -> 16 bytes of packed codes (q[w] holds elements 8w .. 8w + 7) and the code
__device__ __forceinline__ void mx4_block32(const float* v, uint32_t* q, uint8_t* code) {
  uint32_t mb = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) mb = max(mb, __float_as_uint(v[j]) & 0x7fffffffu);
  const bool nan = mb > 0x7f800000u;
  const int e = nan ? 0 : mx4_exponent(mb);
  *code = nan ? static_cast<uint8_t>(255) : static_cast<uint8_t>(e + 127);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float y[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) y[n] = __builtin_ldexpf(v[8 * w + n], -e);
    q[w] = nan ? e2m1_pack8_slow(y) : e2m1_pack8(y);
  }
}

// Tiles of 128 rows x 64 columns, a thread per 32-element row block (row-wise copy)
// and, through LDS, per 32-element column block (column-wise copy), as k_mxfp8.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_mxfp4(const T* __restrict__ x, int64_t R, int64_t C,
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
  if (out_row != nullptr && r < R && c0 + lc < C) {  // cols % 32 == 0: whole blocks
    uint32_t q[4];
    uint8_t code;
    mx4_block32(v, q, &code);
    *reinterpret_cast<uint4*>(out_row + r * (C / 2) + (c0 + lc) / 2) = make_uint4(q[0], q[1], q[2], q[3]);
    scale_row[r * (C / 32) + (c0 + lc) / 32] = code;
  }
  if (out_col != nullptr) {
#pragma unroll
    for (int j = 0; j < 32; ++j) tile[lr * kMxPitch + lc + j] = v[j];
    __syncthreads();
    const int oc = t & 63, seg = t >> 6;
    const int64_t c = c0 + oc;
    const int64_t rb = r0 + seg * 32;
    if (c < C && rb < R) {  // rows % 32 == 0: whole blocks
      float w[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) w[j] = tile[(seg * 32 + j) * kMxPitch + oc];
      uint32_t q[4];
      uint8_t code;
      mx4_block32(w, q, &code);
      *reinterpret_cast<uint4*>(out_col + c * (R / 2) + rb / 2) = make_uint4(q[0], q[1], q[2], q[3]);
      scale_col[c * (R / 32) + rb / 32] = code;
    }
  }
}

// ----------------------------------------------------------------------------
// MXFP8, bf16 input, whole 128 x 128 tiles (rows and cols multiples of 128):
// persistent blocks, the next tile's loads in flight, as the cast-transpose.
// Row-wise: a 32-element block of a row is 4 lanes x 8 elements; its amax is a
// bit-pattern max reduced over the 4 lanes, and lane 16g writes the row's four
// E8M0 codes of the tile as one dword.  Column-wise: the raw bf16 tile goes
// through LDS (pitch 272 bytes); thread t quantizes columns 2(t%64), 2(t%64)+1
// over rows 32(t/64) .. +31 (one block each), reading one dword per row; the
// codes are staged back through the same LDS so that out_col goes out as whole
// 128-byte lines and scale_col as one dword of four block codes per column.
// ----------------------------------------------------------------------------
constexpr int kMxTPitch = 272;  // LDS bytes per tile row (128 bf16 + 16)
constexpr int kMxQPitch = 144;  // LDS bytes per staged output row (128 codes + 16)
constexpr int kMx4QPitch = 80;  // MXFP4: 64 bytes of packed codes + 16
static_assert(kCT * kMxQPitch + 4 * kCT <= kCT * kMxTPitch, "column staging reuses the tile");

template <bool E5M2>
__device__ __forceinline__ void mx_quant8(const uint4& raw, int e, uint32_t& q0, uint32_t& q1) {
  float v[8];
  unpack16<uint16_t>(raw, v);
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = saturate<E5M2>(__builtin_ldexpf(v[j], -e));
  q0 = cvt4<E5M2>(w[0], w[1], w[2], w[3]);
  q1 = cvt4<E5M2>(w[4], w[5], w[6], w[7]);
}


// The row-wise MXFP8 quantization of one lane's eight bf16 values with the gfx950
// scaled convert, which divides by the scale 2^e and rounds to nearest even in one
// step but does not saturate: values beyond the format's maximum come out as NaN or
// infinity.  The magnitudes are therefore clamped first, in the bf16 bit domain, to
// max * 2^e (exact in bf16: both maxima carry two mantissa bits), which yields what
// saturating after the exact division yields.  The caller takes this path only for
// blocks of finite values with e > -127 (scale 2^e a normal float, max * 2^e finite);
// it gives the same codes as mx_quant8 on every such input.
typedef short mx_s2 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_b2 __attribute__((ext_vector_type(2)));
typedef unsigned short mx_u2 __attribute__((ext_vector_type(2)));
template <bool E5M2>
__device__ __forceinline__ void mx_quant8_scaled(const uint4& raw, int e, uint32_t& q0, uint32_t& q1) {
  constexpr int kMaxBits = E5M2 ? 0x4760 : 0x43e0;  // bf16 bits of 57344 / 448
  const uint32_t lim = static_cast<uint32_t>(kMaxBits + e * 128);
  const mx_u2 lim2 = {static_cast<unsigned short>(lim), static_cast<unsigned short>(lim)};
  const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const mx_u2 mag = __builtin_bit_cast(mx_u2, w[i] & 0x7fff7fffu);
    const uint32_t cl = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(mag, lim2)) | (w[i] & 0x80008000u);
    c[i] = cl;
  }
  const mx_s2 z = {0, 0};
  mx_s2 r0, r1;
  if constexpr (E5M2) {
    r0 = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(z, __builtin_bit_cast(mx_b2, c[0]), sc, false);
    r0 = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r0, __builtin_bit_cast(mx_b2, c[1]), sc, true);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(z, __builtin_bit_cast(mx_b2, c[2]), sc, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r1, __builtin_bit_cast(mx_b2, c[3]), sc, true);
  } else {
    r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(mx_b2, c[0]), sc, false);
    r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r0, __builtin_bit_cast(mx_b2, c[1]), sc, true);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(z, __builtin_bit_cast(mx_b2, c[2]), sc, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r1, __builtin_bit_cast(mx_b2, c[3]), sc, true);
  }
  q0 = __builtin_bit_cast(uint32_t, r0);
  q1 = __builtin_bit_cast(uint32_t, r1);
}

// FP4: the same tiles written as MXFP4 (four bytes of codes per lane and pass for the
// row-wise copy, 64 bytes per column of the tile for the column-wise one).
// PANEL: the E8M0 scales go out in the GEMM's panel layout: the dword of row r and
// 128-element group g is dword ((r / 256) * G + g) * 256 + r % 256 (G = groups per row),
// so a tile's 128 row dwords are 512 contiguous bytes instead of 128 scattered ones.
// DBIAS: also the per-tile column sums of x (the bias gradient's partials, summed in the
// cast-transpose pass's order) into dbias_part [R / 128, C].
template <bool E5M2, bool ROW, bool COL, bool FP4 = false, bool PANEL = false, bool DBIAS = false>
__global__ __launch_bounds__(kThreads) void k_mxfp8_tiles(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                          uint8_t* __restrict__ out_row,
                                                          uint8_t* __restrict__ scale_row,
                                                          uint8_t* __restrict__ out_col,
                                                          uint8_t* __restrict__ scale_col,
                                                          float* __restrict__ dbias_part) {
  // the scale dword of (row r of a copy with `cols` elements per row, group of c0)
  auto scale_dw = [](uint8_t* base, int64_t r, int64_t cols, int64_t c0) {
    if constexpr (PANEL)
      return reinterpret_cast<uint32_t*>(base) + ((r >> 8) * (cols >> 7) + (c0 >> 7)) * 256 + (r & 255);
    else
      return reinterpret_cast<uint32_t*>(base + r * (cols / 32) + c0 / 32);
  };
  constexpr int NP = 8, RPP = 16;  // passes of 16 rows, 16 lanes x 8 elements per row
  static_assert(NP == CTMap<uint16_t>::NP && RPP == CTMap<uint16_t>::RPP, "the cast-transpose pass's order");
  __shared__ __attribute__((aligned(16))) uint8_t tile[COL ? kCT * kMxTPitch : 16];
  __shared__ float red[DBIAS ? RPP * kCT : 1];
  const int64_t ntc = C / kCT;
  const int64_t ntiles = ntc * (R / kCT);
  const int t = threadIdx.x, lane = t & 63;
  const int prow = t >> 4, pcol = (t & 15) * 8;
  const uint32_t ld_off = static_cast<uint32_t>((prow * C + pcol) * 2);
  const uint32_t ld_pass = static_cast<uint32_t>(RPP * C * 2);
  auto origin = [&](int64_t i, int64_t& r0, int64_t& c0) {
    r0 = (i / ntc) * kCT;
    c0 = (i % ntc) * kCT;
  };
  // one 16-byte load of pass p of the tile at (r0, c0)
  auto load1 = [&](int p, int64_t r0, int64_t c0) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(x + r0 * C + c0);
    return load_stream(base + ld_off + p * ld_pass);
  };
  // The tile's registers are reloaded with the next tile as soon as they are consumed:
  // pass by pass without the column copy, after all passes with it (the column work
  // then runs with the next tile's loads in flight).
  auto process = [&](uint4 (&raw)[NP], int64_t r0, int64_t c0, bool has1, int64_t r1, int64_t c1) {
    if constexpr (COL || DBIAS) __syncthreads();  // the previous tile's LDS reads are done
    float cs[8];  // DBIAS: this lane's column sums over its rows of the tile
#pragma unroll
    for (int j = 0; j < 8; ++j) cs[j] = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int lr = p * RPP + prow;
      if constexpr (COL) *reinterpret_cast<uint4*>(tile + lr * kMxTPitch + pcol * 2) = raw[p];
      if constexpr (DBIAS) {
        float v[8];
        unpack16<uint16_t>(raw[p], v);
#pragma unroll
        for (int j = 0; j < 8; ++j) cs[j] = __fadd_rn(cs[j], v[j]);
      }
      if constexpr (ROW) {
        uint32_t m = absmax_bits<uint16_t>(0u, raw[p]);
        m = max(m & 0xffffu, m >> 16);
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0xb1, 0xf, 0xf, false)));
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x4e, 0xf, 0xf, false)));
        const int64_t r = r0 + lr;
        uint32_t code;
        if constexpr (FP4) {
          const bool nan = m > 0x7f80u;
          const int e = nan ? 0 : mx4_exponent(m << 16);
          float v[8];
          unpack16<uint16_t>(raw[p], v);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = __builtin_ldexpf(v[j], -e);
          *reinterpret_cast<uint32_t*>(out_row + r * (C / 2) + (c0 + pcol) / 2) =
              nan ? e2m1_pack8_slow(v) : e2m1_pack8(v);
          code = nan ? 255u : static_cast<uint32_t>(e + 127);
        } else {
          const int e = mx_exponent<E5M2>(__uint_as_float(m << 16));
          uint32_t q0, q1;
          if (m < 0x7f80u && e > -127) mx_quant8_scaled<E5M2>(raw[p], e, q0, q1);
          else mx_quant8<E5M2>(raw[p], e, q0, q1);
          *reinterpret_cast<uint2*>(out_row + r * C + c0 + pcol) = make_uint2(q0, q1);
          code = static_cast<uint32_t>(e + 127);
        }
        const uint32_t k1 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x104, 0xf, 0xf, true));
        const uint32_t k2 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x108, 0xf, 0xf, true));
        const uint32_t k3 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x10c, 0xf, 0xf, true));
        if ((lane & 15) == 0)
          *scale_dw(scale_row, r, C, c0) = code | (k1 << 8) | (k2 << 16) | (k3 << 24);
      }
      if constexpr (!COL) {
        if (has1) raw[p] = load1(p, r1, c1);
      }
    }
    if constexpr (COL) {
      if (has1) {
#pragma unroll
        for (int p = 0; p < NP; ++p) raw[p] = load1(p, r1, c1);
      }
    }
    if constexpr (DBIAS) {  // one partial per (tile row, column): lane groups in order
#pragma unroll
      for (int j = 0; j < 8; ++j) red[prow * kCT + pcol + j] = cs[j];
      __syncthreads();
      if (t < kCT) {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < RPP; ++g) acc = __fadd_rn(acc, red[g * kCT + t]);
        dbias_part[(r0 / kCT) * C + c0 + t] = acc;
      }
    }
    if constexpr (COL) {
      __syncthreads();
      const int cp = t & 63, blk = t >> 6;
      uint32_t d[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) d[k] = *reinterpret_cast<const uint32_t*>(tile + (32 * blk + k) * kMxTPitch + 4 * cp);
      uint32_t mm = 0u;
#pragma unroll
      for (int k = 0; k < 32; ++k) mm = absmax_bits<uint16_t>(mm, make_uint4(d[k], 0u, 0u, 0u));
      if constexpr (FP4) {
        uint32_t q[2][4], code[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // h = 0: column 2cp (low halves), 1: column 2cp + 1
          const uint32_t m = h ? (mm >> 16) : (mm & 0xffffu);
          const bool nan = m > 0x7f80u;
          const int e = nan ? 0 : mx4_exponent(m << 16);
          code[h] = nan ? 255u : static_cast<uint32_t>(e + 127);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t b = h ? (d[8 * g + j] & 0xffff0000u) : (d[8 * g + j] << 16);
              w[j] = __builtin_ldexpf(__uint_as_float(b), -e);
            }
            q[h][g] = nan ? e2m1_pack8_slow(w) : e2m1_pack8(w);
          }
        }
        // stage the packed column blocks (Q[col][row / 2], pitch 80) and the codes, then
        // write each column's 64 bytes and one code dword per column
        __syncthreads();  // every thread has read its column pair
        uint8_t* qt = tile;
        uint8_t* qs = tile + kCT * kMx4QPitch;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          *reinterpret_cast<uint4*>(qt + (2 * cp + h) * kMx4QPitch + 16 * blk) =
              make_uint4(q[h][0], q[h][1], q[h][2], q[h][3]);
          qs[(2 * cp + h) * 4 + blk] = static_cast<uint8_t>(code[h]);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = (t >> 2) + 64 * k, chunk = t & 3;
          const uint4 v = *reinterpret_cast<const uint4*>(qt + c * kMx4QPitch + 16 * chunk);
          *reinterpret_cast<uint4*>(out_col + (c0 + c) * (R / 2) + r0 / 2 + 16 * chunk) = v;
        }
        if (t < kCT)
          *scale_dw(scale_col, c0 + t, R, r0) = *reinterpret_cast<const uint32_t*>(qs + 4 * t);
        return;
      }
      uint32_t q[2][8];
      int e[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // h = 0: column 2cp (low halves), 1: column 2cp + 1
        const uint32_t m = h ? (mm >> 16) : (mm & 0xffffu);
        e[h] = mx_exponent<E5M2>(__uint_as_float(m << 16));
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          float w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t b = h ? (d[4 * g + j] & 0xffff0000u) : (d[4 * g + j] << 16);
            w[j] = saturate<E5M2>(__builtin_ldexpf(__uint_as_float(b), -e[h]));
          }
          q[h][g] = cvt4<E5M2>(w[0], w[1], w[2], w[3]);
        }
      }
      // Stage the transposed bytes (Q[col][row], pitch 144) and the codes (one dword
      // of four blocks per column) in the tile's LDS, then write whole 128-byte lines
      // of out_col and one code dword per column.
      __syncthreads();  // every thread has read its column pair
      uint8_t* qt = tile;
      uint8_t* qs = tile + kCT * kMxQPitch;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint4* dst = reinterpret_cast<uint4*>(qt + (2 * cp + h) * kMxQPitch + 32 * blk);
        dst[0] = make_uint4(q[h][0], q[h][1], q[h][2], q[h][3]);
        dst[1] = make_uint4(q[h][4], q[h][5], q[h][6], q[h][7]);
        qs[(2 * cp + h) * 4 + blk] = static_cast<uint8_t>(e[h] + 127);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = (t >> 3) + 32 * k, chunk = t & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(qt + c * kMxQPitch + 16 * chunk);
        *reinterpret_cast<uint4*>(out_col + (c0 + c) * R + r0 + 16 * chunk) = v;
      }
      if (t < kCT)
        *scale_dw(scale_col, c0 + t, R, r0) = *reinterpret_cast<const uint32_t*>(qs + 4 * t);
    }
  };
  int64_t i = blockIdx.x;
  if (i >= ntiles) return;
  uint4 raw[NP];
  int64_t r0, c0;
  origin(i, r0, c0);
#pragma unroll
  for (int p = 0; p < NP; ++p) raw[p] = load1(p, r0, c0);
  for (;;) {
    const int64_t i1 = i + gridDim.x;
    const bool has1 = i1 < ntiles;
    int64_t r1 = 0, c1 = 0;
    if (has1) origin(i1, r1, c1);
    process(raw, r0, c0, has1, r1, c1);
    if (!has1) break;
    i = i1;
    r0 = r1;
    c0 = c1;
  }
}

// ----------------------------------------------------------------------------
// The FP4 recipe steps around MXFP4 ([LP-opt] "実モデルにおける結果の解釈": a random
// Hadamard transform of the Wgrad inputs, stochastic rounding of gradients, 2D block
// scaling of weights).  bf16 input of whole 128 x 128 tiles, E8M0 scales in the panel
// layout the GEMM loads (same tile walk and staging as k_mxfp8_tiles).
//
// Hadamard transform (column copy only: along the rows, which are the Wgrad reduction
// axis): per 16 consecutive rows, y = (1/4) H16 diag(s) x with s from a 16-bit sign mask;
// the sum is formed by the fast transform's butterflies in fp64 (pairs i, i + h for h =
// 1, 2, 4, 8) and rounded once to fp32 after the exact scaling by 1/4.
//
// Stochastic rounding: the random 16-bit integer of element i (row-major index in the
// copy written) is lane i % 16 of Philox4x64-10 with counter (i / 16, copy, 0, 0) and key
// (seed, 0); lane l is bits 16 (l % 4) .. of output word l / 4.  A scaled magnitude
// between neighbouring E2M1 magnitudes lo <= a < hi rounds up iff r < 65536 (a - lo) /
// (hi - lo); every step of that test is exact in fp32.
// ----------------------------------------------------------------------------
// the 128-bit product m b as (hi, lo): four 32 x 32 -> 64 multiply-adds (v_mad_u64_u32),
// each partial sum below 2^64, and one 64-bit add
__device__ __forceinline__ void mulhilo64(uint64_t m, uint64_t b, uint64_t& lo, uint64_t& hi) {
  const uint32_t m0 = static_cast<uint32_t>(m), m1 = static_cast<uint32_t>(m >> 32);
  const uint32_t b0 = static_cast<uint32_t>(b), b1 = static_cast<uint32_t>(b >> 32);
  const uint64_t p00 = static_cast<uint64_t>(m0) * b0;
  const uint64_t p01 = static_cast<uint64_t>(m0) * b1 + (p00 >> 32);
  const uint64_t p10 = static_cast<uint64_t>(m1) * b0 + static_cast<uint32_t>(p01);
  const uint64_t p11 = static_cast<uint64_t>(m1) * b1 + (p01 >> 32);
  lo = (p10 << 32) | static_cast<uint32_t>(p00);
  hi = p11 + (p10 >> 32);
}

__device__ __forceinline__ void philox4x64_10(uint64_t& c0, uint64_t& c1, uint64_t& c2, uint64_t& c3, uint64_t k0,
                                              uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t lo0, hi0, lo1, hi1;
    mulhilo64(M0, c0, lo0, hi0);
    mulhilo64(M1, c2, lo1, hi1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

// the 16 random 16-bit integers of call `call` of copy `copy` (lane l: r[l / 4] >> 16 (l % 4))
__device__ __forceinline__ void sr_call(uint64_t call, uint32_t copy, uint64_t seed, uint64_t (&r)[4]) {
  r[0] = call;
  r[1] = copy;
  r[2] = 0;
  r[3] = 0;
  philox4x64_10(r[0], r[1], r[2], r[3], seed, 0);
}

// E2M1 code of an already scaled value y, rounded stochastically with the 16-bit r16;
// saturates at 6, keeps the sign, NaN -> +0.  Without branches: the magnitudes are
// spaced w = 0.5 below 2, 1 in [2, 4) and 2 in [4, 6], so t = a / w (exact) has
// floor(t) = the lower neighbour in units of w and t - floor(t) = (a - lo) / (hi - lo)
// (exact); the code is floor(t) + up, plus 2 for each of the bounds 2 and 4 that a
// passes (0.5 ... 2 are codes 1 ... 4; 3, 4 are codes 5, 6; 6 is code 7).
__device__ __forceinline__ uint32_t e2m1_sr_code(float y, uint32_t r16) {
  const float a = __builtin_fminf(__builtin_fabsf(y), 6.0f);
  const bool ge2 = a >= 2.0f, ge4 = a >= 4.0f;
  const float t = __fmul_rn(a, ge4 ? 0.5f : (ge2 ? 1.0f : 2.0f));
  const float fl = __builtin_floorf(t);
  const uint32_t up = static_cast<float>(r16) < __fmul_rn(__fsub_rn(t, fl), 65536.0f);
  const uint32_t c = static_cast<uint32_t>(fl) + up + (ge2 ? 2u : 0u) + (ge4 ? 2u : 0u);
  const uint32_t keep = 0u - static_cast<uint32_t>(y == y);  // all ones unless NaN
  return (c | ((__float_as_uint(y) >> 31) << 3)) & keep;
}

// in place: v[0..15] <- fl32((1/4) H16 diag(s) v), fp64 butterflies
__device__ __forceinline__ void rht16(float* v, uint32_t sign_mask) {
  double t[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] = ((sign_mask >> j) & 1u) ? -static_cast<double>(v[j]) : static_cast<double>(v[j]);
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const double a = t[i], b = t[i + h];
        t[i] = __dadd_rn(a, b);
        t[i + h] = __dsub_rn(a, b);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = static_cast<float>(t[j] * 0.25);
}

// the value of the other lane of the pair (2k, 2k + 1)
__device__ __forceinline__ uint64_t swap_lane_pairs64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(v)), 0xb1, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(v >> 32)), 0xb1, 0xf, 0xf, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

struct Mx4Recipe {
  uint32_t sign_mask;  // Hadamard signs of the column copy
  uint64_t seed;       // stochastic rounding key
};

// 8 scaled values -> one dword of codes (value j in nibble j): round to nearest even, or
// stochastically with the random integers of 8 consecutive lanes, the four 16-bit lanes
// of w0 then those of w1
template <bool SR>
__device__ __forceinline__ uint32_t mx4_pack8(const float* w, bool nan, uint64_t w0, uint64_t w1) {
  if constexpr (SR) {
    uint32_t d = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t word = j < 4 ? w0 : w1;
      d |= e2m1_sr_code(w[j], static_cast<uint32_t>(word >> (16 * (j & 3))) & 0xffffu) << (4 * j);
    }
    return d;
  } else {
    return nan ? e2m1_pack8_slow(w) : e2m1_pack8(w);
  }
}

template <bool ROW, bool COL, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void k_mxfp4_recipe(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ out_row,
                                                           uint8_t* __restrict__ scale_row,
                                                           uint8_t* __restrict__ out_col,
                                                           uint8_t* __restrict__ scale_col, Mx4Recipe rc) {
  auto scale_dw = [](uint8_t* base, int64_t r, int64_t cols, int64_t c0) {
    return reinterpret_cast<uint32_t*>(base) + ((r >> 8) * (cols >> 7) + (c0 >> 7)) * 256 + (r & 255);
  };
  constexpr int NP = 8, RPP = 16;
  __shared__ __attribute__((aligned(16))) uint8_t tile[COL ? kCT * kMxTPitch : 16];
  const int64_t ntc = C / kCT;
  const int64_t ntiles = ntc * (R / kCT);
  const int t = threadIdx.x, lane = t & 63;
  const int prow = t >> 4, pcol = (t & 15) * 8;
  const uint32_t ld_off = static_cast<uint32_t>((prow * C + pcol) * 2);
  const uint32_t ld_pass = static_cast<uint32_t>(RPP * C * 2);
  auto origin = [&](int64_t i, int64_t& r0, int64_t& c0) {
    r0 = (i / ntc) * kCT;
    c0 = (i % ntc) * kCT;
  };
  auto load1 = [&](int p, int64_t r0, int64_t c0) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(x + r0 * C + c0);
    return load_stream(base + ld_off + p * ld_pass);
  };
  auto process = [&](uint4 (&raw)[NP], int64_t r0, int64_t c0, bool has1, int64_t r1, int64_t c1) {
    if constexpr (COL) __syncthreads();
    static_assert(NP % 2 == 0, "the stochastic-rounding row path pairs passes");
    uint64_t nw0 = 0, nw1 = 0;  // stochastic rounding: this lane's words for the odd pass
#pragma clang loop unroll(full)
    for (int p = 0; p < NP; ++p) {
      const int lr = p * RPP + prow;
      if constexpr (COL) *reinterpret_cast<uint4*>(tile + lr * kMxTPitch + pcol * 2) = raw[p];
      if constexpr (ROW) {
        uint32_t m = absmax_bits<uint16_t>(0u, raw[p]);
        m = max(m & 0xffffu, m >> 16);
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0xb1, 0xf, 0xf, false)));
        m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x4e, 0xf, 0xf, false)));
        const int64_t r = r0 + lr;
        const bool nan = m > 0x7f80u;
        const int e = nan ? 0 : mx4_exponent(m << 16);
        float v[8];
        unpack16<uint16_t>(raw[p], v);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_ldexpf(v[j], -e);
        uint64_t w0 = 0, w1 = 0;
        if constexpr (SR) {
          // Lanes 2k and 2k + 1 hold the two halves (elements 0..7: words 0, 1; 8..15:
          // words 2, 3) of one Philox call per pass, so each lane computes one call per
          // two passes: the even lane the call of pass p, the odd lane that of pass p + 1,
          // and each hands the other the two words it needs (a DPP swap of lane pairs).
          if ((p & 1) == 0) {
            const bool odd = lane & 1;
            const int64_t rq = r0 + (p + (odd ? 1 : 0)) * RPP + prow;
            uint64_t a0 = static_cast<uint64_t>((rq * C + c0 + pcol) >> 4), a1 = 0, a2 = 0, a3 = 0;
            philox4x64_10(a0, a1, a2, a3, rc.seed, 0);
            const uint64_t x0 = swap_lane_pairs64(odd ? a0 : a2), x1 = swap_lane_pairs64(odd ? a1 : a3);
            w0 = odd ? x0 : a0;
            w1 = odd ? x1 : a1;
            nw0 = odd ? a2 : x0;
            nw1 = odd ? a3 : x1;
          } else {
            w0 = nw0;
            w1 = nw1;
          }
        }
        *reinterpret_cast<uint32_t*>(out_row + r * (C / 2) + (c0 + pcol) / 2) = mx4_pack8<SR>(v, nan, w0, w1);
        const uint32_t code = nan ? 255u : static_cast<uint32_t>(e + 127);
        const uint32_t k1 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x104, 0xf, 0xf, true));
        const uint32_t k2 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x108, 0xf, 0xf, true));
        const uint32_t k3 = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(code), 0x10c, 0xf, 0xf, true));
        if ((lane & 15) == 0) *scale_dw(scale_row, r, C, c0) = code | (k1 << 8) | (k2 << 16) | (k3 << 24);
      }
      if constexpr (!COL) {
        if (has1) raw[p] = load1(p, r1, c1);
      }
    }
    if constexpr (COL) {
      if (has1) {
#pragma unroll
        for (int p = 0; p < NP; ++p) raw[p] = load1(p, r1, c1);
      }
      __syncthreads();
      const int cp = t & 63, blk = t >> 6;
      uint32_t q[2][4], code[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // h = 0: column 2cp (low halves), 1: column 2cp + 1
        float v[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(tile + (32 * blk + k) * kMxTPitch + 4 * cp);
          v[k] = __uint_as_float(h ? (d & 0xffff0000u) : (d << 16));
        }
        if constexpr (RHT) {
          rht16(v, rc.sign_mask);
          rht16(v + 16, rc.sign_mask);
        }
        uint32_t mb = 0u;
#pragma unroll
        for (int k = 0; k < 32; ++k) mb = max(mb, __float_as_uint(v[k]) & 0x7fffffffu);
        const bool nan = mb > 0x7f800000u;
        const int e = nan ? 0 : mx4_exponent(mb);
        code[h] = nan ? 255u : static_cast<uint32_t>(e + 127);
        const int64_t c = c0 + 2 * cp + h;
        const int64_t i0 = c * R + r0 + 32 * blk;  // column copy: element index of v[0] (a multiple of 32)
        uint64_t ra[4] = {0, 0, 0, 0}, rb[4] = {0, 0, 0, 0};
        if constexpr (SR) {
          sr_call(static_cast<uint64_t>(i0 >> 4), 1u, rc.seed, ra);
          sr_call(static_cast<uint64_t>(i0 >> 4) + 1, 1u, rc.seed, rb);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float w[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = __builtin_ldexpf(v[8 * g + j], -e);
          const uint64_t* rw = g < 2 ? ra : rb;  // lanes 8 (g % 2) .. of the call
          q[h][g] = mx4_pack8<SR>(w, nan, rw[2 * (g & 1)], rw[2 * (g & 1) + 1]);
        }
      }
      __syncthreads();  // every thread has read its column pair
      uint8_t* qt = tile;
      uint8_t* qs = tile + kCT * kMx4QPitch;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        *reinterpret_cast<uint4*>(qt + (2 * cp + h) * kMx4QPitch + 16 * blk) = make_uint4(q[h][0], q[h][1], q[h][2], q[h][3]);
        qs[(2 * cp + h) * 4 + blk] = static_cast<uint8_t>(code[h]);
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = (t >> 2) + 64 * k, chunk = t & 3;
        const uint4 vv = *reinterpret_cast<const uint4*>(qt + c * kMx4QPitch + 16 * chunk);
        *reinterpret_cast<uint4*>(out_col + (c0 + c) * (R / 2) + r0 / 2 + 16 * chunk) = vv;
      }
      if (t < kCT) *scale_dw(scale_col, c0 + t, R, r0) = *reinterpret_cast<const uint32_t*>(qs + 4 * t);
    }
  };
  int64_t i = blockIdx.x;
  if (i >= ntiles) return;
  uint4 raw[NP];
  int64_t r0, c0;
  origin(i, r0, c0);
#pragma unroll
  for (int p = 0; p < NP; ++p) raw[p] = load1(p, r0, c0);
  for (;;) {
    const int64_t i1 = i + gridDim.x;
    const bool has1 = i1 < ntiles;
    int64_t r1 = 0, c1 = 0;
    if (has1) origin(i1, r1, c1);
    process(raw, r0, c0, has1, r1, c1);
    if (!has1) break;
    i = i1;
    r0 = r1;
    c0 = c1;
  }
}

// 2D block scaling of weights: one E8M0 scale per 32 x 32 sub-tile, the MXFP4 rule on
// the sub-tile's amax; the row copy repeats it for each row's block and the column copy
// (the transpose) for each column's block, so both copies hold the same codes.  ROW /
// COL: which copies the launch writes.  The tile
// goes through LDS; thread t finds the amax of sub-tile t / 16 over two of its rows per
// lane group (16 lanes, xor-reduced), then quantizes like k_mxfp4_recipe's row and
// column paths with the sub-tile exponents.
template <bool ROW, bool COL>
__global__ __launch_bounds__(kThreads) void k_mxfp4_2d(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                       uint8_t* __restrict__ out_row, uint8_t* __restrict__ scale_row,
                                                       uint8_t* __restrict__ out_col, uint8_t* __restrict__ scale_col) {
  auto scale_dw = [](uint8_t* base, int64_t r, int64_t cols, int64_t c0) {
    return reinterpret_cast<uint32_t*>(base) + ((r >> 8) * (cols >> 7) + (c0 >> 7)) * 256 + (r & 255);
  };
  constexpr int NP = 8, RPP = 16;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kCT * kMxTPitch];
  __shared__ int sub_e[16];
  __shared__ uint32_t sub_m[16];
  const int64_t ntc = C / kCT;
  const int64_t ntiles = ntc * (R / kCT);
  const int t = threadIdx.x, lane = t & 63;
  const int prow = t >> 4, pcol = (t & 15) * 8;
  for (int64_t i = blockIdx.x; i < ntiles; i += gridDim.x) {
    const int64_t r0 = (i / ntc) * kCT, c0 = (i % ntc) * kCT;
    uint4 raw[NP];
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      raw[p] = load_stream(x + (r0 + p * RPP + prow) * C + c0 + pcol);
      *reinterpret_cast<uint4*>(tile + (p * RPP + prow) * kMxTPitch + pcol * 2) = raw[p];
    }
    __syncthreads();
    {  // sub-tile (st / 4, st % 4): lanes 16 st .. 16 st + 15, lane j reads rows 2j, 2j + 1
      const int st = t >> 4, j = t & 15;
      const int sr = (st >> 2) * 32 + 2 * j, sc = (st & 3) * 32;
      uint32_t m = 0u;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          m = absmax_bits<uint16_t>(m, *reinterpret_cast<const uint4*>(tile + (sr + rr) * kMxTPitch + (sc + 8 * q) * 2));
      m = max(m & 0xffffu, m >> 16);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 16)));
      if (j == 0) {
        sub_m[st] = m;
        sub_e[st] = m > 0x7f80u ? 0 : mx4_exponent(m << 16);
      }
    }
    __syncthreads();
    // row copy: the lane's 8 elements of row lr, sub-tile (lr / 32, pcol / 32)
#pragma unroll
    for (int p = 0; p < (ROW ? NP : 0); ++p) {
      const int lr = p * RPP + prow;
      const int st = (lr >> 5) * 4 + (pcol >> 5);
      const bool nan = sub_m[st] > 0x7f80u;
      const int e = sub_e[st];
      float v[8];
      unpack16<uint16_t>(raw[p], v);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) v[jj] = __builtin_ldexpf(v[jj], -e);
      const int64_t r = r0 + lr;
      *reinterpret_cast<uint32_t*>(out_row + r * (C / 2) + (c0 + pcol) / 2) = nan ? e2m1_pack8_slow(v) : e2m1_pack8(v);
      if ((lane & 15) == 0) {
        uint32_t dw = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int sb = (lr >> 5) * 4 + b;
          dw |= (sub_m[sb] > 0x7f80u ? 255u : static_cast<uint32_t>(sub_e[sb] + 127)) << (8 * b);
        }
        *scale_dw(scale_row, r, C, c0) = dw;
      }
    }
    if constexpr (!COL) continue;
    // column copy: columns 2cp, 2cp + 1 over rows 32 blk .. + 31 (sub-tile (blk, cp / 16))
    const int cp = t & 63, blk = t >> 6;
    const int st = blk * 4 + (cp >> 4);
    const bool nan = sub_m[st] > 0x7f80u;
    const int e = sub_e[st];
    const uint32_t code = nan ? 255u : static_cast<uint32_t>(e + 127);
    uint32_t q[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(tile + (32 * blk + 8 * g + jj) * kMxTPitch + 4 * cp);
          w[jj] = __builtin_ldexpf(__uint_as_float(h ? (d & 0xffff0000u) : (d << 16)), -e);
        }
        q[h][g] = nan ? e2m1_pack8_slow(w) : e2m1_pack8(w);
      }
    }
    __syncthreads();  // every thread has read its column pair
    uint8_t* qt = tile;
    uint8_t* qs = tile + kCT * kMx4QPitch;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(qt + (2 * cp + h) * kMx4QPitch + 16 * blk) = make_uint4(q[h][0], q[h][1], q[h][2], q[h][3]);
      qs[(2 * cp + h) * 4 + blk] = static_cast<uint8_t>(code);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = (t >> 2) + 64 * k, chunk = t & 3;
      const uint4 vv = *reinterpret_cast<const uint4*>(qt + c * kMx4QPitch + 16 * chunk);
      *reinterpret_cast<uint4*>(out_col + (c0 + c) * (R / 2) + r0 / 2 + 16 * chunk) = vv;
    }
    if (t < kCT) *scale_dw(scale_col, c0 + t, R, r0) = *reinterpret_cast<const uint32_t*>(qs + 4 * t);
  }
}

// Blocks of `kernel` (kThreads threads) that fit at once on one compute unit, and the
// compute units of the current device, asked of the runtime at every launch (the
// library keeps no cache of them).
std::pair<int, int> occupancy(const void* kernel) {
  int dev = 0, per_cu = 1, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess) return {1, 256};
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  return {per_cu, cus};
}

// Persistent grid: one block per `per_block` work units, at most max_per_cu resident
// blocks per compute unit.
int persistent_grid(const void* kernel, int64_t units, int64_t per_block, int max_per_cu) {
  int64_t g = (units + per_block - 1) / per_block;
  const auto oc = occupancy(kernel);
  const int64_t cap = std::min<int64_t>(static_cast<int64_t>(std::min(oc.first, max_per_cu)) * oc.second,
                                       kAmaxMaxBlocks);
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

// Resident blocks per compute unit for each persistent kernel, measured on the
// 5B-layer tensors: four blocks per CU stream best for the flat cast and the
// cast-transpose (their input read with nontemporal loads), two for the row-wise MX
// copy; the column-wise MX copy, which spends more time per tile in LDS, prefers a
// full CU.  LayerNorm: up to four blocks of four rows (one per wave, each with its next
// row in flight); its registers allow two.
constexpr int kCapFlat = 4;
constexpr int kCapCT = 4;
constexpr int kCapMxRow = 2;
constexpr int kCapMxCol = 8;
constexpr int kCapLn = 4;

template <typename T, bool E5M2, int MODE>
void launch_flat(const T* x, int64_t n, int margin, float* scale, float* scale_inv, float* amax,
                 uint8_t* out, AmaxWork* work, int flags, hipStream_t st) {
  const auto fn = k_amax_cast<T, E5M2, MODE>;
  const int g = persistent_grid(reinterpret_cast<const void*>(fn), (n / (16 / static_cast<int64_t>(sizeof(T)))) / kFlatU, kThreads, kCapFlat);
  hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, st, x, n, scale, scale_inv, amax, out, margin, work, flags);
}

// mode: 0 delayed (one pass: amax + cast with *scale), 1 current (amax pass, then the
// cast pass with the scale from it), 2 current with the amax already in *amax (the cast
// pass only).
template <typename T, bool E5M2>
hipError_t amax_cast_t(const T* x, int64_t n, int mode, int margin, float* scale, float* scale_inv, float* amax,
                       uint8_t* out, AmaxWork* w, hipStream_t st) {
  if (mode == 0) {
    if (out) launch_flat<T, E5M2, 0>(x, n, margin, scale, scale_inv, amax, out, w, kPublishInv, st);
    else launch_flat<T, E5M2, 1>(x, n, margin, scale, scale_inv, amax, out, w, kPublishInv, st);
    return hipGetLastError();
  }
  if (mode == 1) launch_flat<T, E5M2, 1>(x, n, margin, scale, scale_inv, amax, out, w, 0, st);
  if (out)
    launch_flat<T, E5M2, 2>(x, n, margin, scale, scale_inv, amax, out, w, 0, st);
  else
    hipLaunchKernelGGL(k_current_scale, dim3(1), dim3(1), 0, st, amax, scale, scale_inv, Fp8Traits<E5M2>::max,
                       margin);
  return hipGetLastError();
}

template <typename T, bool E5M2, int MODE, bool DBIAS>
void ct_launch(const T* x, int64_t R, int64_t C, int margin, float* scale, float* scale_inv,
               float* amax, uint8_t* out_row, uint8_t* out_col, AmaxWork* work, int flags, float* part,
               hipStream_t st) {
  const int64_t whole = ct_vec_ok<T>(R, C) ? (R / kCT) * (C / kCT) : 0;
  const int64_t ragged = ((R + kCT - 1) / kCT) * ((C + kCT - 1) / kCT) - whole;
  if (whole > 0) {
    const auto fn = k_cast_transpose<T, E5M2, MODE, true, DBIAS>;
    const int g = persistent_grid(reinterpret_cast<const void*>(fn), whole, 1, kCapCT);
    hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, st, x, R, C, scale, scale_inv, amax, out_row,
                       out_col, margin, work, flags, part);
  }
  if (ragged > 0) {  // the edge tiles' amax joins the whole tiles'
    const auto fn = k_cast_transpose<T, E5M2, MODE, false, DBIAS>;
    const int g = persistent_grid(reinterpret_cast<const void*>(fn), ragged, 1, kCapCT);
    hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, st, x, R, C, scale, scale_inv, amax, out_row,
                       out_col, margin, work, whole > 0 ? flags | kAccAmax : flags, part);
  }
}

template <typename T, bool E5M2>
hipError_t cast_transpose_t(const T* x, int64_t R, int64_t C, int mode, int margin, float* scale, float* scale_inv,
                            float* amax, uint8_t* out_row, uint8_t* out_col, float* dbias, float* part,
                            AmaxWork* w, hipStream_t st) {
  const bool current = mode != 0;
  if (R == 0 || C == 0) {
    if (mode != 2) hipLaunchKernelGGL(k_prologue, dim3(1), dim3(1), 0, st, amax, scale, scale_inv, current ? 0 : 1);
    if (current)
      hipLaunchKernelGGL(k_current_scale, dim3(1), dim3(1), 0, st, amax, scale, scale_inv,
                         Fp8Traits<E5M2>::max, margin);
    if (dbias != nullptr && C > 0)  // a sum over no rows
      hipLaunchKernelGGL(k_dbias_reduce, dim3(static_cast<unsigned>((C + kDbCols - 1) / kDbCols)), dim3(256), 0, st,
                         part, int64_t{0}, C, dbias);
    return hipGetLastError();
  }
  // the row-wise copy alone is the flat cast of x
  if (out_col == nullptr && dbias == nullptr) return amax_cast_t<T, E5M2>(x, R * C, mode, margin, scale, scale_inv, amax, out_row, w, st);
  if (mode == 1) launch_flat<T, E5M2, 1>(x, R * C, margin, scale, scale_inv, amax, nullptr, w, 0, st);
  if (dbias != nullptr) {
    if (current) ct_launch<T, E5M2, 2, true>(x, R, C, margin, scale, scale_inv, amax, out_row, out_col, w, 0, part, st);
    else ct_launch<T, E5M2, 0, true>(x, R, C, margin, scale, scale_inv, amax, out_row, out_col, w, kPublishInv, part, st);
    hipLaunchKernelGGL(k_dbias_reduce, dim3(static_cast<unsigned>((C + kDbCols - 1) / kDbCols)), dim3(256), 0, st, part,
                       (R + kCT - 1) / kCT, C, dbias);
  } else {
    if (current) ct_launch<T, E5M2, 2, false>(x, R, C, margin, scale, scale_inv, amax, out_row, out_col, w, 0, nullptr, st);
    else ct_launch<T, E5M2, 0, false>(x, R, C, margin, scale, scale_inv, amax, out_row, out_col, w, kPublishInv, nullptr, st);
  }
  return hipGetLastError();
}

template <bool E5M2, bool ROW, bool COL, bool FP4 = false, bool PANEL = false, bool DBIAS = false>
void mx_tiles_launch(const uint16_t* x, int64_t R, int64_t C, uint8_t* out_row, uint8_t* scale_row,
                     uint8_t* out_col, uint8_t* scale_col, hipStream_t st, float* part = nullptr) {
  const auto fn = k_mxfp8_tiles<E5M2, ROW, COL, FP4, PANEL, DBIAS>;
  const int g = persistent_grid(reinterpret_cast<const void*>(fn), (R / kCT) * (C / kCT), 1, COL ? kCapMxCol : kCapMxRow);
  hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, st, x, R, C, out_row, scale_row, out_col, scale_col, part);
}

// part != nullptr: the bias gradient's per-tile column sums go to part [ceil(R / 128), C]
// (the caller reduces them)
template <typename T, bool E5M2>
hipError_t mxfp8_t(const T* x, int64_t R, int64_t C, uint8_t* out_row, uint8_t* scale_row,
                   uint8_t* out_col, uint8_t* scale_col, hipStream_t st, float* part = nullptr) {
  if (R == 0 || C == 0) return hipSuccess;
  // bf16 matrices of whole 128 x 128 tiles take the persistent tile kernel (32-bit
  // offsets inside a tile; the row-wise codes go out as dwords)
  if constexpr (sizeof(T) == 2) {
    const bool row = out_row != nullptr, col = out_col != nullptr;
    if (R % kCT == 0 && C % kCT == 0 && C * kCT * 2 < (int64_t{1} << 31) && R * kCT < (int64_t{1} << 31) &&
        (!row || (reinterpret_cast<uintptr_t>(scale_row) & 3u) == 0) &&
        (!col || (reinterpret_cast<uintptr_t>(scale_col) & 3u) == 0)) {
      if (part) {
        if (row && col) mx_tiles_launch<E5M2, true, true, false, false, true>(x, R, C, out_row, scale_row, out_col, scale_col, st, part);
        else if (row) mx_tiles_launch<E5M2, true, false, false, false, true>(x, R, C, out_row, scale_row, out_col, scale_col, st, part);
        else mx_tiles_launch<E5M2, false, true, false, false, true>(x, R, C, out_row, scale_row, out_col, scale_col, st, part);
      } else {
        if (row && col) mx_tiles_launch<E5M2, true, true>(x, R, C, out_row, scale_row, out_col, scale_col, st);
        else if (row) mx_tiles_launch<E5M2, true, false>(x, R, C, out_row, scale_row, out_col, scale_col, st);
        else mx_tiles_launch<E5M2, false, true>(x, R, C, out_row, scale_row, out_col, scale_col, st);
      }
      return hipGetLastError();
    }
  }
  const dim3 grid(static_cast<unsigned>((C + kTC - 1) / kTC), static_cast<unsigned>((R + kTR - 1) / kTR));
  if (part)
    hipLaunchKernelGGL((k_mxfp8<T, E5M2, true>), grid, dim3(kThreads), 0, st, x, R, C, out_row, scale_row, out_col,
                       scale_col, part);
  else
    hipLaunchKernelGGL((k_mxfp8<T, E5M2>), grid, dim3(kThreads), 0, st, x, R, C, out_row, scale_row, out_col,
                       scale_col, nullptr);
  return hipGetLastError();
}

template <typename T, typename P, bool E5M2, int MODE>
void ln_launch(const T* x, int64_t R, int64_t C, const P* g, const P* b, float eps, int margin, float* scale,
               float* sinv, float* amax, uint8_t* out, float* mu, float* rs, AmaxWork* w, int flags,
               hipStream_t st) {
  // registers per lane for a row: two 16-byte chunks for rows of up to 128 chunks, else eight
  const bool narrow = C / (16 / static_cast<int64_t>(sizeof(T))) <= 128;
  const auto fn = narrow ? k_layernorm<T, P, E5M2, MODE, 2> : k_layernorm<T, P, E5M2, MODE, kLnReg>;
  const int grid = persistent_grid(reinterpret_cast<const void*>(fn), R, kThreads / 64, kCapLn);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), 0, st, x, R, C, g, b, eps, scale, sinv, amax, out, mu, rs,
                     margin, w, flags);
}

template <typename T, typename P, bool E5M2>
hipError_t layernorm_t(const T* x, int64_t R, int64_t C, const P* g, const P* b, float eps, int current,
                       int margin, float* scale, float* sinv, float* amax, uint8_t* out, float* mu, float* rs,
                       AmaxWork* w, hipStream_t st) {
  if (R == 0) {
    hipLaunchKernelGGL(k_prologue, dim3(1), dim3(1), 0, st, amax, scale, sinv, current ? 0 : 1);
    if (current)
      hipLaunchKernelGGL(k_current_scale, dim3(1), dim3(1), 0, st, amax, scale, sinv, Fp8Traits<E5M2>::max,
                         margin);
    return hipGetLastError();
  }
  if (!current) {
    ln_launch<T, P, E5M2, 0>(x, R, C, g, b, eps, margin, scale, sinv, amax, out, mu, rs, w, kPublishInv, st);
  } else {
    ln_launch<T, P, E5M2, 1>(x, R, C, g, b, eps, margin, scale, sinv, amax, out, mu, rs, w, 0, st);
    ln_launch<T, P, E5M2, 2>(x, R, C, g, b, eps, margin, scale, sinv, amax, out, mu, rs, w, 0, st);
  }
  return hipGetLastError();
}

template <typename T, typename P>
hipError_t layernorm_fmt(const T* x, int64_t R, int64_t C, const P* g, const P* b, float eps, int e5m2,
                         int current, int margin, float* scale, float* sinv, float* amax, uint8_t* out,
                         float* mu, float* rs, AmaxWork* w, hipStream_t st) {
  return e5m2 ? layernorm_t<T, P, true>(x, R, C, g, b, eps, current, margin, scale, sinv, amax, out, mu, rs, w, st)
              : layernorm_t<T, P, false>(x, R, C, g, b, eps, current, margin, scale, sinv, amax, out, mu, rs, w, st);
}

}  // namespace

// ----------------------------------------------------------------------------
// Static scratch for te_cast_transpose_dbias_noalloc (callers that cannot allocate):
// the amax counters (the first kAmaxScratch bytes) and the per-tile partial sums of the
// bias gradient.  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
// ----------------------------------------------------------------------------
constexpr int64_t kAmaxScratch = sizeof(AmaxWork);
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ void k_clear_words(uint32_t* p, int n) {
  const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

hipError_t static_scratch(void** ptr, hipStream_t s) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // the counters start at zero (static storage is zero at load; cleared once more here
    // by a kernel, which a stream capture records like any other launch)
    constexpr int nw = static_cast<int>(kAmaxScratch / 4);
    hipLaunchKernelGGL(k_clear_words, dim3((nw + 255) / 256), dim3(256), 0, s, static_cast<uint32_t*>(p), nw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

hipError_t launch_amax_cast(const void* x, int x_dtype, int64_t n, int out_e5m2, int mode, int margin, float* scale,
                            float* scale_inv, float* amax, uint8_t* out, void* ws, hipStream_t s) {
  auto* w = static_cast<AmaxWork*>(ws);
  if (x_dtype == BF16)
    return out_e5m2 ? amax_cast_t<uint16_t, true>(static_cast<const uint16_t*>(x), n, mode, margin, scale, scale_inv, amax, out, w, s)
                    : amax_cast_t<uint16_t, false>(static_cast<const uint16_t*>(x), n, mode, margin, scale, scale_inv, amax, out, w, s);
  return out_e5m2 ? amax_cast_t<float, true>(static_cast<const float*>(x), n, mode, margin, scale, scale_inv, amax, out, w, s)
                  : amax_cast_t<float, false>(static_cast<const float*>(x), n, mode, margin, scale, scale_inv, amax, out, w, s);
}

hipError_t launch_cast_transpose(const void* x, int x_dtype, int64_t rows, int64_t cols, int out_e5m2, int mode,
                                 int margin, float* scale, float* scale_inv, float* amax, uint8_t* out_row,
                                 uint8_t* out_col, float* dbias, float* dbias_part, void* ws, hipStream_t s) {
  auto* w = static_cast<AmaxWork*>(ws);
  if (x_dtype == BF16)
    return out_e5m2 ? cast_transpose_t<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, mode, margin, scale, scale_inv, amax, out_row, out_col, dbias, dbias_part, w, s)
                    : cast_transpose_t<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, mode, margin, scale, scale_inv, amax, out_row, out_col, dbias, dbias_part, w, s);
  return out_e5m2 ? cast_transpose_t<float, true>(static_cast<const float*>(x), rows, cols, mode, margin, scale, scale_inv, amax, out_row, out_col, dbias, dbias_part, w, s)
                  : cast_transpose_t<float, false>(static_cast<const float*>(x), rows, cols, mode, margin, scale, scale_inv, amax, out_row, out_col, dbias, dbias_part, w, s);
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
                                 uint8_t* scale_col, hipStream_t s, float* dbias, float* part) {
  hipError_t e;
  if (x_dtype == BF16)
    e = e5m2 ? mxfp8_t<uint16_t, true>(static_cast<const uint16_t*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s, part)
             : mxfp8_t<uint16_t, false>(static_cast<const uint16_t*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s, part);
  else
    e = e5m2 ? mxfp8_t<float, true>(static_cast<const float*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s, part)
             : mxfp8_t<float, false>(static_cast<const float*>(x), rows, cols, out_row, scale_row, out_col, scale_col, s, part);
  if (e != hipSuccess || dbias == nullptr || cols == 0) return e;
  // the bias gradient: the tile partials added over tile rows in order (an empty x: zeros)
  hipLaunchKernelGGL(k_dbias_reduce, dim3(static_cast<unsigned>((cols + kDbCols - 1) / kDbCols)), dim3(256), 0, s,
                     part, (rows + kCT - 1) / kCT, cols, dbias);
  return hipGetLastError();
}

hipError_t launch_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* out_row,
                                 uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  // bf16 matrices of whole 128 x 128 tiles: the persistent tile kernel, as for MXFP8
  const bool row = out_row != nullptr, col = out_col != nullptr;
  if (x_dtype == BF16 && rows % kCT == 0 && cols % kCT == 0 && cols * kCT * 2 < (int64_t{1} << 31) &&
      rows * kCT < (int64_t{1} << 31) && (!row || (reinterpret_cast<uintptr_t>(scale_row) & 3u) == 0) &&
      (!col || (reinterpret_cast<uintptr_t>(scale_col) & 3u) == 0)) {
    const auto* xx = static_cast<const uint16_t*>(x);
    if (row && col) mx_tiles_launch<false, true, true, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
    else if (row) mx_tiles_launch<false, true, false, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
    else mx_tiles_launch<false, false, true, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((cols + kTC - 1) / kTC), static_cast<unsigned>((rows + kTR - 1) / kTR));
  if (x_dtype == BF16)
    hipLaunchKernelGGL(k_mxfp4<uint16_t>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(x), rows, cols,
                       out_row, scale_row, out_col, scale_col);
  else
    hipLaunchKernelGGL(k_mxfp4<float>, grid, dim3(kThreads), 0, s, static_cast<const float*>(x), rows, cols, out_row,
                       scale_row, out_col, scale_col);
  return hipGetLastError();
}

template <bool E5M2, bool FP4>
void mx_panel_launch(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* out_row, uint8_t* scale_row,
                     uint8_t* out_col, uint8_t* scale_col, hipStream_t s) {
  const bool row = out_row != nullptr, col = out_col != nullptr;
  if (row && col) mx_tiles_launch<E5M2, true, true, FP4, true>(x, rows, cols, out_row, scale_row, out_col, scale_col, s);
  else if (row) mx_tiles_launch<E5M2, true, false, FP4, true>(x, rows, cols, out_row, scale_row, out_col, scale_col, s);
  else mx_tiles_launch<E5M2, false, true, FP4, true>(x, rows, cols, out_row, scale_row, out_col, scale_col, s);
}

// MX quantization with the scales in the panel layout: bf16 input of whole 128 x 128
// tiles only (the caller checks), the persistent tile kernel.
hipError_t launch_mx_quantize_panel(const void* x, int64_t rows, int64_t cols, int fp4, int e5m2,
                                    uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col, uint8_t* scale_col,
                                    hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const auto* xx = static_cast<const uint16_t*>(x);
  if (fp4) mx_panel_launch<false, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
  else if (e5m2) mx_panel_launch<true, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
  else mx_panel_launch<false, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, s);
  return hipGetLastError();
}

template <bool ROW, bool COL, bool RHT, bool SR>
void mx4_recipe_launch(const uint16_t* x, int64_t R, int64_t C, uint8_t* out_row, uint8_t* scale_row, uint8_t* out_col,
                       uint8_t* scale_col, Mx4Recipe rc, hipStream_t st) {
  const auto fn = k_mxfp4_recipe<ROW, COL, RHT, SR>;
  const int g = persistent_grid(reinterpret_cast<const void*>(fn), (R / kCT) * (C / kCT), 1, COL ? kCapMxCol : kCapMxRow);
  hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, st, x, R, C, out_row, scale_row, out_col, scale_col, rc);
}

hipError_t launch_mxfp4_recipe(const void* x, int64_t rows, int64_t cols, int rht, int sr, int two_d,
                               uint32_t sign_mask, uint64_t seed, uint8_t* out_row, uint8_t* scale_row,
                               uint8_t* out_col, uint8_t* scale_col, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const auto* xx = static_cast<const uint16_t*>(x);
  if (two_d) {
    const auto fn = out_row ? (out_col ? k_mxfp4_2d<true, true> : k_mxfp4_2d<true, false>) : k_mxfp4_2d<false, true>;
    const int g = persistent_grid(reinterpret_cast<const void*>(fn), (rows / kCT) * (cols / kCT), 1, kCapMxCol);
    hipLaunchKernelGGL(fn, dim3(g), dim3(kThreads), 0, s, xx, rows, cols, out_row, scale_row, out_col, scale_col);
    return hipGetLastError();
  }
  const Mx4Recipe rc{sign_mask, seed};
  const bool row = out_row != nullptr, col = out_col != nullptr;
  if (row && col) {
    if (rht) sr ? mx4_recipe_launch<true, true, true, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s)
             : mx4_recipe_launch<true, true, true, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s);
    else sr ? mx4_recipe_launch<true, true, false, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s)
            : mx4_recipe_launch<true, true, false, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s);
  } else if (col) {
    if (rht) sr ? mx4_recipe_launch<false, true, true, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s)
             : mx4_recipe_launch<false, true, true, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s);
    else sr ? mx4_recipe_launch<false, true, false, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s)
            : mx4_recipe_launch<false, true, false, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s);
  } else {
    sr ? mx4_recipe_launch<true, false, false, true>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s)
       : mx4_recipe_launch<true, false, false, false>(xx, rows, cols, out_row, scale_row, out_col, scale_col, rc, s);
  }
  return hipGetLastError();
}

hipError_t launch_layernorm_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, const void* gamma,
                                const void* beta, int param_dtype, float eps, int out_e5m2, int current,
                                int margin, float* scale, float* scale_inv, float* amax, uint8_t* out,
                                float* mu, float* rsigma, void* ws, hipStream_t s) {
  auto* w = static_cast<AmaxWork*>(ws);
  if (x_dtype == BF16) {
    const auto* xx = static_cast<const uint16_t*>(x);
    if (param_dtype == BF16)
      return layernorm_fmt(xx, rows, cols, static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(beta),
                           eps, out_e5m2, current, margin, scale, scale_inv, amax, out, mu, rsigma, w, s);
    return layernorm_fmt(xx, rows, cols, static_cast<const float*>(gamma), static_cast<const float*>(beta), eps,
                         out_e5m2, current, margin, scale, scale_inv, amax, out, mu, rsigma, w, s);
  }
  const auto* xx = static_cast<const float*>(x);
  if (param_dtype == BF16)
    return layernorm_fmt(xx, rows, cols, static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(beta),
                         eps, out_e5m2, current, margin, scale, scale_inv, amax, out, mu, rsigma, w, s);
  return layernorm_fmt(xx, rows, cols, static_cast<const float*>(gamma), static_cast<const float*>(beta), eps,
                       out_e5m2, current, margin, scale, scale_inv, amax, out, mu, rsigma, w, s);
}

}  // namespace te
