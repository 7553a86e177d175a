// Grid-wide amax inside the launch that produces the values (a quantizer's input, a
// LayerNorm's output, a GEMM's output), with the counters in a caller-owned workspace.
//
// One atomic per block on the amax word would queue every block's update on one
// address at the end of the launch, and the word would need a zeroing launch first.
// Instead block b folds its maximum (magnitude bits; NaN, whose bits are largest,
// wins) into the max word of group b % kAmaxGroups and then arrives at that group's
// counter; the last arrival of a group folds the group max into the top max word and
// arrives at the top counter, and the last arrival there -- the last block of the
// grid -- writes *amax (the max with the value already there when `acc` is set, for a
// second launch over the same tensor).  Every word is cleared by the read that
// consumes it, so a launch that completes leaves the workspace as it found it: all
// zero.  At most 64 blocks queue on one address.
//
// Ordering: every access to the workspace is a device-scope atomic read-modify-write,
// performed where all of them are, and each arrival is issued only after the
// preceding max has returned, i.e. has been performed; so when a counter reaches its
// count, every max folded before those arrivals is already in the max word.  No
// release fence is needed, which matters: a device-scope release writes back the
// whole L2 of the XCD, and one per block costs more than the contended atomics it
// replaces.
//
// The workspace belongs to the caller (te_amax_workspace_bytes() bytes, zero before
// its first use); launches that may run at the same time must not share one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace te {

constexpr int kAmaxGroups = 32;
constexpr int kAmaxLine = 64;         // words per 256-byte line: [0] max bits, [1] arrivals
constexpr int kAmaxMaxBlocks = 4096;  // grids that reduce an amax are capped below this

struct AmaxWork {
  uint32_t grp[kAmaxGroups * kAmaxLine];
  uint32_t top[kAmaxLine];
};
static_assert(sizeof(AmaxWork) == 8448, "te_amax_workspace_bytes() documents 8448 bytes");

__device__ __forceinline__ uint32_t amax_rmw_max(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t amax_rmw_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t amax_rmw_take(uint32_t* p) {  // read and clear
  return __hip_atomic_exchange(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until the returned value of an atomic is here (it has been performed); the
// memory clobber keeps later accesses from being moved above
__device__ __forceinline__ void amax_performed(uint32_t v) {
  asm volatile("s_waitcnt vmcnt(0)" : : "v"(v) : "memory");
}

// Every block of the grid calls this exactly once, with all NTHREADS threads, after its
// last use of `red` (NTHREADS / 64 words of LDS, free for this call).  v: this thread's
// maximum magnitude as a non-negative float (or NaN).
template <int NTHREADS>
__device__ __forceinline__ void grid_amax(float v, float* amax, AmaxWork* w, bool acc, uint32_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t b = __float_as_uint(v);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) b = max(b, static_cast<uint32_t>(__shfl_xor(static_cast<int>(b), off, 64)));
  if (lane == 0) red[wid] = b;
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t mb = red[0];
#pragma unroll
  for (int i = 1; i < NTHREADS / 64; ++i) mb = max(mb, red[i]);
  const int G = static_cast<int>(gridDim.x), blk = static_cast<int>(blockIdx.x);
  const int g = blk % kAmaxGroups;
  const uint32_t members = static_cast<uint32_t>((G - 1 - g) / kAmaxGroups + 1);
  const uint32_t groups = static_cast<uint32_t>(min(G, kAmaxGroups));
  uint32_t* gw = w->grp + g * kAmaxLine;
  amax_performed(amax_rmw_max(gw, mb));
  if (amax_rmw_add(gw + 1, 1u) != members - 1) return;
  const uint32_t gm = amax_rmw_take(gw);
  amax_performed(amax_rmw_take(gw + 1));
  amax_performed(amax_rmw_max(w->top, gm));
  if (amax_rmw_add(w->top + 1, 1u) != groups - 1) return;
  uint32_t r = amax_rmw_take(w->top);
  amax_performed(amax_rmw_take(w->top + 1));
  if (acc) r = max(r, __float_as_uint(*amax));
  *amax = __uint_as_float(r);
}

}  // namespace te
