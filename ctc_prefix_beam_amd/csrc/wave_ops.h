// wave_ops.h -- wave64 building blocks for gfx950 (CDNA4): cross-lane
// shuffles of 64-bit keys, ballot compaction and a register bitonic sort.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ctcpb {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Orders this wave's memory operations: everything written before (LDS or
// global, by any lane) is visible to every lane's reads after.  Waves run in
// lockstep, so this is all the synchronisation wave-synchronous code needs.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src, 64);
  const int hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  const int lo = __shfl_xor((int)(uint32_t)v, mask, 64);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), mask, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Number of set bits of `mask` held by lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Bitonic sort of 64*E keys held E per lane (element index lane*E + e) into
// descending order.  Compare-exchanges between lanes go through shuffles,
// those inside a lane are register swaps.
template <int E>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&v)[E]) {
  const int lane = lane_id();
  constexpr int N = 64 * E;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; e++) {
          if ((e & j) == 0) {
            const int i = lane * E + e;
            const bool desc = (i & k) == 0;
            const uint64_t a = v[e], b = v[e ^ j];
            const bool sw = desc ? (a < b) : (a > b);
            v[e] = sw ? b : a;
            v[e ^ j] = sw ? a : b;
          }
        }
      } else {
        const int lj = j / E;
#pragma unroll
        for (int e = 0; e < E; e++) {
          const uint64_t p = shfl_xor_u64(v[e], lj);
          const int i = lane * E + e;
          const bool keep_max = ((i & j) == 0) == ((i & k) == 0);
          const uint64_t mx = v[e] > p ? v[e] : p;
          const uint64_t mn = v[e] > p ? p : v[e];
          v[e] = keep_max ? mx : mn;
        }
      }
    }
  }
}

// Sort buf[0..n) (n <= 256) in place, descending; entries n.. of the
// smallest power-of-two block are treated as 0.  Wave-synchronous: call
// from all 64 lanes.
__device__ __forceinline__ void wave_sort_lds(uint64_t* buf, int n) {
  const int lane = lane_id();
  if (n <= 64) {
    uint64_t v[1];
    v[0] = lane < n ? buf[lane] : 0ull;
    wave_sort_desc<1>(v);
    buf[lane] = v[0];
  } else if (n <= 128) {
    uint64_t v[2];
#pragma unroll
    for (int e = 0; e < 2; e++) v[e] = (lane * 2 + e) < n ? buf[lane * 2 + e] : 0ull;
    wave_sort_desc<2>(v);
#pragma unroll
    for (int e = 0; e < 2; e++) buf[lane * 2 + e] = v[e];
  } else {
    uint64_t v[4];
#pragma unroll
    for (int e = 0; e < 4; e++) v[e] = (lane * 4 + e) < n ? buf[lane * 4 + e] : 0ull;
    wave_sort_desc<4>(v);
#pragma unroll
    for (int e = 0; e < 4; e++) buf[lane * 4 + e] = v[e];
  }
}

}  // namespace ctcpb
