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

// Lanes i with (i & J) == 0, as a wave mask (all lanes for J = 64).
__host__ __device__ constexpr uint64_t lanes_bit_clear(int j) {
  uint64_t m = 0;
  for (int i = 0; i < 64; i++)
    if ((i & j) == 0) m |= 1ull << i;
  return m;
}

// Lanes i < n, as a wave mask.
__host__ __device__ constexpr uint64_t lanes_below_n(int n) {
  return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
}

// DPP lane moves (VALU, no LDS round trip).  Controls follow the GCN/CDNA
// DPP encoding: quad_perm, row_half_mirror, row_mirror, row_shr:n,
// row_bcast:15 and row_bcast:31.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_mov(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppXor1 = 0xb1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // reverse within 8 lanes
constexpr int kDppMirror = 0x140;       // reverse within 16 lanes
constexpr int kDppBcast15 = 0x142;      // lane 15 of each row -> next row
constexpr int kDppBcast31 = 0x143;      // lane 31 -> rows 2 and 3
constexpr int kDppWaveShl1 = 0x130;     // lane i <- lane i + 1 across the wave
__device__ __forceinline__ constexpr int dpp_row_shr(int n) { return 0x110 + n; }
__device__ __forceinline__ constexpr int dpp_row_shl(int n) { return 0x100 + n; }
__device__ __forceinline__ constexpr int dpp_row_ror(int n) { return 0x120 + n; }

// Value of lane i + 1 (0 on the last lane), both halves by one DPP move each.
__device__ __forceinline__ uint64_t wave_shl1_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, kDppWaveShl1, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kDppWaveShl1, 0xf, 0xf, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Value of lane `src` (wave-uniform), in scalar registers.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), src) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
}


// Value held by lane (lane ^ J), J in {1, 2, 4, 8, 16, 32}, without an LDS
// round trip: quad permutes for 1 and 2; for 4, a row shift each way, each
// written only to the banks (groups of 4 lanes) it serves; a rotation by 8
// within the row for 8; the gfx950 lane-swap instructions across rows (16)
// and halves (32).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = (int)v;
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, kDppXor1, 0xf, 0xf, true);
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, kDppXor2, 0xf, 0xf, true);
  } else if constexpr (J == 4) {
    // banks 0 and 2 read lane i + 4, banks 1 and 3 lane i - 4
    const int up = __builtin_amdgcn_update_dpp(0, x, dpp_row_shl(4), 0xf, 0x5, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(up, x, dpp_row_shr(4), 0xf, 0xa, false);
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(x, dpp_row_ror(8), 0xf, 0xf, true);
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(~lanes_bit_clear(16)) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(~lanes_bit_clear(32)) ? r[0] : r[1];
  }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v) {
  const uint32_t lo = xor_lane<J>((uint32_t)v);
  const uint32_t hi = xor_lane<J>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange stage of a 64-lane bitonic sort (descending overall):
// lane i keeps the larger of (own, lane i ^ J) when bit J of i equals bit K of
// i, else the smaller.  The pair is (a, b) = (own, partner) for J <= 8; for
// J = 16 and 32 the lane-swap instruction leaves the lower block's key in a
// and the upper block's in b on both sides of the pair, which serves as well
// since the kept key depends only on the pair and the lane's side.  One
// compare gives the wave mask of a > b; a scalar XOR with the stage's lane
// constant turns it into "take a", which selects both halves of the key.
template <int K, int J, typename T>
__device__ __forceinline__ T bitonic_stage(T v) {
  // lanes that keep the smaller key of their pair
  constexpr uint64_t kFlip = lanes_bit_clear(J) ^ lanes_bit_clear(K);
  T a, b;
  if constexpr (J <= 8) {
    a = v;
    if constexpr (sizeof(T) == 8) {
      b = ((uint64_t)xor_lane<J>((uint32_t)(v >> 32)) << 32) | xor_lane<J>((uint32_t)v);
    } else {
      b = xor_lane<J>(v);
    }
  } else if constexpr (sizeof(T) == 8) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    if constexpr (J == 16) {
      const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
      const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
      a = ((uint64_t)h[0] << 32) | l[0];
      b = ((uint64_t)h[1] << 32) | l[1];
    } else {
      static_assert(J == 32, "lane distance");
      const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      a = ((uint64_t)h[0] << 32) | l[0];
      b = ((uint64_t)h[1] << 32) | l[1];
    }
  } else {
    if constexpr (J == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      a = r[0];
      b = r[1];
    } else {
      static_assert(J == 32, "lane distance");
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      a = r[0];
      b = r[1];
    }
  }
  const uint64_t gt = __builtin_amdgcn_ballot_w64(a > b);
  return __builtin_amdgcn_inverse_ballot_w64(gt ^ kFlip) ? a : b;
}

// The stages of a bitonic sort over blocks of N lanes (N = 16, 32 or 64),
// each block into descending order.
template <int N, typename T>
__device__ __forceinline__ T wave_sort_blocks_desc(T v) {
  v = bitonic_stage<2, 1>(v);
  v = bitonic_stage<4, 2>(v);
  v = bitonic_stage<4, 1>(v);
  v = bitonic_stage<8, 4>(v);
  v = bitonic_stage<8, 2>(v);
  v = bitonic_stage<8, 1>(v);
  v = bitonic_stage<16, 8>(v);
  v = bitonic_stage<16, 4>(v);
  v = bitonic_stage<16, 2>(v);
  v = bitonic_stage<16, 1>(v);
  if constexpr (N >= 32) {
    v = bitonic_stage<32, 16>(v);
    v = bitonic_stage<32, 8>(v);
    v = bitonic_stage<32, 4>(v);
    v = bitonic_stage<32, 2>(v);
    v = bitonic_stage<32, 1>(v);
  }
  if constexpr (N >= 64) {
    v = bitonic_stage<64, 32>(v);
    v = bitonic_stage<64, 16>(v);
    v = bitonic_stage<64, 8>(v);
    v = bitonic_stage<64, 4>(v);
    v = bitonic_stage<64, 2>(v);
    v = bitonic_stage<64, 1>(v);
  }
  return v;
}

// Sorts one 32- or 64-bit unsigned key per lane into descending lane order.
template <typename T>
__device__ __forceinline__ T wave_sort64_desc(T v) {
  v = bitonic_stage<2, 1>(v);
  v = bitonic_stage<4, 2>(v);
  v = bitonic_stage<4, 1>(v);
  v = bitonic_stage<8, 4>(v);
  v = bitonic_stage<8, 2>(v);
  v = bitonic_stage<8, 1>(v);
  v = bitonic_stage<16, 8>(v);
  v = bitonic_stage<16, 4>(v);
  v = bitonic_stage<16, 2>(v);
  v = bitonic_stage<16, 1>(v);
  v = bitonic_stage<32, 16>(v);
  v = bitonic_stage<32, 8>(v);
  v = bitonic_stage<32, 4>(v);
  v = bitonic_stage<32, 2>(v);
  v = bitonic_stage<32, 1>(v);
  v = bitonic_stage<64, 32>(v);
  v = bitonic_stage<64, 16>(v);
  v = bitonic_stage<64, 8>(v);
  v = bitonic_stage<64, 4>(v);
  v = bitonic_stage<64, 2>(v);
  v = bitonic_stage<64, 1>(v);
  return v;
}

// The 64 largest of two sorted runs of 64 keys, a descending and b
// ascending (a lane each), in descending lane order: the half-cleaner of a
// bitonic merge keeps the larger of each pair a[l], b[l] (a bitonic sequence
// holding the 64 largest), and the last six stages order it.
__device__ __forceinline__ uint64_t wave_top64_merge(uint64_t a, uint64_t b) {
  uint64_t v = a > b ? a : b;
  v = bitonic_stage<64, 32>(v);
  v = bitonic_stage<64, 16>(v);
  v = bitonic_stage<64, 8>(v);
  v = bitonic_stage<64, 4>(v);
  v = bitonic_stage<64, 2>(v);
  v = bitonic_stage<64, 1>(v);
  return v;
}

// One key per lane sorted ascending (the complements sorted descending).
__device__ __forceinline__ uint64_t wave_sort64_asc(uint64_t v) {
  return ~wave_sort64_desc<uint64_t>(~v);
}

// Maximum over the wave, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppXor1>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppXor2>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppHalfMirror>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppMirror>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppBcast15, 0xa>(x, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp_mov<kDppBcast31, 0xc>(x, x))));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

__device__ __forceinline__ int wave_sum(int v) {
  v += dpp_mov<kDppXor1>(0, v);
  v += dpp_mov<kDppXor2>(0, v);
  v += dpp_mov<kDppHalfMirror>(0, v);
  v += dpp_mov<kDppMirror>(0, v);
  v += dpp_mov<kDppBcast15, 0xa>(0, v);
  v += dpp_mov<kDppBcast31, 0xc>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Inclusive prefix sum over the wave (row_shr within rows of 16, then row
// broadcasts carry the row totals forward).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_mov<dpp_row_shr(1)>(0, v);
  v += dpp_mov<dpp_row_shr(2)>(0, v);
  v += dpp_mov<dpp_row_shr(4)>(0, v);
  v += dpp_mov<dpp_row_shr(8)>(0, v);
  v += dpp_mov<kDppBcast15, 0xa>(0, v);
  v += dpp_mov<kDppBcast31, 0xc>(0, v);
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
