// ctcpb.hip -- batched CTC prefix beam search for gfx950 (MI355X), and the C
// ABI declared in include/ctcpb.h.
//
// Method: the page "GPU CTC Prefix Beam Search Decoder" (OASR docs).  Every
// step of its pipeline is computed here, but not with its kernels:
//
//   select_kernel   frame filter, sec. 3.5 (one block per row, ordered
//                   ballot compaction instead of a block scan).
//   decode_kernel   one workgroup per row (offline) or stream, the whole
//                   frame loop in-kernel (the idea of sec. 3.4.8).  A loader
//                   wave streams each frame's log-probabilities HBM -> LDS
//                   (16-byte global-to-LDS loads) into a ring of P+1 frame
//                   slots; P producer waves take the frames in turn:
//     - vocabulary top-K (sec. 3.3 step 0, sec. 3.4.7): the best
//       min(2W+3, 40) non-blank labels by (log-prob desc, label asc), radix threshold,
//       ballot gather and count ranking; publish the slot by an LDS flag.
//   Wave 0 runs the serial beam recursion over the published slots:
//     - step 0 seeding (sec. 3.3) from the ranked list;
//     - steps >= 1: the beam x vocab extension scores of sec. 3.4.1/3.4.2
//       are never materialised.  An ordinary label c of beam k scores
//       lp[c] + logsumexp(pb, pnb) (sec. 3.4.6), so only the ranked labels
//       plus each beam's blank and repeated-label slots can reach the top W;
//       the merge of sec. 3.4.3 folds a parent's (i, last label of j)
//       extension into child j's blank slot and removes it from i's list;
//       the top W by (score desc, k*V + c asc) is taken with a register
//       bitonic sort of the few candidates above a provable lower bound, and
//       an exactness test falls back to the full beam x vocab selection
//       whenever a label outside the ranked list could still tie or win;
//     - state update (sec. 3.4.5): new (pb, pnb), length, last label, and the
//       token store: flat double-buffered lists (sec. 3.1, 7) or pages with
//       reference-counted sharing (sec. 3.4.5 paged variant, 4.2).
//   Prefix identity for the merge is tracked structurally: every beam knows
//   which live beam is its prefix minus the last label ("parent"), derived
//   from how the winners were formed; the one case the structure cannot
//   decide (a parent prefix re-created from its own parent) is settled by a
//   32-bit prefix hash filter and an exact token comparison.
//
// Numerics: float32, one rounding per operation, no contraction; exp / log1p
// are fixed operation sequences (device_math.h).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <climits>
#include <mutex>
#include <string>

#include "../../include/ctcpb.h"
#include "device_math.h"
#include "layout.h"
#include "wave_ops.h"

namespace ctcpb {

constexpr int kMaxVocab = 16384;
constexpr int kMaxRanked = 40;            // ranked labels used per frame
constexpr int kBuf = 256;                 // candidate buffer (keys)
constexpr int kHtab = 256;   // open-addressing table of new prefixes (>= 8 x beam)
constexpr int kLdsLimit = 160 * 1024;     // LDS per CU on gfx950
constexpr int kMaxPages = 32767;          // pages per row: ids are kept as 16-bit in LDS
constexpr int kDefaultCapacity = 4096;    // streaming tokens per stream (sec. 11)

// LDS offsets computed on the host: the frame slots and everything whose size
// depends on the configuration (the fixed part is the lds namespace below).
struct LdsPlan {
  int slot_stride, slot_rank;   // frame slot: row of V floats, then the label -> rank map
  int nslot, nprod;             // slots, producer waves
  int rk, nrk;                  // ring of ranked lists (labels, then log-probs), entries
  int scr;                      // producer scratch
  int clist, clist_lds;         // flat token lists held in LDS
  int tab, ref, fstk, tail, tlen, total;
};
constexpr int kMaxSlots = 8;
constexpr int kRing = 8;   // steps of winners the store wave may lag behind

struct Params {
  Layout L;
  LdsPlan S;
  int N, max_out_len;
  int sel_mode;       // offline frame filter: 0 keep all, 1 keep none, 2 threshold
  float log_thr;
  const float* lp;
  int64_t stride_b, stride_t;
  int T;              // offline: max_T; streaming: chunk_T
  int num_rows;       // streaming: streams in the blob
  const int* seq_lengths;
  const int* rows;
  const uint8_t* speech;    // streaming: [rows of the call][T] frame flags (0 = skip), or null
  const int* start_frame;   // streaming: [rows of the call] index of the chunk's first frame,
                            // or null (the stream's own count)
  char* state;
  int* out_tokens;
  int* out_lengths;
  float* out_scores;
  int vec4;           // frame rows are 16-byte aligned and V % 4 == 0
};

// Per-row scalars kept in LDS while a row is decoded (mirrors of header fields).
enum : int {
  kScalFreeTop = 0, kScalNextFree, kScalStatus, kScalHigh, kScalLive0, kScalLive1, kScalCpl0,
  kScalCpl1, kScalPcp0, kScalPcp1, kScalFallbacks, kScalVerifies, kScalSurv, kScalWide,
  kScalCount
};

// The fixed part of the workgroup's LDS: structures whose sizes do not depend
// on the configuration, at compile-time offsets (immediate LDS addresses in
// the kernels).  The frame slots follow at lds::end.
namespace lds {
constexpr int a16(int x) { return (x + 15) & ~15; }
constexpr int buf = 0;                                  // candidate keys
constexpr int A = buf + a16(kBuf * 8);                  // per-beam values of the fallbacks
constexpr int kb = A + a16(kMaxBeam * 4);
constexpr int kc = kb + a16(kMaxBeam * 4);
constexpr int lastk = kc + a16(kMaxBeam * 4);
constexpr int offs = lastk + a16(kMaxBeam * 4);
// one entry per lane (not per beam) where lanes write without a guard: the
// entries past the beam absorb writes that have no effect
constexpr int exm = offs + a16(128 * 4);                // 2 words per beam: ranks 0..63
constexpr int exclast = exm + a16(kWave * 2 * 4);
constexpr int bslot = exclast + a16(kWave * 4);
constexpr int htab = bslot + a16(kWave * 4);
constexpr int newh = htab + a16(kHtab * 4);
constexpr int newlen = newh + a16(kMaxBeam * 4);
constexpr int nchild = newlen + a16(kMaxBeam * 4);
constexpr int childc = nchild + a16(kMaxBeam * 4);
constexpr int scal = childc + a16(kMaxBeam * kMaxBeam * 4);
constexpr int flags = scal + a16(kScalCount * 4);      // hand-off flags
constexpr int ring = flags + a16((3 * kMaxSlots + 6) * 4);  // winners ring
constexpr int soffs = ring + a16(kRing * kWave * 8);    // store-wave scratch
constexpr int slot_k = a16(kMaxRanked * 4);             // ranked labels (or log-probs) of a frame
constexpr int end = soffs + a16(128 * 4);
}  // namespace lds

struct Beam {
  int live;
  float pb, pnb, score;
  float A;        // logsumexp(pb, pnb) (NEG if dead), kept with the state
  int len, last, parent, last2;
  uint32_t h, hp;
};

constexpr int kProfBase = 32;   // header word of the first phase counter (beam wave)
constexpr int kProfSlots = 12;
constexpr int kProfExtra = 56;  // header word of the producer / store-wave counters

struct Ctx {
  Layout L;       // copied from the kernel arguments (never address-taken)
  int N, mol;
  int* out_tokens;
  int* out_lengths;
  float* out_scores;
  char* base;
  int* hdr;
  int8_t* rank;
  int* Rc;
  float* Rl;
  uint64_t* buf;
  float* A;      // per beam: logsumexp(pb, pnb) after the gap collapse (NEG if dead)
  float* kb;     // per beam: key of the blank slot (after the merge fold)
  float* kc;     // per beam: key of the repeated-label slot (NEG if none / merged away)
  int* lastk;    // per beam: last label
  int* offs;
  uint32_t* exm;
  int* exclast;
  int* bslot;
  int* htab;
  uint32_t* newh;
  int* newlen;
  int* nchild;
  int* childc;
  int* scal;
  int16_t* tab;   // paged: LDS copy of both block-table parities (page ids fit 15 bits)
  int* ref;
  int16_t* fstk;  // paged: free-page stack
  int* tail;      // paged: LDS mirror of each beam's partial last page, both parities
  int* tlen;      // paged: valid leading entries of each block-table row, both parities
  int* clist;     // flat: global or LDS
  int* pages;     // paged: global
  int* tdone;     // last step whose tokens the store wave has written, durably
                  // (global page / list writes complete)
  int* release;   // last frame whose slot the beam wave has handed back
  int frame;      // frame of the current step
  const float* grow;  // its log-prob row in global memory (the exact fallback)
  int* abortf;
#ifdef CTCPB_PHASE_PROF
  uint64_t prof[kProfSlots];
  uint64_t prof_t;
  uint64_t sprof[4];
  uint64_t sprof_t;
  uint64_t stat_multi;   // steps that needed the general gather
#endif
};

// Optional per-phase cycle counters (build with -DCTCPB_PHASE_PROF): the
// shader clock is read at phase boundaries and the deltas are summed into
// header words kProfBase.. of the row (a diagnostics build, not the product).
#ifdef CTCPB_PHASE_PROF
#define PROF_MARK(slot)                                                       \
  do {                                                                        \
    const uint64_t now_ = clock64();                                          \
    if (lane_id() == 0) C.prof[slot] += now_ - C.prof_t;                      \
    C.prof_t = now_;                                                          \
  } while (0)
#else
#define PROF_MARK(slot) \
  do {                  \
  } while (0)
#endif

// LDS-only ordering between the lanes of this wave (no wait on global memory).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
}

// Orders this wave's LDS accesses for the compiler only.  The LDS performs
// one wave's operations in issue order, so a read issued after a write or
// atomic of this wave (by any of its lanes) sees it without a wait for the
// write's completion.
__device__ __forceinline__ void lds_order() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
}

// Producer / consumer hand-off inside a workgroup: LDS flags written with
// release and read with acquire semantics at workgroup scope.  A wait gives up
// after kSpinLimit polls and raises the workgroup's abort flag, which every
// wave checks, so no wave can wait forever.
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ int flag_load(int* f) {
  return __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_store(int* f, int v) {
  __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Publishes data that lives only in LDS and is complete in it (the release
// above would also wait for this wave's outstanding global loads, e.g. a row
// being prefetched into another slot).  LDS operations of a wave complete in
// order, so waiting for them and then storing the flag orders the two.
__device__ __forceinline__ void flag_publish_lds(int* f, int v) {
  lds_sync();
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until *flag == target (eq) or *flag >= target (!eq); false on abort
// (abortf == nullptr: not cancelled by the abort flag, still bounded).
__device__ __forceinline__ bool spin_wait(int* flag, int target, bool eq, int* abortf) {
  for (int it = 0; it < kSpinLimit; it++) {
    const int v = flag_load(flag);
    if (eq ? v == target : v >= target) return true;
    if (abortf && flag_load(abortf)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if (abortf) flag_store(abortf, 1);
  return false;
}

template <typename TabT>
__device__ __forceinline__ int tok_at(const Ctx& C, const TabT* tab, int parity, int slot, int pos) {
  const Layout& L = C.L;
  if (!L.paged) return C.clist[((int64_t)(parity * L.W + slot)) * L.ldc + pos];
  const int page = (int)tab[(parity * L.W + slot) * L.max_lp + (pos >> L.ps_log2)];
  if (page < 0) return -1;  // only after a row ran out of pages
  return C.pages[(int64_t)page * L.ps + (pos & (L.ps - 1))];
}

// ----------------------------------------------------------------- frames --
// Asynchronous copy of a frame row from global memory straight into LDS
// (global_load_lds: lane l of each wave-wide load lands at base + 16 l, or
// base + 4 l for the 4-byte variant, so coalesced reads stay contiguous).
// The data is usable after row_fetch_wait().
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void row_fetch_async(const float* g, float* s, int V, int vec4) {
  const int lane = lane_id();
  if (vec4) {
    const int n4 = V >> 2;
    for (int i = 0; i * kWave < n4; i++) {
      const int idx = i * kWave + lane;
      if (idx < n4)
        __builtin_amdgcn_global_load_lds(g + (int64_t)idx * 4, (lds_ptr_t)(s + i * 4 * kWave), 16,
                                         0, 0);
    }
  } else {
    for (int i = 0; i * kWave < V; i++) {
      const int idx = i * kWave + lane;
      if (idx < V) __builtin_amdgcn_global_load_lds(g + idx, (lds_ptr_t)(s + i * kWave), 4, 0, 0);
    }
  }
}

__device__ __forceinline__ void row_fetch_wait() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------ generic selection --
// Keeps the best `K` (K <= 128) keys of a stream in C.buf.  Keys must be
// distinct or 0 (= no candidate).  Items are produced 64 at a time by gen(i)
// for i in [0, n); the buffer is sorted and cut back to K whenever it fills.
template <typename Gen>
__device__ __forceinline__ int stream_topk_buf(uint64_t* buf, int K, int64_t n, Gen gen) {
  const int lane = lane_id();
  uint64_t thr = comp_floor();
  int cnt = 0;
  for (int64_t base = 0; base < n; base += kWave) {
    const int64_t i = base + lane;
    const uint64_t x = i < n ? gen(i) : 0ull;
    const bool pass = x > thr;
    const uint64_t m = __ballot(pass);
    if (pass) buf[cnt + lanes_below(m)] = x;
    cnt += __popcll(m);
    if (cnt > kBuf - kWave) {
      lds_sync();
      wave_sort_lds(buf, cnt);
      lds_sync();
      cnt = cnt < K ? cnt : K;
      if (cnt == K) thr = buf[K - 1];
    }
  }
  lds_sync();
  wave_sort_lds(buf, cnt);
  lds_sync();
  return cnt < K ? cnt : K;
}

template <typename Gen>
__device__ __forceinline__ int stream_topk(const Ctx& C, int K, int64_t n, Gen gen) {
  return stream_topk_buf(C.buf, K, n, gen);
}

// ------------------------------------------------------- vocabulary top-K --
// (All LDS hand-offs inside the ranking are between lanes of the one wave,
// whose LDS operations are performed in issue order: no waits.)
// Ranks one frame (run by a producer wave): the best K non-blank labels by
// (lp desc, label asc) into Rc / Rl, rank[label] = position (-1 elsewhere).
// prevK = size of the list Rc_old of the frame this slot held before (its
// rank entries are cleared).  The row is read as groups of four labels (the LDS row is 16-byte
// aligned whatever V is; the blank and the padding past V are set to -inf
// while the frame is ranked and the blank is restored before returning):
//   1. every lane keeps the two largest group maxima it sees;
//   2. thr = a lower bound (exact to 16 bits of the key) of the K-th largest
//      of those 128 values: at least K groups, hence K labels, reach it;
//   3. the groups whose maximum reaches thr are listed;
//   4. their labels at or above thr are gathered as composite keys;
//   5. the gathered keys are ranked: sorted one per lane, or by counting
//      (broadcast LDS reads) when there are more than 64.
// Lists that do not fit the scratch fall back to a streaming top-K over the
// whole row.
constexpr int kMaxGroups = 256;   // listed groups (step 3), ints after the keys
constexpr int kMaxGather = 128;   // gathered keys (step 4)

#ifdef CTCPB_PHASE_PROF
// store-wave sub-phases: cycles since the previous mark into C.sprof[i]
#define SP_MARK(i)                                              \
  do {                                                          \
    const uint64_t now_ = clock64();                            \
    C.sprof[i] += now_ - C.sprof_t;                             \
    C.sprof_t = now_;                                           \
  } while (0)
#define RF_MARK(i)                        \
  do {                                    \
    const uint64_t now_ = clock64();      \
    rprof[i] += now_ - rprof_t;           \
    rprof_t = now_;                       \
  } while (0)
#else
#define SP_MARK(i) \
  do {             \
  } while (0)
#define RF_MARK(i) \
  do {             \
  } while (0)
#endif

__device__ __forceinline__ void rank_frame(float* row, int V, int blank, int K, int prevK,
                                           const int* Rc_old, int* Rc, float* Rl, int8_t* rank,
                                           uint64_t* scr
#ifdef CTCPB_PHASE_PROF
                                           , uint64_t (&rprof)[8]
#endif
) {
#ifdef CTCPB_PHASE_PROF
  uint64_t rprof_t = clock64();
#endif
  const int lane = lane_id();
  const float ninf = -__builtin_inff();
  for (int r = lane; r < prevK; r += kWave) rank[Rc_old[r]] = -1;
  const int n4 = (V + 3) >> 2;
  const float lpb = row[blank];
  lds_order();
  if (lane == 0) row[blank] = ninf;
  if (lane < 4 * n4 - V) row[V + lane] = ninf;
  lds_order();
  const float4* r4 = reinterpret_cast<const float4*>(row);
  constexpr int U = 8;  // groups per lane loaded before use
  RF_MARK(0);

  // 1. two largest group maxima per lane.  Rows of up to kRegRounds rounds
  // of U groups per lane (V <= 8192) keep every group maximum in registers
  // for step 3; longer rows read complete rounds at constant offsets, then
  // the last partial round with bounds, and are read again in step 3.
  constexpr int kRegRounds = 4;
  const bool in_regs = n4 <= kRegRounds * U * kWave;   // wave-uniform
  float gm[kRegRounds][U];
  float hi = ninf, lo = ninf;
  int base = 0;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kRegRounds; r++) {
      const int rb = r * U * kWave;
      if (rb < n4) {
        const bool full = rb + U * kWave <= n4;
        float4 q[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int g = rb + u * kWave + lane;
          q[u] = r4[full ? g : (g < n4 ? g : n4 - 1)];   // in bounds; masked below
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int g = rb + u * kWave + lane;
          float m = fmaxf(fmaxf(q[u].x, q[u].y), fmaxf(q[u].z, q[u].w));
          m = (full || g < n4) ? m : ninf;
          gm[r][u] = m;
          lo = __builtin_amdgcn_fmed3f(m, hi, lo);
          hi = fmaxf(hi, m);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; u++) gm[r][u] = ninf;
      }
    }
  } else {
    for (; base + U * kWave <= n4; base += U * kWave) {
      const float4* p4 = r4 + base + lane;
      float4 q[U];
#pragma unroll
      for (int u = 0; u < U; u++) q[u] = p4[u * kWave];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const float m = fmaxf(fmaxf(q[u].x, q[u].y), fmaxf(q[u].z, q[u].w));
        lo = __builtin_amdgcn_fmed3f(m, hi, lo);
        hi = fmaxf(hi, m);
      }
    }
    if (base < n4) {
      float4 q[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int g = base + u * kWave + lane;
        q[u] = r4[g < n4 ? g : n4 - 1];   // in bounds; groups past the row are masked below
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int g = base + u * kWave + lane;
        float m = fmaxf(fmaxf(q[u].x, q[u].y), fmaxf(q[u].z, q[u].w));
        m = g < n4 ? m : ninf;
        lo = __builtin_amdgcn_fmed3f(m, hi, lo);
        hi = fmaxf(hi, m);
      }
    }
  }
  const int base_tail = base;
  RF_MARK(1);
  // 2. threshold: the largest value (to 16 bits of its key: sign, exponent
  // and 7 mantissa bits, two bits per round) that at least K of the 128
  // values reach; never below -inf
  const uint32_t a = sortable(hi), b = sortable(lo);
  uint32_t thr = 0u;
  for (int bit = 30; bit >= 16; bit -= 2) {
    const uint32_t c1 = thr | (1u << bit), c2 = thr | (2u << bit), c3 = thr | (3u << bit);
    const int n1 = __popcll(__ballot(a >= c1)) + __popcll(__ballot(b >= c1));
    const int n2 = __popcll(__ballot(a >= c2)) + __popcll(__ballot(b >= c2));
    const int n3 = __popcll(__ballot(a >= c3)) + __popcll(__ballot(b >= c3));
    thr = n3 >= K ? c3 : (n2 >= K ? c2 : (n1 >= K ? c1 : thr));
  }
  const uint32_t thr_min = sortable(ninf);
  thr = thr > thr_min ? thr : thr_min;
  const float tf = __uint_as_float((thr & 0x80000000u) ? (thr & 0x7fffffffu) : ~thr);

  RF_MARK(2);
  // 3. groups reaching the threshold: a bit per group of this lane (group
  // (u0 + u) * 64 + lane at bit u0 + u), then one wave scan places every
  // lane's list
  int* gid = reinterpret_cast<int*>(scr + kMaxGather);
  uint64_t pm = 0ull;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kRegRounds; r++)
#pragma unroll
      for (int u = 0; u < U; u++) pm |= (gm[r][u] >= tf) ? (1ull << (r * U + u)) : 0ull;
  } else {
    int u0 = 0;   // bit of round base / (U * kWave), group u: u0 + u
    for (base = 0; base < base_tail; base += U * kWave, u0 += U) {
      const float4* p4 = r4 + base + lane;
      float4 q[U];
#pragma unroll
      for (int u = 0; u < U; u++) q[u] = p4[u * kWave];
      uint32_t m8 = 0u;   // this round's U bits (constant positions), then placed at u0
#pragma unroll
      for (int u = 0; u < U; u++) {
        const float m = fmaxf(fmaxf(q[u].x, q[u].y), fmaxf(q[u].z, q[u].w));
        m8 |= (m >= tf) ? (1u << u) : 0u;
      }
      pm |= (uint64_t)m8 << u0;
    }
    if (base_tail < n4) {
      float4 q[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int g = base_tail + u * kWave + lane;
        q[u] = r4[g < n4 ? g : n4 - 1];
      }
      uint32_t m8 = 0u;
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int g = base_tail + u * kWave + lane;
        const float m = fmaxf(fmaxf(q[u].x, q[u].y), fmaxf(q[u].z, q[u].w));
        m8 |= ((g < n4) & (m >= tf)) ? (1u << u) : 0u;
      }
      pm |= (uint64_t)m8 << u0;
    }
  }
  int ng;
  {
    const int cnt = __popcll(pm);
    const int incl = wave_incl_scan(cnt);
    ng = __builtin_amdgcn_readlane(incl, 63);
    int pos = incl - cnt;
    while (pm) {
      const int u = __builtin_ctzll(pm);
      pm &= pm - 1ull;
      if (pos < kMaxGroups) gid[pos] = u * kWave + lane;
      pos++;
    }
  }
  lds_order();

  RF_MARK(3);
  // 4. their labels at or above the threshold, placed the same way
  int n = 0;
  if (ng <= kMaxGroups) {
    for (int j0 = 0; j0 < ng; j0 += kWave) {
      const int j = j0 + lane;
      const bool in = j < ng;
      const int g = in ? gid[j] : 0;
      const float4 q = r4[g];
      const float xv[4] = {q.x, q.y, q.z, q.w};
      uint32_t em = 0u;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int c = 4 * g + e;
        if (in && c != blank && c < V && xv[e] >= tf) em |= 1u << e;
      }
      const int cnt = __popcll(em);
      const int incl = wave_incl_scan(cnt);
      int pos = n + incl - cnt;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        if ((em >> e) & 1u) {
          if (pos < kMaxGather)
            scr[pos] = ((uint64_t)sortable(xv[e]) << 32) | (uint32_t)(~(4 * g + e));
          pos++;
        }
      }
      n += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  lds_order();

  RF_MARK(4);
  if (ng <= kMaxGroups && n >= K && n <= kWave) {
    // 5. up to one key per lane: sort, lane r holds rank r
    const uint64_t x = wave_sort64_desc<uint64_t>(lane < n ? scr[lane] : 0ull);
    if (lane < K) {
      const int c = (int)(~(uint32_t)x);
      Rc[lane] = c;
      Rl[lane] = row[c];
      rank[c] = (int8_t)lane;
    }
  } else if (ng <= kMaxGroups && n >= K && n <= kMaxGather) {
    // 5'. more keys: rank by counting, two keys per lane
    const int n8 = (n + 7) & ~7;
    if (n + lane < n8) scr[n + lane] = 0ull;
    lds_order();
    const uint64_t x0 = lane < n ? scr[lane] : 0ull;
    const uint64_t x1 = lane + kWave < n ? scr[lane + kWave] : 0ull;
    int rk0 = 0, rk1 = 0;
    const ulonglong2* y2 = reinterpret_cast<const ulonglong2*>(scr);
    if (n <= kWave) {
      for (int j = 0; j < n8; j += 8) {
        const ulonglong2 p0 = y2[j / 2], p1 = y2[j / 2 + 1], p2 = y2[j / 2 + 2], p3 = y2[j / 2 + 3];
        rk0 += (p0.x > x0 ? 1 : 0) + (p0.y > x0 ? 1 : 0) + (p1.x > x0 ? 1 : 0) +
               (p1.y > x0 ? 1 : 0) + (p2.x > x0 ? 1 : 0) + (p2.y > x0 ? 1 : 0) +
               (p3.x > x0 ? 1 : 0) + (p3.y > x0 ? 1 : 0);
      }
    } else {
      for (int j = 0; j < n8; j += 8) {
        const ulonglong2 p0 = y2[j / 2], p1 = y2[j / 2 + 1], p2 = y2[j / 2 + 2], p3 = y2[j / 2 + 3];
        rk0 += (p0.x > x0 ? 1 : 0) + (p0.y > x0 ? 1 : 0) + (p1.x > x0 ? 1 : 0) +
               (p1.y > x0 ? 1 : 0) + (p2.x > x0 ? 1 : 0) + (p2.y > x0 ? 1 : 0) +
               (p3.x > x0 ? 1 : 0) + (p3.y > x0 ? 1 : 0);
        rk1 += (p0.x > x1 ? 1 : 0) + (p0.y > x1 ? 1 : 0) + (p1.x > x1 ? 1 : 0) +
               (p1.y > x1 ? 1 : 0) + (p2.x > x1 ? 1 : 0) + (p2.y > x1 ? 1 : 0) +
               (p3.x > x1 ? 1 : 0) + (p3.y > x1 ? 1 : 0);
      }
    }
    if (lane < n && rk0 < K) {
      const int c = (int)(~(uint32_t)x0);
      Rc[rk0] = c;
      Rl[rk0] = row[c];
      rank[c] = (int8_t)rk0;
    }
    if (lane + kWave < n && rk1 < K) {
      const int c = (int)(~(uint32_t)x1);
      Rc[rk1] = c;
      Rl[rk1] = row[c];
      rank[c] = (int8_t)rk1;
    }
  } else {
    // fallback: streaming top-K over the whole row (exact for any input)
    auto gen = [&](int64_t i) -> uint64_t {
      const int c = (int)i;
      return c == blank ? 0ull : (((uint64_t)sortable(row[c]) << 32) | (uint32_t)(~c));
    };
    const int got = stream_topk_buf(scr, K, V, gen);
    for (int r = lane; r < K; r += kWave) {
      // fewer than K orderable labels only with NaN input: pad with the blank
      const int c = r < got ? (int)(~(uint32_t)scr[r]) : blank;
      Rc[r] = c;
      Rl[r] = r < got ? row[c] : ninf;
      if (r < got) rank[c] = (int8_t)r;
    }
  }
  RF_MARK(5);
  lds_order();
  if (lane == 0) row[blank] = lpb;
  lds_order();
  RF_MARK(6);
}

// --------------------------------------------------------------- step 0 ----
__device__ __forceinline__ void first_step(const Ctx& C, Beam& b, const float* row, int g, int nR) {
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W, blank = L.blank;
  const int nb = W > 1 ? W - 1 : 1;
  const int m = nb < nR ? nb : nR;
  b.live = 0;
  b.len = 0;
  b.last = blank;
  b.parent = -1;
  b.last2 = -1;
  b.pb = b.pnb = b.score = kNeg;
  b.h = kHashEmpty;
  b.hp = 0;
  if (lane < m) {
    const int c = C.Rc[lane];
    const float key = C.Rl[lane];
    b.live = 1;
    b.len = 1;
    b.last = c;
    b.score = key;
    if (g) {
      b.pb = key;
      b.pnb = kNeg;
    } else {
      b.pb = kNeg;
      b.pnb = key;
    }
    b.h = hash_push(kHashEmpty, c);
    b.hp = kHashEmpty;
    b.parent = W > 1 ? W - 1 : -1;
  }
  if (W > 1 && lane == W - 1) {
    b.live = 1;
    b.pb = row[blank];
    b.score = row[blank];
  }
  b.A = b.live ? lse(b.pb, b.pnb) : kNeg;
}

// ------------------------------------------------------------ token stores --
// Winner of output slot `lane` (valid lanes < W): source beam k, label c, the
// source's length.  k == kSeed marks a step-0 slot (tokens = [c]).
struct Winner {
  bool valid;
  int k, c, len_k;
};
constexpr int kSeed = 0x7f;

// Candidate id (k, c) as (k << 14) | c: ordered exactly like k * V + c since
// c < V <= 2^14, and decoded without a division.
static_assert(kMaxRanked <= 64, "ranks of a frame fit one 64-bit mask");

// c ? a : b over values already computed (a select, not a branch).
template <typename T>
__device__ __forceinline__ T sel(bool c, T a, T b) {
  return c ? a : b;
}

constexpr int kIdShift = 14;
static_assert(kMaxVocab <= (1 << kIdShift), "labels must fit the id field");
__device__ __forceinline__ uint32_t cand_id(int k, int c) {
  return ((uint32_t)k << kIdShift) | (uint32_t)c;
}

// Store-wave bookkeeping kept in registers from step to step: wave-uniform
// masks, prefixes and free-page counters, and per lane its slot's lineage.
// Read from LDS when the wave starts and written back after its last step
// (the launch's epilogue and the stream state take them from there).
struct StoreState {
  uint32_t live0, live1;   // live slots of parity 0 / 1
  int pre0, pre1;          // leading part shared by every live row of parity 0 / 1
                           // (flat: tokens, paged: pages)
  int freetop, nextfree, high;   // paged: free-stack top, next never-used page, high water
  int len0, len1;          // this lane's slot (flat: row length, -1 unknown; paged: pages)
  int src0, src1;          // this lane's slot: source slot of its last fork (-1 none)
  int lab0, lab1;          // flat: the label its last fork appended (-1 none)
  int m0, m1;              // flat: which common-prefix matrix holds parity 0 / 1's
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// dst[i] = src[i] for i < n by one wave, four loads per lane in flight before
// their stores.
template <typename D, typename S>
__device__ __forceinline__ void wave_copy(D* dst, const S* src, int n) {
  const int lane = lane_id();
  for (int i = lane; i < n; i += 4 * kWave) {
    const int j1 = i + kWave, j2 = i + 2 * kWave, j3 = i + 3 * kWave;
    const S v0 = src[i], v1 = src[min(j1, n - 1)], v2 = src[min(j2, n - 1)],
            v3 = src[min(j3, n - 1)];
    dst[i] = (D)v0;
    if (j1 < n) dst[j1] = (D)v1;
    if (j2 < n) dst[j2] = (D)v2;
    if (j3 < n) dst[j3] = (D)v3;
  }
}

// The store wave's per-slot lineage and, for flat lists, the two matrices of
// common-prefix bounds at the start of a launch.  A stream's flat lists go on
// from what its previous chunk kept (the lineage and bounds describe the rows
// in its state); otherwise every row's lineage is unknown and both parities
// start on matrix 0, all zeros (a valid lower bound).  None of this is LDS
// state that the beam wave sets up, so it runs before the first hand-off and
// its loads overlap that wait.
__device__ __forceinline__ void store_state_init(const Ctx& C, StoreState& ss, bool kept) {
  const Layout& L = C.L;
  const int lane = lane_id();
  ss.len0 = ss.len1 = -1;
  ss.src0 = ss.src1 = -1;
  ss.lab0 = ss.lab1 = -1;
  ss.m0 = ss.m1 = 0;
  if (L.paged) return;
  int16_t* mats = reinterpret_cast<int16_t*>(C.tail);
  const int n = L.W * L.W;
  if (kept) {
    const char* a = C.base + L.o_sst;
    const int* len = reinterpret_cast<const int*>(a + StoreArrays::len);
    const int* src = reinterpret_cast<const int*>(a + StoreArrays::src);
    const int* lab = reinterpret_cast<const int*>(a + StoreArrays::lab);
    if (lane < kMaxBeam) {
      ss.len0 = len[lane];
      ss.len1 = len[kMaxBeam + lane];
      ss.src0 = src[lane];
      ss.src1 = src[kMaxBeam + lane];
      ss.lab0 = lab[lane];
      ss.lab1 = lab[kMaxBeam + lane];
    }
    const int16_t* gm = reinterpret_cast<const int16_t*>(a + StoreArrays::mat);
    wave_copy(mats, gm, n);   // parity 0's matrix into buffer 0, parity 1's into buffer 1
    wave_copy(mats + n, gm + kMaxBeam * kMaxBeam, n);
    ss.m1 = 1;
  } else {
    int4* z = reinterpret_cast<int4*>(C.tail);
    const int n4 = (4 * n + 15) >> 4;   // within the 16-byte aligned region
    for (int i = lane; i < n4; i += kWave) z[i] = make_int4(0, 0, 0, 0);
  }
}

// The wave-uniform part, from the LDS scalars (and the paged row lengths)
// that the beam wave sets up: read once its first step is published.
__device__ __forceinline__ void store_state_load(const Ctx& C, StoreState& ss) {
  const Layout& L = C.L;
  const int lane = lane_id();
  ss.live0 = (uint32_t)uni(C.scal[kScalLive0]);
  ss.live1 = (uint32_t)uni(C.scal[kScalLive1]);
  const int pk = L.paged ? kScalPcp0 : kScalCpl0;
  ss.pre0 = uni(C.scal[pk]);
  ss.pre1 = uni(C.scal[pk + 1]);
  ss.freetop = uni(C.scal[kScalFreeTop]);
  ss.nextfree = uni(C.scal[kScalNextFree]);
  ss.high = uni(C.scal[kScalHigh]);
  if (L.paged) {
    const bool in = lane < kMaxBeam;
    ss.len0 = in ? C.tlen[lane] : 0;
    ss.len1 = in ? C.tlen[kMaxBeam + lane] : 0;
  }
}

// After the launch's last step: the scalars back to LDS (the beam wave moves
// them to the header), paged row lengths to LDS, and a stream's flat lineage
// and bounds to its state (`keep`).
__device__ __forceinline__ void store_state_save(const Ctx& C, const StoreState& ss, bool keep) {
  const Layout& L = C.L;
  const int lane = lane_id();
  lds_order();
  if (lane == 0) {
    C.scal[kScalLive0] = (int)ss.live0;
    C.scal[kScalLive1] = (int)ss.live1;
    const int pk = L.paged ? kScalPcp0 : kScalCpl0;
    C.scal[pk] = ss.pre0;
    C.scal[pk + 1] = ss.pre1;
    C.scal[kScalFreeTop] = ss.freetop;
    C.scal[kScalNextFree] = ss.nextfree;
    C.scal[kScalHigh] = ss.high;
  }
  if (L.paged && lane < kMaxBeam) {
    C.tlen[lane] = ss.len0;
    C.tlen[kMaxBeam + lane] = ss.len1;
  }
  if (keep && !L.paged) {
    char* a = C.base + L.o_sst;
    int* len = reinterpret_cast<int*>(a + StoreArrays::len);
    int* src = reinterpret_cast<int*>(a + StoreArrays::src);
    int* lab = reinterpret_cast<int*>(a + StoreArrays::lab);
    if (lane < kMaxBeam) {
      len[lane] = ss.len0;
      len[kMaxBeam + lane] = ss.len1;
      src[lane] = ss.src0;
      src[kMaxBeam + lane] = ss.src1;
      lab[lane] = ss.lab0;
      lab[kMaxBeam + lane] = ss.lab1;
    }
    const int n = L.W * L.W;
    const int16_t* mats = reinterpret_cast<const int16_t*>(C.tail);
    int16_t* gm = reinterpret_cast<int16_t*>(a + StoreArrays::mat);
    wave_copy(gm, mats + ss.m0 * n, n);
    wave_copy(gm + kMaxBeam * kMaxBeam, mats + ss.m1 * n, n);
  }
  lds_order();
}

// Step 0 (sec. 3.3): each seeded slot holds its one label, written fresh.
__device__ __forceinline__ void store_seed(const Ctx& C, StoreState& ss, const Winner& w) {
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W;
  const bool want = w.valid && w.c != L.blank;
  ss.src0 = -1;
  ss.lab0 = want ? w.c : -1;
  if (!L.paged) {
    ss.len0 = want ? 1 : 0;
    if (want) C.clist[(int64_t)lane * L.ldc] = w.c;
  } else {
    // one fresh page per seeded label
    const uint64_t mk = __ballot(want);
    const int idx = lanes_below(mk);
    const int nw = __popcll(mk);
    const int avail = ss.freetop, nf = ss.nextfree;
    int page = kInvalidPage;
    if (want) {
      if (idx < avail) page = C.fstk[avail - 1 - idx];
      else if (nf + idx - avail < L.npages) page = nf + idx - avail;
    }
    const int pops = nw < avail ? nw : avail;
    ss.freetop = avail - pops;
    const int nn = nf + (nw - pops);
    ss.nextfree = nn < L.npages ? nn : L.npages;
    if (want) {
      if (page == kInvalidPage) {
        atomicOr(&C.scal[kScalStatus], kStatusOutOfPages);
      } else {
        C.ref[page] = 1;
        C.tab[(0 * W + lane) * L.max_lp + 0] = (int16_t)page;
        ss.len0 = 1;
        C.pages[(int64_t)page * L.ps] = w.c;
        C.tail[(0 * W + lane) * L.ps] = w.c;
      }
    }
  }
  ss.live0 = (uint32_t)__ballot(lane < W && w.valid);
  lds_order();
}

// ------------------------------------------------------------ steps >= 1 ---
// The full beam x vocab selection (exact for any input): every candidate of
// the step, from the per-beam values left in LDS and the frame's row in
// global memory (its LDS slot has been handed back), into C.buf by a
// streaming top-W.  Used when the pruned candidate set cannot be proven to
// contain the top W.  The blank and repeated-label slots go first; then the
// ordinary labels beam by beam, in slot order (slots are ranked, so the
// beams' scores mostly decrease), each beam's labels read 256 at a time with
// coalesced loads.  A beam is skipped when even the row's largest
// log-probability plus its score, with the smallest id it could have, does
// not beat the W-th candidate found so far: ordinary keys lp + A never exceed
// max(lp) + A (rounded addition is monotone).
//
// It takes plain values (the LDS structures it uses sit at fixed offsets).
// It is inlined although it is rare: a call would make the kernel reserve
// scalar registers for the stack and the return address, and the beam
// wave's frame loop, short of scalar registers, would spill more of its own.
__device__ __forceinline__ int full_select(const float* row, int par, int last, int W,
                                                     int V, int blank, int space) {
  extern __shared__ __align__(16) char smem[];
  uint64_t* const buf = reinterpret_cast<uint64_t*>(smem + lds::buf);
  const float* const sA = reinterpret_cast<const float*>(smem + lds::A);
  const float* const skb = reinterpret_cast<const float*>(smem + lds::kb);
  const float* const skc = reinterpret_cast<const float*>(smem + lds::kc);
  const int* const slastk = reinterpret_cast<const int*>(smem + lds::lastk);
  int* const nchild = reinterpret_cast<int*>(smem + lds::nchild);
  int* const childc = reinterpret_cast<int*>(smem + lds::childc);
  const int lane = lane_id();
  // labels merged away from each beam: the last label of each of its children
  if (lane < W) nchild[lane] = 0;
  lds_sync();
  if (par >= 0) {
    const int pos = atomicAdd(&nchild[par], 1);
    childc[par * kMaxBeam + pos] = last;
  }
  lds_sync();
  // the row's largest non-blank log-probability
  float rmax = -__builtin_inff();
  for (int c0 = lane; c0 < V; c0 += 4 * kWave) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int c = c0 + u * kWave;
      v[u] = c < V ? row[c] : -__builtin_inff();
    }
#pragma unroll
    for (int u = 0; u < 4; u++) rmax = (c0 + u * kWave != blank) ? fmaxf(rmax, v[u]) : rmax;
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, m, 64));

  uint64_t thr = comp_floor();   // the W-th key of the buffer once it holds W
  int cnt = 0;
  auto flush = [&]() {   // sort the buffer and keep its best W
    lds_sync();
    wave_sort_lds(buf, cnt);
    lds_sync();
    cnt = cnt < W ? cnt : W;
    if (cnt == W) thr = buf[W - 1];
  };
  auto push = [&](uint64_t x) {   // keys of this lane (0 = none), 64 at a time
    const bool pass = x > thr;
    const uint64_t m = __ballot(pass);
    if (pass) buf[cnt + lanes_below(m)] = x;
    cnt += __popcll(m);
    if (cnt > kBuf - kWave) flush();
  };
  // the blank and repeated-label slots of every beam
  {
    const bool in = lane < W;
    const float A = in ? sA[lane] : kNeg;
    const float kb = in ? skb[lane] : kNeg, kc = in ? skc[lane] : kNeg;
    const int lk = in ? slastk[lane] : blank;
    const bool lv = A > kNeg;
    push(lv && kb > kNeg ? compose(kb, cand_id(lane, blank)) : 0ull);
    push(lv && lk != blank && lk != space && kc > kNeg ? compose(kc, cand_id(lane, lk)) : 0ull);
  }
  flush();
  // ordinary labels, beam by beam
  for (int k = 0; k < W; k++) {
    const float Ak = sA[k];
    if (!(Ak > kNeg)) continue;
    if (cnt == W && compose(rmax + Ak, cand_id(k, 0)) <= thr) continue;
    const int lk = slastk[k];
    const int lk_rep = lk != space ? lk : -1;   // the label of the repeated-label slot
    const int nc = nchild[k];
    const int chl = lane < nc ? childc[k * kMaxBeam + lane] : -1;
    for (int c0 = lane; c0 - lane < V; c0 += 4 * kWave) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int c = c0 + u * kWave;
        v[u] = c < V ? row[c] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int c = c0 + u * kWave;
        bool ok = c < V && c != blank && c != lk_rep;
        for (int j = 0; j < nc; j++) ok = ok && c != __builtin_amdgcn_readlane(chl, j);
        const float key = v[u] + Ak;
        push(ok && key > kNeg ? compose(key, cand_id(k, c)) : 0ull);
      }
    }
    flush();
  }
  return cnt;
}

template <int NB>
__device__ __forceinline__ Winner beam_step(Ctx& C, Beam& b, const float* row, int g, int step, int nR,
                            int complete) {
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W, V = L.V, blank = L.blank;
  // (values are computed on every lane and then selected: conditional
  // operators over computed values, no control flow on the common path)
  const bool lv = (lane < W) & (b.live != 0);

  const int last = b.last;
  // merge (sec. 3.4.3): beam j = parent i + `last`; i's extension by `last`
  // is folded into j's blank slot.  The parent's state is exchanged first so
  // that the exchange overlaps the arithmetic below.
  const int par = sel(lv, b.parent, -1);
  const int src = sel(par >= 0, par, lane);
  const float pb_par = __shfl(b.pb, src, 64);
  const int last_par = __shfl(last, src, 64);
  const float A_par = __shfl(b.A, src, 64);
  // (reads and writes below run on every lane: `last` is always a label, and
  // lanes without an effect write to their own spare entry or OR in zero)
  const bool has_last = lv & (last != blank);
  // a beam ending in the space label (sec. 3.4.2) extends by it like by any
  // other label and has no repeated-label slot and no stay term
  const bool rep_last = has_last & (last != L.space);
  const float lpc_raw = row[last];
  const float lpb = row[blank];
  const int rr_raw = (int)C.rank[last];
  // nothing else of the slot (row, label map) is read in this step: the exact
  // fallback reads the row from global memory.  The slot goes back to the
  // loader now (the reads above are LDS operations of this wave, performed
  // before the flag store that follows them).
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(C.release, C.frame, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const float lpc = sel(has_last, lpc_raw, kNeg);
  // labels removed from a beam's ordinary list: its own last label (that is
  // the repeated-label slot) and the last label of each child (merged away).
  // The masks (two words per lane: ranks 0..63) were cleared at the end of
  // the previous step.
  const bool same = (par >= 0) & (last == last_par) & rep_last;
  const bool child_other = (par >= 0) & !same;
  const bool rr_in = has_last & (rr_raw >= 0);
  const int rw = sel(rr_in, rr_raw, 0);
  const uint32_t rbit = sel(rr_in, 1u << (rw & 31), 0u);
  C.exclast[sel(same, par, kWave - 1 - lane % (kWave - kMaxBeam))] = 1;
  atomicOr(&C.exm[sel(par >= 0, par, lane) * 2 + (rw >> 5)], sel(child_other, rbit, 0u));
  atomicOr(&C.exm[lane * 2 + (rw >> 5)], sel(rep_last, rbit, 0u));
  // The reads of the exclusion masks below follow this wave's writes above
  // (one wave's LDS operations are performed in issue order); the fence only
  // keeps the compiler from moving them up.  The reads are issued before the
  // blank slot's two dependent logsumexp chains, whose arithmetic then
  // overlaps their latency.
  lds_order();
  PROF_MARK(1);
  const int excl_own = C.exclast[lane];
  // ---- each beam's two best candidates, as composite keys (0 = none): the
  // blank slot, the repeated-label slot and its first non-excluded ranked
  // labels.  Sorting those 2W keys gives the top W exactly whenever no beam
  // has a third candidate above the W-th of them (checked below); otherwise
  // the W-th key is a tight threshold for the general gather.
  const int nPool = complete ? nR : nR - 1;
  // in-pool ranks still open to this beam (nPool <= kMaxRanked <= 64)
  const uint64_t in_pool = nPool >= 64 ? ~0ull : ((1ull << nPool) - 1ull);
  const uint64_t exw = reinterpret_cast<const uint64_t*>(C.exm)[lane & (kMaxBeam - 1)];
  const float bound = C.Rl[nR - 1];   // no label outside the ranked list scores above A + bound

  // A_k = logsumexp(pb, pnb) was computed with the state.  The collapse for
  // skipped frames (sec. 3.4) turns (pb, pnb) into (A_k, NEG), and since
  // logsumexp(x, NEG) == x exactly, A_k is the same either way.
  const float A = sel(lv, b.A, kNeg);
  const float pb1 = g ? A : b.pb, pnb1 = g ? kNeg : b.pnb;
  const float pb1_par = g ? A_par : pb_par;
  const bool rep_ok = rep_last & (excl_own == 0);
  const float keyc = sel(rep_ok, lpc + pb1, kNeg);

  const uint64_t fr = sel(lv, ~exw & in_pool, (uint64_t)0);
  // the first three open ranks, without branches (-1: none)
  int rr[3];
  {
    uint64_t g01 = fr;
#pragma unroll
    for (int i = 0; i < 3; i++) {
      rr[i] = __ffsll((long long)g01) - 1;
      g01 &= g01 - 1ull;
    }
  }
  // their lists entries, all loads issued together (index 0 stands in for none)
  const uint32_t idb = cand_id(lane, 0);
  float rl[3];
  int rc[3];
#pragma unroll
  for (int i = 0; i < 3; i++) {
    const int r = sel(rr[i] >= 0, rr[i], 0);
    rl[i] = C.Rl[r];
    rc[i] = C.Rc[r];
  }

  // blank slot (sec. 3.4.2) holding the same-label "stay" term (sec. 3.4.1)
  const float ptb = sel(lv, lpb + A, kNeg);
  // logsumexp(x, NEG) == x exactly, so beams without a parent pass through
  const float from_parent = sel(par < 0, kNeg, sel(same, lpc + pb1_par, lpc + A_par));
  const float ptnb = lse(sel(!g & rep_last, lpc + pnb1, kNeg), from_parent);
  const float keyb = sel(lv, lse(ptb, ptnb), kNeg);
  // per-beam values that only the rare selection fallbacks read from LDS
  auto share_beam_values = [&]() {
    if (lane < W) {
      C.A[lane] = A;
      C.kb[lane] = keyb;
      C.kc[lane] = keyc;
      C.lastk[lane] = last;
    }
    lds_sync();
  };

  uint64_t oc[3];
#pragma unroll
  for (int i = 0; i < 3; i++) {
    const float key = rl[i] + A;
    oc[i] = sel(lv & (rr[i] >= 0) & (key > kNeg), compose(key, idb + (uint32_t)rc[i]), (uint64_t)0);
  }
  const uint64_t o1 = oc[0], o2 = oc[1], o3 = oc[2];
  const uint64_t cb = sel(lv & (keyb > kNeg), compose(keyb, idb + (uint32_t)blank), (uint64_t)0);
  const uint64_t cc = sel(lv & (keyc > kNeg), compose(keyc, idb + (uint32_t)last), (uint64_t)0);
  const uint64_t shi = cb > cc ? cb : cc, slo = cb > cc ? cc : cb;
  const uint64_t t1 = shi > o1 ? shi : o1;
  const uint64_t mid = shi > o1 ? o1 : shi, lo2 = slo > o2 ? slo : o2;
  const uint64_t t2 = mid > lo2 ? mid : lo2;
  // the beam's third candidate (its lists are sorted, so no later one scores
  // above it); ranked labels past the list are bounded separately below
  const uint64_t n3 = slo > o1 ? o1 : (shi > o2 ? lo2 : (shi > o3 ? shi : o3));
  PROF_MARK(9);
  // beam j's best goes to lane j, its second best to lane j + NB / 2 (one
  // lane swap; W <= NB / 2); the sorting network covers those first NB lanes
  // only (lane exchanges run on every lane, outside any lane-dependent
  // branch: a lane that is switched off supplies no value to the exchange)
  //
  // Usually the sort is not needed: when each beam's best candidate ranks in
  // beam order (beam j's above beam j + 1's) and every beam's second candidate
  // scores below the last beam's best, the top W are exactly the beams' best
  // candidates, already in rank order (nonzero keys are distinct, and beams
  // without a candidate hold 0, so t1[j] >= t1[j + 1] means "in order").
  //
  // Both checks on the candidates left out compare scores (the keys' upper 32
  // bits), not whole keys: a later label whose score rounds to the same value
  // as an earlier one's outranks it when its id is smaller, so only a strictly
  // lower score bounds the labels that follow a beam's first ones.
  constexpr uint64_t kScoreBits = 0xffffffff00000000ull;
  const uint64_t t1_next = wave_shl1_u64(t1);   // lane j: t1 of lane j + 1 (0 past the end)
  const uint64_t c1W = readlane_u64(t1, W - 1);
  const bool in_order = __ballot(t1 < t1_next) == 0ull;
  const bool no_second = __ballot((t2 != 0ull) & (t2 >= (c1W & kScoreBits))) == 0ull;
  uint64_t top, cW;
  bool exact;
  if (__builtin_expect(in_order & no_second, 1)) {
    top = t1;
    cW = c1W;
    exact = true;   // every later candidate scores below its beam's second
  } else {
    constexpr int H = NB / 2;
    const uint64_t t2x = xor_lane_u64<H>(t2);
    top = wave_sort_blocks_desc<NB>(
        __builtin_amdgcn_inverse_ballot_w64(lanes_below_n(H)) ? t1 : t2x);
    cW = readlane_u64(top, W - 1);
    exact = __ballot((n3 != 0ull) & (n3 >= (cW & kScoreBits))) == 0ull;
  }
  PROF_MARK(3);
  uint64_t wc;  // winner of slot `lane` (composite key, 0 = none)
  uint64_t wW;  // the W-th winner (wave-uniform)
  if (__builtin_expect(exact, 1)) {
    wc = lane < W ? top : 0ull;
    wW = cW;
    PROF_MARK(4);
  } else {
    const float tau0 = cW > comp_floor() ? comp_key(cW) : kNeg;
    // ---- every candidate at or above tau0 (ranked labels are sorted, so each
    // beam's qualifying labels form a prefix of its list)
    // gathered with a wave-uniform running count (ballot + lane prefix), the
    // ranked labels in chunks of four until no beam has one at or above tau0
    int nsurv = 0;
    {
      auto put = [&](bool pass, uint64_t key) {
        const uint64_t m = __ballot(pass);
        const int pos = nsurv + lanes_below(m);
        if (pass && pos < kBuf) C.buf[pos] = key;
        nsurv += __popcll(m);
      };
      put(lv && keyb > kNeg && keyb >= tau0, compose(keyb, cand_id(lane, blank)));
      put(lv && keyc > kNeg && keyc >= tau0, compose(keyc, cand_id(lane, last)));
      bool more = lv;
      for (int r = 0; r < nPool; r += 4) {
        if (!__ballot(more)) break;
#ifdef CTCPB_PHASE_PROF
#endif
        const float4 q = *reinterpret_cast<const float4*>(C.Rl + r);
        const int4 cq = *reinterpret_cast<const int4*>(C.Rc + r);
        const float lpv[4] = {q.x, q.y, q.z, q.w};
        const int cv[4] = {cq.x, cq.y, cq.z, cq.w};
        bool any = false;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int rr = r + j;
          const float key = lpv[j] + A;
          const bool above = more && rr < nPool && key >= tau0;
          any = any || above;
          const uint64_t open = fr >> (rr & 63);
          put(above && (open & 1u), compose(key, cand_id(lane, cv[j])));
        }
        more = more && any;
      }
    }
    lds_sync();
    PROF_MARK(4);
#ifdef CTCPB_PHASE_PROF
    C.stat_multi += 1;
#endif
    if (nsurv <= kWave) {
      // one survivor per lane, sorted in registers
      wc = wave_sort64_desc<uint64_t>(lane < nsurv ? C.buf[lane] : 0ull);
      if (lane >= W) wc = 0ull;
    } else {
      // many survivors: exact streaming top-W over them (regenerated per beam
      // from the ranked list, since the buffer kept only the first kBuf)
      share_beam_values();
      int lo = 0, hi = lv ? nPool : 0;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (C.Rl[mid] + A >= tau0) lo = mid + 1;
        else hi = mid;
      }
      const int nk = lo;
      const int incl = wave_incl_scan(lane < W ? nk : 0);
      const int M = __shfl(incl, 63, 64);
      if (lane < W) C.offs[lane] = incl - nk;
      lds_sync();
      const int ncand = M + 2 * W;
      auto candidate = [&](int64_t q64) -> uint64_t {
        const int q = (int)q64;
        if (q >= M) {
          const int j = q - M, kk = j >> 1;
          const float key = (j & 1) ? C.kc[kk] : C.kb[kk];
          const int c = (j & 1) ? C.lastk[kk] : blank;
          return (key > kNeg && key >= tau0) ? compose(key, cand_id(kk, c)) : 0ull;
        }
        int a = 0, z = W - 1;
        while (a < z) {
          const int mid = (a + z + 1) >> 1;
          if (C.offs[mid] <= q) a = mid;
          else z = mid - 1;
        }
        const int rho = q - C.offs[a];
        const uint32_t ex = (C.exm[a * 2 + (rho >> 5)] >> (rho & 31)) & 1u;
        return ex ? 0ull : compose(C.Rl[rho] + C.A[a], cand_id(a, C.Rc[rho]));
      };
      stream_topk(C, W, ncand, candidate);
      if (lane == 0) C.scal[kScalWide] += 1;
      wc = lane < W ? C.buf[lane] : 0ull;
    }
    wW = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(wc >> 32), W - 1) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wc, W - 1);
  }
  bool need_full = false;
  if (!complete) {
    // labels outside the ranked list score at most A_k + (last ranked lp);
    // they must stay strictly below the W-th selected key
    const float keyW = wW > comp_floor() ? comp_key(wW) : kNeg;
    const bool bad = lv && !((bound + A) < keyW);
    need_full = __ballot(bad) != 0ull;
  }
  if (__builtin_expect(need_full, 0)) {
    share_beam_values();
    full_select(C.grow, par, last, W, V, blank, L.space);
    if (lane == 0) C.scal[kScalFallbacks] += 1;
    wc = lane < W ? C.buf[lane] : 0ull;
  }

  PROF_MARK(5);
  // winners in rank order (slot r = rank r), sec. 3.4.5
  Winner w;
  w.valid = lane < W && wc > comp_floor();
  const uint32_t id = comp_id(wc);
  w.k = w.valid ? (int)(id >> kIdShift) : lane;
  w.c = w.valid ? (int)(id & ((1u << kIdShift) - 1u)) : blank;
  const float key = comp_key(wc);
  const int k = w.k & 63;
  // parent slots of the new beams (the prefix one label shorter, if live):
  // the slot that beam k's blank winner went to.  Written first, so that its
  // LDS round trip overlaps the state exchange below; bslot was cleared at the
  // end of the previous step.
  C.bslot[(w.valid && w.c == blank) ? w.k : kWave - 1 - lane % (kWave - kMaxBeam)] = lane;
  const float ptb_k = __shfl(ptb, k, 64);
  const float ptnb_k = __shfl(ptnb, k, 64);
  const int len_k = __shfl(b.len, k, 64);
  const int last_k = __shfl(last, k, 64);
  const int par_k = __shfl(b.parent, k, 64);
  const int last2_k = __shfl(b.last2, k, 64);
  const uint32_t h_k = (uint32_t)__shfl((int)b.h, k, 64);
  const uint32_t hp_k = (uint32_t)__shfl((int)b.hp, k, 64);
  w.len_k = len_k;
  const bool ext = w.valid && w.c != blank;
  Beam nb;
  nb.live = w.valid ? 1 : 0;
  nb.len = w.valid ? len_k + (ext ? 1 : 0) : 0;
  nb.last = ext ? w.c : (w.valid ? last_k : blank);
  nb.last2 = ext ? (len_k >= 1 ? last_k : -1) : (w.valid ? last2_k : -1);
  const uint32_t h_ext = hash_push(h_k, w.c);   // computed on every lane, then selected
  nb.h = ext ? h_ext : (w.valid ? h_k : kHashEmpty);
  nb.hp = ext ? h_k : (w.valid ? hp_k : 0u);
  nb.score = w.valid ? key : kNeg;
  // (pb, pnb): dead (NEG, NEG); after skipped frames (key, NEG); blank slot
  // (its two parts); a new label (NEG, key)
  const bool stay = w.c == blank;
  nb.pb = !w.valid ? kNeg : (g ? key : (stay ? ptb_k : kNeg));
  nb.pnb = !w.valid ? kNeg : (g ? kNeg : (stay ? ptnb_k : key));

  // The hash table (cleared at the end of the previous step) is only needed
  // when some stay winner's parent prefix was not live (it may just have been
  // re-created by extending its own parent).
  const bool need_look = w.valid && !ext && par_k < 0 && len_k >= 2;
  const bool any_look = __ballot(need_look) != 0ull;
  int hslot = -1;
  if (__builtin_expect(any_look, 0)) {
    if (lane < W) {
      C.newh[lane] = nb.h;
      C.newlen[lane] = nb.len;
    }
    if (ext) {
      int s = (int)(nb.h & (kHtab - 1));
      while (atomicCAS(&C.htab[s], -1, lane) != -1) s = (s + 1) & (kHtab - 1);
      hslot = s;
    }
  }
  // the next step's A = logsumexp(pb, pnb) of every new beam is its selection
  // key: a stay winner's key is logsumexp of the two parts it keeps, computed
  // from the same operands in the same order, and every other winner has one
  // part at NEG, where logsumexp(x, NEG) == x
  nb.A = w.valid ? key : kNeg;
  lds_order();
  const bool from_slot = ext || (w.valid && par_k >= 0);
  const int npar_raw = C.bslot[ext ? w.k : (par_k >= 0 ? par_k : 0)];
  int npar = from_slot ? npar_raw : -1;
  if (__builtin_expect(any_look, 0)) {
    int cand = -1;
    if (need_look) {
      int s = (int)(hp_k & (kHtab - 1));
      for (int probe = 0; probe < kHtab; probe++) {
        const int e = C.htab[s];
        if (e < 0) break;
        if (C.newh[e] == hp_k && C.newlen[e] == len_k - 1) {
          cand = e;
          break;
        }
        s = (s + 1) & (kHtab - 1);
      }
    }
    const int ce = cand >= 0 ? cand : lane;
    const int k2 = __shfl(w.k, ce, 64);
    const int c2 = __shfl(w.c, ce, 64);
    if (cand >= 0 && c2 != last2_k) cand = -1;
    uint64_t todo = __ballot(cand >= 0);
    // the previous step's tokens must have been written by the store wave
    if (todo && !spin_wait(C.tdone, step - 1, false, C.abortf)) todo = 0ull;
    if (todo) {
      const int q = (step - 1) & 1;
      const int from = C.scal[kScalCpl0 + q];
      while (todo) {
        const int v = __ffsll((long long)todo) - 1;
        todo &= todo - 1;
        const int ka = __shfl(w.k, v, 64);
        const int kb2 = __shfl(k2, v, 64);
        const int n = __shfl(len_k, v, 64) - 2;
        bool eq = true;
        for (int p = from + lane; p < n; p += kWave)
          eq = eq && tok_at(C, C.tab, q, ka, p) == tok_at(C, C.tab, q, kb2, p);
        const bool all = __ballot(!eq) == 0ull;
        if (lane == v && all) npar = cand;
        if (lane == 0) C.scal[kScalVerifies] += 1;
      }
    }
  }
  nb.parent = npar;
  b = nb;   // lanes past the beam hold the dead state either way
  // clear the exclusion masks, parent slots and hash entries for the next
  // step (LDS operations of this wave complete in order, after every read of
  // them above)
  reinterpret_cast<uint64_t*>(C.exm)[lane] = 0ull;
  C.exclast[lane] = 0;
  C.bslot[lane] = -1;
  if (hslot >= 0) C.htab[hslot] = -1;
  PROF_MARK(6);
  return w;
}

// ------------------------------------------------------------ token stores --
// Flat (sec. 3.1, 7): slot r of parity p receives its source's tokens from
// parity p^1 plus the new label.  Only positions that can differ from what
// the row already holds are written: if the source beam was itself forked
// from slot r one step earlier, the row's old content is the source's tokens
// but the label that fork appended, which is written directly (no copy);
// otherwise the row's old beam and the source's own source (both of two steps
// ago) share a known prefix, which is in place, and the rest is copied, 4
// tokens at once, eight such pieces per lane in flight.  In a step where no
// slot changes lineage nothing is copied.
// The shared prefixes are lower bounds kept per parity in a W x W matrix:
// rows forked from one source share its tokens, rows from two sources share
// at least what those shared; a step where every slot keeps its lineage keeps
// the previous step's matrix.
__device__ __forceinline__ void store_flat(const Ctx& C, StoreState& ss, int step, const Winner& w) {
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W, blank = L.blank;
  const int p = step & 1, q = p ^ 1;
  const uint32_t live2 = p ? ss.live1 : ss.live0;
  const int cplp = p ? ss.pre1 : ss.pre0;
  const int old_len = p ? ss.len1 : ss.len0;
  const int ksrc = __shfl(p ? ss.src0 : ss.src1, w.k, 64);   // source of w.k one step earlier
  const int klab = __shfl(p ? ss.lab0 : ss.lab1, w.k, 64);   // and the label it got then
  int16_t* mats = reinterpret_cast<int16_t*>(C.tail);
  const int16_t* mp = mats + (p ? ss.m1 : ss.m0) * W * W;    // rows of parity p (two steps ago)
  int start = 0;
  bool own = false;
  if (w.valid) {
    if (ksrc == lane && old_len >= 0) {
      start = old_len;
      own = true;
    } else if ((live2 >> lane) & 1u) {
      start = cplp;
      if (ksrc >= 0 && ((live2 >> ksrc) & 1u)) start = max(start, (int)mp[lane * W + ksrc]);
    }
    if (start > w.len_k) start = w.len_k;
  }
  // the row holds the source's tokens but (at most) the label of its last fork
  const bool direct = own && (w.len_k == old_len || (w.len_k == old_len + 1 && klab >= 0));
  const int s4 = start >> 2;
  const int e4 = w.valid ? (w.len_k + 3) >> 2 : 0;
  const int cnt = (w.valid && !direct) ? e4 - s4 : 0;
  int* row = C.clist + (int64_t)(p * W + (lane < W ? lane : 0)) * L.ldc;
  if (__ballot(lane < W && cnt > 0) != 0ull) {
    const int incl = wave_incl_scan(lane < W ? cnt : 0);
    const int total = __shfl(incl, 63, 64);
    int* offs = C.offs;  // [0, 33): offsets; [40, 72): first int4; [80, 112): sources
    if (lane < W) {
      offs[lane] = incl - cnt;
      offs[40 + lane] = s4;
      offs[80 + lane] = w.k;
    }
    lds_sync();
    int4* c4 = reinterpret_cast<int4*>(C.clist);
    const int64_t ld4 = L.ldc >> 2;
    // piece i goes to row a, the last with offs[a] <= i.  A lane's pieces
    // only move forward: the row of its first is found by binary lifting, the
    // later ones by stepping on (the next row's first piece kept at hand).
    int a = 0;
#pragma unroll
    for (int st = 16; st > 0; st >>= 1)
      if (a + st < W && offs[a + st] <= lane) a += st;
    int oa = offs[a], sa = offs[40 + a], ka = offs[80 + a];
    int nx = a + 1 < W ? offs[a + 1] : 0x7fffffff;
    struct Piece {
      int64_t d, s;   // destination and source, in 16-byte units of the lists
    };
    auto locate = [&](int i) -> Piece {
      while (i >= nx) {
        a++;
        oa = nx;
        sa = offs[40 + a];
        ka = offs[80 + a];
        nx = a + 1 < W ? offs[a + 1] : 0x7fffffff;
      }
      const int64_t pos4 = sa + (i - oa);
      return Piece{(int64_t)(p * W + a) * ld4 + pos4, (int64_t)(q * W + ka) * ld4 + pos4};
    };
    // eight pieces per lane in flight before any is stored (pieces past the
    // end stand on the last one and are not stored; with the lists in global
    // memory each round is one memory round trip)
    for (int i0 = lane; i0 < total; i0 += 8 * kWave) {
      auto at = [&](int u) { return locate(min(i0 + u * kWave, total - 1)); };
      const Piece p0 = at(0), p1 = at(1), p2 = at(2), p3 = at(3), p4 = at(4), p5 = at(5),
                  p6 = at(6), p7 = at(7);
      const int4 v0 = c4[p0.s], v1 = c4[p1.s], v2 = c4[p2.s], v3 = c4[p3.s], v4 = c4[p4.s],
                 v5 = c4[p5.s], v6 = c4[p6.s], v7 = c4[p7.s];
      c4[p0.d] = v0;
      if (i0 + kWave < total) c4[p1.d] = v1;
      if (i0 + 2 * kWave < total) c4[p2.d] = v2;
      if (i0 + 3 * kWave < total) c4[p3.d] = v3;
      if (i0 + 4 * kWave < total) c4[p4.d] = v4;
      if (i0 + 5 * kWave < total) c4[p5.d] = v5;
      if (i0 + 6 * kWave < total) c4[p6.d] = v6;
      if (i0 + 7 * kWave < total) c4[p7.d] = v7;
    }
    wave_sync();  // the copies land before the labels written below
  }
  if (direct && w.len_k == old_len + 1) row[old_len] = klab;
  if (w.valid && w.c != blank) row[w.len_k] = w.c;
  // this step's matrix (read above for parity p: the new one goes to the
  // buffer that parity q's does not use)
  const int mq = p ? ss.m0 : ss.m1;
  int mnew = mq;
  if (__ballot(lane < W && w.valid && w.k != lane) != 0ull) {
    mnew = 1 - mq;
    const int16_t* fq = mats + mq * W * W;
    int16_t* fn = mats + mnew * W * W + (lane < W ? lane : 0) * W;
    const int k1 = w.k < W ? w.k : 0;   // (slots without a beam: any row, never read)
    const int16_t lk1 = (int16_t)min(w.len_k, 32767);
    if (lane < W) {
#pragma unroll 4
      for (int r2 = 0; r2 < W; r2++) {
        const int k2 = __builtin_amdgcn_readlane(k1, r2);
        fn[r2] = k1 == k2 ? lk1 : fq[k1 * W + k2];
      }
    }
  }
  const int nlen = w.valid ? w.len_k + (w.c != blank ? 1 : 0) : -1;
  const int nsrc = w.valid ? w.k : -1;
  const int nlab = (w.valid && w.c != blank) ? w.c : -1;
  const uint32_t vm = (uint32_t)__ballot(w.valid);
  const int cplq = q ? ss.pre1 : ss.pre0;
  if (p) {
    ss.len1 = nlen;
    ss.src1 = nsrc;
    ss.lab1 = nlab;
    ss.live1 = vm;
    ss.pre1 = cplq;
    ss.m1 = mnew;
  } else {
    ss.len0 = nlen;
    ss.src0 = nsrc;
    ss.lab0 = nlab;
    ss.live0 = vm;
    ss.pre0 = cplq;
    ss.m0 = mnew;
  }
}

// Grow the common prefix of the live beams of parity p (flat store), reading
// the next 64 positions of every live row (every 16th store step).
__device__ __forceinline__ int common_prefix_flat(const int* clist, int W, int ldc, int p, int cpl,
                                                  bool nlive, int nlen) {
  const int lane = lane_id();
  const uint64_t live = __ballot(lane < W && nlive);
  if (live == 0ull) return cpl;
  int minlen = lane < W && nlive ? nlen : 0x7fffffff;
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) minlen = min(minlen, __shfl_xor(minlen, m, 64));
  const int pos = cpl + lane;
  const bool inside = pos < minlen;
  const int* base = clist + (int64_t)(p * W) * ldc + pos;
  int tk[kMaxBeam];
#pragma unroll
  for (int r = 0; r < kMaxBeam; r++)
    tk[r] = (inside && ((live >> r) & 1ull)) ? base[(int64_t)r * ldc] : -3;
  const int first = __ffsll((long long)live) - 1;
  int ref = -3;
#pragma unroll
  for (int r = 0; r < kMaxBeam; r++)
    if (r == first) ref = tk[r];
  bool same = inside;
#pragma unroll
  for (int r = 0; r < kMaxBeam; r++)
    if ((live >> r) & 1ull) same = same && tk[r] == ref;
  const uint64_t ok = __ballot(same);
  return cpl + (ok == ~0ull ? 64 : __ffsll((long long)~ok) - 1);
}

// The LDS copy that the exact prefix comparison reads is refreshed too (any
// older value is a lower bound: the common prefix never shrinks).
__device__ __forceinline__ void advance_cpl_flat(const Ctx& C, StoreState& ss, int p, bool nlive,
                                                 int nlen) {
  wave_sync();
  const int ncpl = common_prefix_flat(C.clist, C.L.W, C.L.ldc, p, p ? ss.pre1 : ss.pre0, nlive,
                                      nlen);
  if (p) ss.pre1 = ncpl;
  else ss.pre0 = ncpl;
  if (lane_id() == 0) C.scal[kScalCpl0 + p] = ncpl;
}

// Copies min(n, 4) int4 (n >= 1) from LDS: the loads are issued together,
// then the stores.
__device__ __forceinline__ void copy4_lds(int4* d, const int4* s, int n) {
  const int4 v0 = s[0];
  int4 v1, v2, v3;
  if (n > 1) v1 = s[1];
  if (n > 2) v2 = s[2];
  if (n > 3) v3 = s[3];
  d[0] = v0;
  if (n > 1) d[1] = v1;
  if (n > 2) d[2] = v2;
  if (n > 3) d[3] = v3;
}

// Paged (sec. 3.4.5 paged variant, 4.2): fork every slot's block-table row
// from its source (pages acquired / released by reference count), then
// append the new label on a fresh page, in place, or on a copy of the shared
// partial page rebuilt from the LDS mirror of that page (no global read).
// Leading full pages shared by every live row of two steps ago are identical
// in the old and the new row and are skipped.
// (The paged metadata is touched only by this wave here, in issue order: its
// LDS hand-offs between lanes need no waits.)
__device__ __forceinline__ void store_paged(Ctx& C, StoreState& ss, int step, const Winner& w,
                                            bool nlive, int nlen) {
#ifdef CTCPB_PHASE_PROF
  C.sprof_t = clock64();
#endif
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W, ps = L.ps, blank = L.blank, max_lp = L.max_lp;
  const int p = step & 1, q = p ^ 1;
  const bool in = lane < W;
  const uint32_t live2 = p ? ss.live1 : ss.live0;
  const int pcpp = p ? ss.pre1 : ss.pre0;
  const int old_t = in ? (p ? ss.len1 : ss.len0) : 0;
  const int ksrc = __shfl(p ? ss.src0 : ss.src1, w.k, 64);   // source of w.k one step earlier
  const int sh = L.ps_log2;   // page size = 1 << sh
  const int np_new = w.valid ? (w.len_k + ps - 1) >> sh : 0;
  const bool ext = w.valid && w.c != blank;
  const int off = w.len_k & (ps - 1);   // position of the new label in its page
  const int qq2 = w.len_k >> sh;        // and that page's entry
  int16_t* drow = C.tab + (p * W + (in ? lane : 0)) * max_lp;
  const int16_t* srow = C.tab + (q * W + (in ? w.k : 0)) * max_lp;
  // the page the label joins when it does not start one: the source's (the
  // fork copies that entry), read before any row of parity p changes
  const int phys = (ext && off != 0) ? (int)srow[qq2] : kInvalidPage;

  // tail mirror: the source's partial last page (its loads issued together)
  int* dt = C.tail + (p * W + (in ? lane : 0)) * ps;
  {
    const int4* st4 = reinterpret_cast<const int4*>(C.tail + (q * W + (in ? w.k : 0)) * ps);
    int4* dt4 = reinterpret_cast<int4*>(dt);
    const int n4 = w.valid ? (off + 3) >> 2 : 0;
    for (int j0 = 0; j0 < n4; j0 += 4) copy4_lds(dt4 + j0, st4 + j0, n4 - j0);
  }
  SP_MARK(0);

  // pass 1: fork, two entries per round (the round count is the wave's
  // largest, so the free-stack top stays wave-uniform).  The top is capped at
  // the pool size: after a row has run out of pages its tables can name pages
  // twice, and the cap keeps every stack read and page index inside the pool.
  // (Only the row's own pool is affected; its outputs are then unspecified.)
  int start = (in && ((live2 >> lane) & 1u)) ? (pcpp < old_t ? pcpp : old_t) : 0;
  // if the source was forked from this very slot one step earlier, the two
  // rows differ at most from the old row's last page on
  if (w.valid && ksrc == lane && old_t > 0 && start < old_t - 1) start = old_t - 1;
  const int end = in ? (old_t > np_new ? old_t : np_new) : 0;
  int ft = ss.freetop;
  for (int qq = start; __ballot(qq < end) != 0ull; qq += 2) {
    const bool a0 = qq < end, a1 = qq + 1 < end;
    const int o0 = (a0 && qq < old_t) ? (int)drow[qq] : kInvalidPage;
    const int n0 = (a0 && qq < np_new) ? (int)srow[qq] : kInvalidPage;
    const int o1 = (a1 && qq + 1 < old_t) ? (int)drow[qq + 1] : kInvalidPage;
    const int n1 = (a1 && qq + 1 < np_new) ? (int)srow[qq + 1] : kInvalidPage;
    const bool c0 = o0 != n0, c1 = o1 != n1;
    // (usually no entry of the round changes: the rows are already equal)
    if (__builtin_expect(__ballot(c0 | c1) == 0ull, 1)) continue;
    // a page released here is held by no row of parity p^1, so no fork of
    // this step acquires it: the order of the updates does not matter
    if (c0 && n0 != kInvalidPage) atomicAdd(&C.ref[n0], 1);
    if (c1 && n1 != kInvalidPage) atomicAdd(&C.ref[n1], 1);
    const bool f0 = c0 && o0 != kInvalidPage && atomicSub(&C.ref[o0], 1) == 1;
    const bool f1 = c1 && o1 != kInvalidPage && atomicSub(&C.ref[o1], 1) == 1;
    if (c0) drow[qq] = (int16_t)n0;
    if (c1) drow[qq + 1] = (int16_t)n1;
    const uint64_t m0 = __ballot(f0);
    const int at0 = ft + lanes_below(m0);
    if (f0 && at0 < L.npages) C.fstk[at0] = (int16_t)o0;
    ft = min(ft + __popcll(m0), L.npages);
    const uint64_t m1 = __ballot(f1);
    const int at1 = ft + lanes_below(m1);
    if (f1 && at1 < L.npages) C.fstk[at1] = (int16_t)o1;
    ft = min(ft + __popcll(m1), L.npages);
  }
  int new_t = in ? (np_new > 0 ? np_new : start) : old_t;
  lds_order();
  SP_MARK(1);

  // pass 2: append.  A label that goes into a partial page:
  //  - with a pool the caller sized (num_pages > 0), exactly as the page's
  //    allocator in ascending slot order (sec. 3.4.5), so that a pool runs
  //    out where the page's would: in place only if no other row holds the
  //    page (its reference count, less the earlier slots that copy it away
  //    first, is 1), else the page is copied.  The source's row of the
  //    previous step always holds its last page, so in practice every such
  //    label copies;
  //  - with the default pool, which cannot run out (sec. 4.2), in place also
  //    when only the source's row and this row hold it: the source's row ends
  //    before the label and is released at the next step, so no row can see
  //    the difference, and the copies and their pages are saved.
  const bool strict = L.paged == 2;
  int before = 0;
  if (strict) {
    for (uint64_t m = __ballot(phys >= 0); m != 0ull; m &= m - 1ull) {
      const int j = __ffsll((long long)m) - 1;
      before += (j < lane && __builtin_amdgcn_readlane(phys, j) == phys) ? 1 : 0;
    }
  }
  const bool inplace = phys >= 0 && C.ref[phys] - before <= (strict ? 1 : 2);
  const bool need = ext && !inplace;
  const uint64_t mk = __ballot(need);
  const int idx = lanes_below(mk);
  const int nw = __popcll(mk);
  const int avail = ft, nf = ss.nextfree;
  int page = kInvalidPage;
  if (need) {
    if (idx < avail) page = C.fstk[avail - 1 - idx];
    else if (nf + idx - avail < L.npages) page = nf + idx - avail;
  }
  const int pops = nw < avail ? nw : avail;
  ft = avail - pops;
  const int nn = nf + (nw - pops);
  ss.nextfree = nn < L.npages ? nn : L.npages;
  lds_order();   // the pops above read the stack before the pushes below
  if (ext) dt[off] = w.c;
  bool push_old = false;
  if (need) {
    if (page == kInvalidPage) {
      atomicOr(&C.scal[kScalStatus], kStatusOutOfPages);
    } else {
      C.ref[page] = 1;
      // the page's tokens up to the new label, from the tail mirror
      int4* g4 = reinterpret_cast<int4*>(C.pages + (int64_t)page * ps);
      const int4* t4 = reinterpret_cast<const int4*>(dt);
      const int n4 = (off >> 2) + 1;
      for (int j0 = 0; j0 < n4; j0 += 4) copy4_lds(g4 + j0, t4 + j0, n4 - j0);
      C.tab[(p * W + lane) * max_lp + qq2] = (int16_t)page;
      if (off == 0) new_t = qq2 + 1;
      if (off != 0 && phys >= 0) push_old = atomicSub(&C.ref[phys], 1) == 1;
    }
  } else if (inplace) {
    C.pages[(int64_t)phys * ps + off] = w.c;
  }
  const uint64_t mp = __ballot(push_old);
  const int atp = ft + lanes_below(mp);
  if (push_old && atp < L.npages) C.fstk[atp] = (int16_t)phys;
  ft = min(ft + __popcll(mp), L.npages);
  ss.freetop = ft;
  const int used = ss.nextfree - ft;
  ss.high = used > ss.high ? used : ss.high;
  SP_MARK(2);
  const uint32_t vm = (uint32_t)__ballot(w.valid);
  const int nsrc = w.valid ? w.k : -1;
  // leading full pages shared by every live row of parity p.  Rows only grow
  // at their last page and new rows extend rows of the previous step, so the
  // previous count stays a valid bound; it is advanced every 16 steps.
  int pcp = q ? ss.pre1 : ss.pre0;
  if ((step & 15) == 15) {
    lds_order();
    const bool lv = in && nlive;
    const uint64_t lm = __ballot(lv);
    const int first_live = lm ? __ffsll((long long)lm) - 1 : 0;
    while (lm != 0ull && pcp < max_lp) {
      const bool full = !lv || nlen >= ((pcp + 1) << sh);  // len <= cap keeps pcp < max_lp
      const int e = (lv && full) ? (int)drow[pcp] : kInvalidPage;
      const int first = __builtin_amdgcn_readlane(e, first_live);
      const bool ok = full && (!lv || e == first);
      if (__ballot(!ok) != 0ull) break;
      pcp++;
    }
  }
  if (p) {
    ss.len1 = new_t;
    ss.src1 = nsrc;
    ss.live1 = vm;
    ss.pre1 = pcp;
  } else {
    ss.len0 = new_t;
    ss.src0 = nsrc;
    ss.live0 = vm;
    ss.pre0 = pcp;
  }
  lds_order();
  SP_MARK(3);
}

// ------------------------------------------------------------------ output --
// N best of the current beams, (score desc, slot asc), tokens of `parity`.
template <typename TabT>
__device__ __forceinline__ void write_outputs(const Ctx& C, const Beam& b, int parity, const TabT* tab,
                              int out_row) {
  const Layout& L = C.L;
  const int lane = lane_id();
  const int W = L.W, N = C.N, mol = C.mol;
  const bool lv = lane < W && b.live;
  int rk = 0;
  for (int j = 0; j < W; j++) {
    const float sj = __shfl(b.score, j, 64);
    const int lj = __shfl(lv ? 1 : 0, j, 64);
    if (lj && (sj > b.score || (sj == b.score && j < lane))) rk++;
  }
  int* slot_of = C.offs;  // rank -> slot (or -1)
  if (lane < N) slot_of[lane] = -1;
  lds_sync();
  if (lv && rk < N) slot_of[rk] = lane;
  lds_sync();
  const int s = lane < N ? slot_of[lane] : -1;
  const int len = __shfl(b.len, s < 0 ? 0 : s, 64);
  const float sc = __shfl(b.score, s < 0 ? 0 : s, 64);
  if (lane < N) {
    C.out_lengths[(int64_t)out_row * N + lane] = s < 0 ? 0 : len;
    C.out_scores[(int64_t)out_row * N + lane] = s < 0 ? kNeg : sc;
    slot_of[40 + lane] = s < 0 ? 0 : len;
  }
  lds_sync();
  int* ot = C.out_tokens + (int64_t)out_row * N * mol;
  const int total = N * mol;
  for (int base = 0; base < total; base += 8 * kWave) {
    int val[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int i = base + u * kWave + lane;
      val[u] = -1;
      if (i < total) {
        const int n = i / mol, pos = i - n * mol;
        const int s = slot_of[n];
        if (s >= 0 && pos < slot_of[40 + n]) val[u] = tok_at(C, tab, parity, s, pos);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int i = base + u * kWave + lane;
      if (i < total) ot[i] = val[u];
    }
  }
}

// ---------------------------------------------------------- state helpers --
// The beam arrays at `a` into registers (lanes past the fused decoder's beams
// hold the dead state); A is left for the caller.
__device__ __forceinline__ void beam_read(const char* a, int blank, Beam& b) {
  const int lane = lane_id();
  if (lane < kMaxBeam) {
    b.pb = reinterpret_cast<const float*>(a + BeamArrays::pb)[lane];
    b.pnb = reinterpret_cast<const float*>(a + BeamArrays::pnb)[lane];
    b.score = reinterpret_cast<const float*>(a + BeamArrays::score)[lane];
    b.len = reinterpret_cast<const int*>(a + BeamArrays::len)[lane];
    b.last = reinterpret_cast<const int*>(a + BeamArrays::last)[lane];
    b.parent = reinterpret_cast<const int*>(a + BeamArrays::parent)[lane];
    b.last2 = reinterpret_cast<const int*>(a + BeamArrays::last2)[lane];
    b.live = reinterpret_cast<const int*>(a + BeamArrays::live)[lane];
    b.h = reinterpret_cast<const uint32_t*>(a + BeamArrays::hash)[lane];
    b.hp = reinterpret_cast<const uint32_t*>(a + BeamArrays::phash)[lane];
  } else {
    b.live = 0;
    b.pb = b.pnb = b.score = kNeg;
    b.len = 0;
    b.last = blank;
    b.parent = b.last2 = -1;
    b.h = kHashEmpty;
    b.hp = 0;
  }
  b.A = kNeg;
}

__device__ __forceinline__ void beam_load(const Ctx& C, Beam& b) {
  beam_read(C.base + C.L.o_beam, C.L.blank, b);
  b.A = b.live ? lse(b.pb, b.pnb) : kNeg;
}

__device__ __forceinline__ void beam_store(const Ctx& C, const Beam& b) {
  const int lane = lane_id();
  char* a = C.base + C.L.o_beam;
  if (lane < kMaxBeam) {
    reinterpret_cast<float*>(a + BeamArrays::pb)[lane] = b.pb;
    reinterpret_cast<float*>(a + BeamArrays::pnb)[lane] = b.pnb;
    reinterpret_cast<float*>(a + BeamArrays::score)[lane] = b.score;
    reinterpret_cast<int*>(a + BeamArrays::len)[lane] = b.len;
    reinterpret_cast<int*>(a + BeamArrays::last)[lane] = b.last;
    reinterpret_cast<int*>(a + BeamArrays::parent)[lane] = b.parent;
    reinterpret_cast<int*>(a + BeamArrays::last2)[lane] = b.last2;
    reinterpret_cast<int*>(a + BeamArrays::live)[lane] = b.live;
    reinterpret_cast<uint32_t*>(a + BeamArrays::hash)[lane] = b.h;
    reinterpret_cast<uint32_t*>(a + BeamArrays::phash)[lane] = b.hp;
  }
}

// The empty hypothesis in slot 0, every other slot dead (sec. 13).
__device__ __forceinline__ void beam_fresh(Beam& b, int blank) {
  const int lane = lane_id();
  b.live = lane == 0;
  b.pb = lane == 0 ? 0.0f : kNeg;
  b.pnb = kNeg;
  b.score = lane == 0 ? 0.0f : kNeg;
  b.A = lane == 0 ? 0.0f : kNeg;   // logsumexp(0, NEG)
  b.len = 0;
  b.last = blank;
  b.parent = -1;
  b.last2 = -1;
  b.h = kHashEmpty;
  b.hp = 0;
}

__device__ __forceinline__ Ctx make_ctx(const Layout& L, const LdsPlan& S, int N, int mol,
                                        int* out_tokens, int* out_lengths, float* out_scores,
                                        char* base, char* smem) {
  Ctx C;
  C.L = L;
  C.N = N;
  C.mol = mol;
  C.out_tokens = out_tokens;
  C.out_lengths = out_lengths;
  C.out_scores = out_scores;
  C.base = base;
  C.hdr = reinterpret_cast<int*>(base);
  C.rank = nullptr;  // per frame slot, set by the frame loop
  C.Rc = nullptr;
  C.Rl = nullptr;
  C.buf = reinterpret_cast<uint64_t*>(smem + lds::buf);
  C.A = reinterpret_cast<float*>(smem + lds::A);
  C.kb = reinterpret_cast<float*>(smem + lds::kb);
  C.kc = reinterpret_cast<float*>(smem + lds::kc);
  C.lastk = reinterpret_cast<int*>(smem + lds::lastk);
  C.offs = reinterpret_cast<int*>(smem + lds::offs);
  C.exm = reinterpret_cast<uint32_t*>(smem + lds::exm);
  C.exclast = reinterpret_cast<int*>(smem + lds::exclast);
  C.bslot = reinterpret_cast<int*>(smem + lds::bslot);
  C.htab = reinterpret_cast<int*>(smem + lds::htab);
  C.newh = reinterpret_cast<uint32_t*>(smem + lds::newh);
  C.newlen = reinterpret_cast<int*>(smem + lds::newlen);
  C.nchild = reinterpret_cast<int*>(smem + lds::nchild);
  C.childc = reinterpret_cast<int*>(smem + lds::childc);
  C.scal = reinterpret_cast<int*>(smem + lds::scal);
  C.tab = reinterpret_cast<int16_t*>(smem + S.tab);
  C.ref = reinterpret_cast<int*>(smem + S.ref);
  C.fstk = reinterpret_cast<int16_t*>(smem + S.fstk);
  C.tail = reinterpret_cast<int*>(smem + S.tail);
  C.tlen = reinterpret_cast<int*>(smem + S.tlen);
  C.clist = S.clist_lds ? reinterpret_cast<int*>(smem + S.clist)
                        : reinterpret_cast<int*>(base + L.o_clist);
  C.pages = reinterpret_cast<int*>(base + L.o_pages);
  C.tdone = nullptr;
  C.abortf = nullptr;
  return C;
}

// Paged metadata: global row region <-> LDS.
__device__ __forceinline__ void paged_meta_io(const Ctx& C, bool to_lds) {
  const Layout& L = C.L;
  int* gt = reinterpret_cast<int*>(C.base + L.o_tab);
  int* gr = reinterpret_cast<int*>(C.base + L.o_ref);
  int* gf = reinterpret_cast<int*>(C.base + L.o_free);
  int* gl = reinterpret_cast<int*>(C.base + L.o_tail);
  int* gn = reinterpret_cast<int*>(C.base + L.o_tlen);
  const int nt = 2 * L.W * L.max_lp, nl = 2 * L.W * L.ps;
  if (to_lds) {
    wave_copy(C.tab, gt, nt);
    wave_copy(C.ref, gr, L.npages);
    wave_copy(C.fstk, gf, L.npages);
    wave_copy(C.tail, gl, nl);
    wave_copy(C.tlen, gn, 2 * kMaxBeam);
  } else {
    wave_copy(gt, C.tab, nt);
    wave_copy(gr, C.ref, L.npages);
    wave_copy(gf, C.fstk, L.npages);
    wave_copy(gl, C.tail, nl);
    wave_copy(gn, C.tlen, 2 * kMaxBeam);
  }
}

// Header fields <-> LDS scalars.
__device__ __forceinline__ void scal_from_header(const Ctx& C) {
  const int lane = lane_id();
  if (lane == 0) {
    const int* h = C.hdr;
    C.scal[kScalFreeTop] = h[kFreeTop];
    C.scal[kScalNextFree] = h[kNextFree];
    C.scal[kScalStatus] = h[kStatus];
    C.scal[kScalHigh] = h[kPagesHigh];
    C.scal[kScalLive0] = h[kLive0];
    C.scal[kScalLive1] = h[kLive1];
    C.scal[kScalCpl0] = h[kCpl0];
    C.scal[kScalCpl1] = h[kCpl1];
    C.scal[kScalPcp0] = h[kPcp0];
    C.scal[kScalPcp1] = h[kPcp1];
    C.scal[kScalFallbacks] = h[kFallbacks];
    C.scal[kScalVerifies] = h[kVerifies];
  }
}

__device__ __forceinline__ void scal_to_header(const Ctx& C, int step, int last_t, int frames) {
  const int lane = lane_id();
  if (lane == 0) {
    int* h = C.hdr;
    h[kStep] = step;
    h[kLastT] = last_t;
    if (frames >= 0) h[kFrames] = frames;
    h[kFreeTop] = C.scal[kScalFreeTop];
    h[kNextFree] = C.scal[kScalNextFree];
    h[kStatus] = C.scal[kScalStatus];
    h[kPagesHigh] = C.scal[kScalHigh];
    h[kLive0] = C.scal[kScalLive0];
    h[kLive1] = C.scal[kScalLive1];
    h[kCpl0] = C.scal[kScalCpl0];
    h[kCpl1] = C.scal[kScalCpl1];
    h[kPcp0] = C.scal[kScalPcp0];
    h[kPcp1] = C.scal[kScalPcp1];
    h[kFallbacks] = C.scal[kScalFallbacks];
    h[kVerifies] = C.scal[kScalVerifies];
  }
}

// ----------------------------------------------------------------- kernels --
// Frame selection (sec. 3.5): sel = ascending t < len with lp[t, blank] <
// log(threshold); one 256-thread block per row, ordered ballot compaction.
__global__ __launch_bounds__(256) void select_kernel(Params P) {
  __shared__ int wave_cnt[4];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  char* base = P.state + (int64_t)b * P.L.row_bytes;
  int* hdr = reinterpret_cast<int*>(base);
  int* sel = reinterpret_cast<int*>(base + P.L.o_sel);
  int len = P.seq_lengths[b];
  len = len < 0 ? 0 : (len > P.T ? P.T : len);
  const float* row = P.lp + (int64_t)b * P.stride_b + P.L.blank;
  int cnt = 0;
  for (int t0 = 0; t0 < len; t0 += 256) {
    const int t = t0 + tid;
    bool keep = false;
    if (t < len) {
      if (P.sel_mode == 0) keep = true;
      else if (P.sel_mode == 2) keep = row[(int64_t)t * P.stride_t] < P.log_thr;
    }
    const uint64_t m = __ballot(keep);
    if (lane == 0) wave_cnt[wv] = __popcll(m);
    __syncthreads();
    int before = cnt;
    for (int j = 0; j < wv; j++) before += wave_cnt[j];
    if (keep) sel[before + lanes_below(m)] = t;
    cnt += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }
  if (tid == 0) hdr[kNSel] = cnt;
}

}  // namespace ctcpb
#include "wide.h"
namespace ctcpb {

// Offline rows (STREAM = false) or streaming chunk rows (STREAM = true).  One
// workgroup per row, four roles:
//   wave 0       the serial beam recursion, frame by frame; it publishes each
//                step's winners (source slot, label, source length) into a
//                ring of kRing entries;
//   store wave   the token store, following the beam wave through that ring
//                (up to kRing steps behind): flat copies or paged forks and
//                appends, so token traffic is off the recursion's path;
//   loader       copies each frame's row into a free LDS slot;
//   producers    each takes every P-th frame once its row has landed and
//                ranks its labels, ahead of the recursion.
// Every row of log_prob is read once.
template <bool STREAM, int NB>
__global__ __launch_bounds__(512, 1) void decode_kernel(Params P) {
  extern __shared__ __align__(16) char smem[];
  const Layout L = P.L;
  const LdsPlan S = P.S;
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x >> 6);
  const int row_i = blockIdx.x;
  int srow = row_i;
  if (STREAM) {
    srow = P.rows ? P.rows[row_i] : row_i;
    if (srow < 0 || srow >= P.num_rows) return;
  }
  char* base = P.state + (int64_t)srow * L.row_bytes;
  const int W = L.W, V = L.V;
  int* hdr = reinterpret_cast<int*>(base);
  const int* sel = reinterpret_cast<const int*>(base + L.o_sel);
  int* flags = reinterpret_cast<int*>(smem + lds::flags);
  int* ready = flags;                    // [kMaxSlots]: frame held by each slot
  int* consumed = flags + kMaxSlots;     // last frame whose slot the beam wave handed back
  int* abortf = consumed + 1;
  int* wpub = consumed + 2;              // last step whose winners are in the ring
  int* wdone = consumed + 3;             // last step the store wave has taken from the ring
  int* loaded = consumed + 4;            // [kMaxSlots]: frame whose row each slot holds
  int* frame_t = loaded + kMaxSlots;     // [kMaxSlots]: time index of that frame
  int* nspeech = frame_t + kMaxSlots;    // streaming: frames of the chunk to decode
  int* tdone = nspeech + 1;              // last step whose token writes are complete
  int2* ring = reinterpret_cast<int2*>(smem + lds::ring);
  const int nslot = S.nslot, nprod = S.nprod;
  auto slot_row = [&](int sl) { return reinterpret_cast<float*>(smem + lds::end + sl * S.slot_stride); };
  // ranked list of frame f: entry f mod nrk of its own ring (nrk = nslot + nprod), so that a
  // slot can be released as soon as the beam wave has read the few row entries it needs
  const int nrk = S.nrk;
  auto rk_Rc = [&](int e) { return reinterpret_cast<int*>(smem + S.rk + e * 2 * lds::slot_k); };
  auto rk_Rl = [&](int e) {
    return reinterpret_cast<float*>(smem + S.rk + e * 2 * lds::slot_k + lds::slot_k);
  };
  auto slot_rank = [&](int sl) { return reinterpret_cast<int8_t*>(smem + lds::end + sl * S.slot_stride + S.slot_rank); };

  const int step_in = STREAM ? hdr[kStep] : 0;
  // wave roles: 0 beam; with 5 or more waves the light loader shares SIMD 0
  // with the beam wave (waves are spread over the 4 SIMDs in order)
  const int nwaves = 3 + nprod;
  const int store_wave = nwaves >= 5 ? 3 : 2;
  const int loader_wave = nwaves >= 5 ? 4 : 3;
  const int pid = wave == 1 ? 0 : (wave == 2 && nwaves >= 5 ? 1 : wave - 3);
  const float* lp_row = P.lp + (int64_t)(STREAM ? row_i : srow) * P.stride_b;
  const int64_t stride_t = P.stride_t;
  const int vec4 = P.vec4;
  // streaming: the beam wave reads the stream's header words and beam state,
  // and the loader fetches the chunk's first frame into slot 0 (without a
  // speech mask step 0 decodes chunk frame 0), while the set-up below runs:
  // these loads overlap the header read instead of following it
  int hv = 0;   // lane i < 16: header word i
  Beam bin;
  if (STREAM && wave == 0) {
    hv = lane < 16 ? hdr[lane] : 0;
    beam_read(base + L.o_beam, L.blank, bin);
  }
  const bool early_row = STREAM && P.speech == nullptr && wave == loader_wave;
  if (early_row) row_fetch_async(lp_row, slot_row(0), V, vec4);
  // set-up shared by all waves: empty label ranks, flags
  for (int sl = 0; sl < nslot; sl++)
    for (int c = (int)threadIdx.x; c < V; c += (int)blockDim.x) slot_rank(sl)[c] = -1;
  if (threadIdx.x < kMaxSlots) {
    ready[threadIdx.x] = -1;
    loaded[threadIdx.x] = -1;
  }
  if (threadIdx.x == 0) {
    *consumed = -1;
    *abortf = 0;
    *wpub = step_in - 1;
    *wdone = step_in - 1;
    *tdone = step_in - 1;
  }
  // streaming: chunk frame f is frame number frame0 + f; with a speech mask
  // only the frames it flags are decoded (sec. 9 is_speech_mask, start_frame_idx)
  const int frame0 = STREAM ? (P.start_frame ? P.start_frame[row_i] : hdr[kFrames]) : 0;
  const uint8_t* speech = STREAM && P.speech ? P.speech + (int64_t)row_i * P.T : nullptr;
  int nframes;
  if (STREAM) {
    int avail = P.T;
    if (speech) {
      if (threadIdx.x == 0) *nspeech = 0;
      __syncthreads();
      int cnt = 0;
      for (int f = (int)threadIdx.x; f < P.T; f += (int)blockDim.x) cnt += speech[f] != 0;
      if (cnt) atomicAdd(nspeech, cnt);
      __syncthreads();
      avail = *nspeech;
    }
    nframes = L.cap - step_in;
    nframes = nframes < 0 ? 0 : (nframes > avail ? avail : nframes);
  } else {
    nframes = hdr[kNSel];
  }
  // ranked labels per frame: 2W + 3, at most 40, so that the labels gathered
  // to rank them mostly fit one per lane.  Any step where a label outside the
  // list could still compete is detected and decoded by the full beam x vocab
  // selection instead.
  const int K = min(V - 1, min(2 * W + 3, kMaxRanked));
  const int complete = K == V - 1;
  __syncthreads();

  if (wave == loader_wave) {
    // ------------------------------------------------------------ loader
    // Copies each frame's row into its slot as soon as the slot is free and
    // flags it once the copy has landed.  It is the only wave that copies
    // global memory into LDS, so no other wave's LDS reads wait on a copy.
    int cur = 0;            // streaming with a mask: next chunk frame to look at
    int blk_base = -64;     // the 64 flags read last, as a bit mask
    uint64_t blk = 0ull;
#ifdef CTCPB_PHASE_PROF
    uint64_t lw = 0, ll = 0, lt = clock64();
#endif
    for (int f = 0, sl = 0; f < nframes; f++, sl = sl + 1 == nslot ? 0 : sl + 1) {
      if (!spin_wait(consumed, f - nslot, false, abortf)) break;
#ifdef CTCPB_PHASE_PROF
      {
        const uint64_t now = clock64();
        lw += now - lt;
        lt = now;
      }
#endif
      int c = f;   // chunk frame decoded as step f
      if (STREAM && speech) {
        // the next flagged frame (nframes counts flagged frames only, so one
        // exists; the scan still stops at the end of the chunk)
        c = -1;
        while (cur < P.T) {
          const int base = cur & ~63;
          if (base != blk_base) {
            blk = __ballot(base + lane < P.T && speech[base + lane] != 0);
            blk_base = base;
          }
          const uint64_t m = blk & (~0ull << (cur & 63));
          if (m) {
            c = base + __ffsll((long long)m) - 1;
            break;
          }
          cur = base + 64;
        }
        if (c < 0) {
          flag_store(abortf, 1);
          break;
        }
        cur = c + 1;
      }
      const int t = STREAM ? frame0 + c : sel[f];
      if (!(early_row && f == 0))   // (frame 0 of an unmasked chunk is on its way)
        row_fetch_async(lp_row + (int64_t)(STREAM ? c : t) * stride_t, slot_row(sl), V, vec4);
      if (lane == 0) frame_t[sl] = t;
      row_fetch_wait();
      flag_publish_lds(&loaded[sl], f);
#ifdef CTCPB_PHASE_PROF
      {
        const uint64_t now = clock64();
        ll += now - lt;
        lt = now;
      }
#endif
    }
    if (early_row) row_fetch_wait();   // the early fetch has landed, even if unused
#ifdef CTCPB_PHASE_PROF
    // (offline: the row region's beam arrays are unused, they take the counters)
    if (!STREAM && lane == 0) {
      uint64_t* d = reinterpret_cast<uint64_t*>(base + L.o_beam);
      d[0] = lw;
      d[1] = ll;
    }
#endif
    return;
  }

  if (wave != 0 && wave != store_wave) {
    // ------------------------------------------------------------ producer
    uint64_t* scr = reinterpret_cast<uint64_t*>(smem + S.scr + pid * kBuf * 8);
#ifdef CTCPB_PHASE_PROF
    uint64_t pw = 0, pr = 0, t0 = clock64(), t1;
    uint64_t rprof[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#endif
    // frame f sits in slot f mod nslot (kept incrementally: nprod <= nslot)
    for (int f = pid, sl = pid % nslot; f < nframes;
         f += nprod, sl = sl + nprod >= nslot ? sl + nprod - nslot : sl + nprod) {
      if (!spin_wait(&loaded[sl], f, true, abortf)) break;
#ifdef CTCPB_PHASE_PROF
      t1 = clock64();
      pw += t1 - t0;
#endif
      // the list of frame f - nslot (this slot's previous frame) is entry
      // (f - nslot) mod nrk = (f + nprod) mod nrk, which only frame f + nprod,
      // ranked next by this wave, overwrites
      rank_frame(slot_row(sl), V, L.blank, K, f >= nslot ? K : 0, rk_Rc((f + nprod) % nrk),
                 rk_Rc(f % nrk), rk_Rl(f % nrk), slot_rank(sl), scr
#ifdef CTCPB_PHASE_PROF
                 , rprof
#endif
      );
      flag_publish_lds(&ready[sl], f);
#ifdef CTCPB_PHASE_PROF
      t0 = clock64();
      pr += t0 - t1;
#endif
    }
#ifdef CTCPB_PHASE_PROF
    if (lane == 0) {
      unsigned long long* dst = reinterpret_cast<unsigned long long*>(hdr + kProfExtra);
      atomicAdd(dst + 0, (unsigned long long)pw);
      atomicAdd(dst + 1, (unsigned long long)pr);
      unsigned long long* rd = reinterpret_cast<unsigned long long*>(hdr + 16);
      for (int i = 0; i < 8; i++) atomicAdd(rd + i, (unsigned long long)rprof[i]);
    }
#endif
    return;
  }

  Ctx C = make_ctx(L, S, P.N, P.max_out_len, P.out_tokens, P.out_lengths, P.out_scores, base,
                   smem);
  C.tdone = tdone;
  C.abortf = abortf;

  if (wave == store_wave) {
    // ---------------------------------------------------------- store wave
    C.offs = reinterpret_cast<int*>(smem + lds::soffs);
    StoreState ss{};
    store_state_init(C, ss, STREAM);
#ifdef CTCPB_PHASE_PROF
    for (int i = 0; i < 4; i++) C.sprof[i] = 0;
#endif
#ifdef CTCPB_PHASE_PROF
    uint64_t sw = 0, sk = 0, t0 = clock64();
#endif
    int durable = step_in - 1;   // last step announced in tdone
    for (int f = 0; f < nframes; f++) {
      const int step = step_in + f;
      if (flag_load(wpub) < step) {
        // caught up with the beam wave: before waiting for its next step,
        // make the token writes so far durable and announce them (the beam
        // wave reads tokens only after tdone: in the rare exact prefix
        // comparison, and for the outputs)
        if (durable < step - 1) {
          __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): global token writes done
          flag_store(tdone, step - 1);
          durable = step - 1;
        }
        if (!spin_wait(wpub, step, false, abortf)) break;
      }
#ifdef CTCPB_PHASE_PROF
      uint64_t t1 = clock64();
      sw += t1 - t0;
#endif
      const int2 rec = lane < W ? ring[(f % kRing) * kWave + lane] : make_int2(-1, 0);
      Winner w;
      w.valid = rec.x >= 0;
      w.k = w.valid ? (rec.x >> 16) : lane;
      w.c = w.valid ? (rec.x & 0xffff) : L.blank;
      w.len_k = w.valid ? rec.y : 0;
      const bool nlive = w.valid;
      const int nlen = w.valid ? w.len_k + (w.c != L.blank ? 1 : 0) : 0;
      // (the beam wave's set-up of the LDS state is visible once its first
      // step is published)
      if (f == 0) store_state_load(C, ss);
      if (step == 0) {
        store_seed(C, ss, w);
      } else if (L.paged) {
        store_paged(C, ss, step, w, nlive, nlen);
      } else {
        store_flat(C, ss, step, w);
        // (every 16 steps, mid-way through a 16-frame stream chunk: its reads
        // of the lists in global memory would otherwise delay the chunk's end)
        if ((step & 15) == 7) advance_cpl_flat(C, ss, step & 1, nlive, nlen);
      }
      if (f == nframes - 1) store_state_save(C, ss, STREAM);
      // the ring entry is free again (its LDS state is written); the token
      // writes may still be in flight
      flag_publish_lds(wdone, step);
      if (f == nframes - 1) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): global token writes done
        flag_store(tdone, step);
      }
#ifdef CTCPB_PHASE_PROF
      t0 = clock64();
      sk += t0 - t1;
#endif
    }
#ifdef CTCPB_PHASE_PROF
    if (lane == 0) {
      unsigned long long* dst = reinterpret_cast<unsigned long long*>(hdr + kProfExtra);
      atomicAdd(dst + 2, (unsigned long long)sw);
      atomicAdd(dst + 3, (unsigned long long)sk);
      unsigned long long* sd = reinterpret_cast<unsigned long long*>(hdr + kProfBase);
      sd[2] = C.sprof[0];
      sd[8] = C.sprof[1];
      sd[10] = C.sprof[2];
      sd[11] = C.sprof[3];
    }
#endif
    return;
  }

  // -------------------------------------------------------------- beam wave
  Beam b;
  int step, last_t;
  if (STREAM) {
    step = step_in;
    last_t = __builtin_amdgcn_readlane(hv, kLastT);
    scal_from_header(C);
    b = bin;
    b.A = b.live ? lse(b.pb, b.pnb) : kNeg;
    if (L.paged) paged_meta_io(C, true);
  } else {
    step = 0;
    last_t = -1;
    if (lane < kScalCount) C.scal[lane] = 0;
    beam_fresh(b, L.blank);
    if (L.paged) {
      for (int i = lane; i < 2 * W * L.max_lp; i += kWave) C.tab[i] = (int16_t)kInvalidPage;
      for (int i = lane; i < L.npages; i += kWave) C.ref[i] = 0;
      for (int i = lane; i < 2 * kMaxBeam; i += kWave) C.tlen[i] = 0;
    }
  }
  reinterpret_cast<uint64_t*>(C.exm)[lane] = 0ull;
  C.exclast[lane] = 0;
  C.bslot[lane] = -1;
  for (int i = lane; i < kHtab; i += kWave) C.htab[i] = -1;
  lds_sync();

  bool aborted = false;
  int next_ready = -2;          // value of the next slot's flag, read one step early
  int next_t = -1;              // and its frame's time index, read with it
  int wdone_seen = step - 1;    // store-wave progress last observed
  C.release = consumed;
  for (int f = 0, sl = 0, ek = 0; f < nframes; f++) {
    const int sl_next = sl + 1 == nslot ? 0 : sl + 1;   // slot of frame f + 1
#ifdef CTCPB_PHASE_PROF
    if (f == 0) {
      for (int i = 0; i < kProfSlots; i++) C.prof[i] = 0;
      C.stat_multi = 0;
      C.prof_t = clock64();
    }
#endif
    if (__builtin_expect(next_ready != f, 0)) {
      if (!spin_wait(&ready[sl], f, true, abortf)) {
        aborted = true;
        break;
      }
      next_t = frame_t[sl];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    PROF_MARK(0);
    const float* row = slot_row(sl);
    C.Rc = rk_Rc(ek);
    C.Rl = rk_Rl(ek);
    C.rank = slot_rank(sl);
    const int t = uni(next_t);
    C.frame = f;
    // its row in global memory: offline, frame t of the row; streaming, chunk
    // row t - frame0 (not f: with a speech mask, step f of the chunk decodes
    // the f-th flagged frame, which can sit further into the chunk)
    C.grow = lp_row + (int64_t)(STREAM ? t - frame0 : t) * stride_t;
    Winner w;
    if (__builtin_expect(step == 0, 0)) {
      first_step(C, b, row, t > 0 ? 1 : 0, K);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __hip_atomic_store(consumed, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      const int nb0 = W > 1 ? W - 1 : 1;
      w.valid = lane < W && b.live;
      w.k = kSeed;
      w.c = lane < (nb0 < K ? nb0 : K) ? C.Rc[lane] : L.blank;
      w.len_k = 0;
    } else {
      const int g = t > last_t + 1 ? 1 : 0;
      w = beam_step<NB>(C, b, row, g, step, K, complete);
    }
    // hand the winners to the store wave (its ring entry must be free)
    if (__builtin_expect(wdone_seen < step - kRing, 0)) {
      if (!spin_wait(wdone, step - kRing, false, abortf)) {
        aborted = true;
        break;
      }
      wdone_seen = flag_load(wdone);
    }
    // peek at the next frame's flag now: its latency overlaps the end of
    // this step instead of stalling the top of the next one (LDS operations
    // complete in order, so a flag seen set here was written after the
    // slot's data)
    next_ready = __hip_atomic_load(&ready[sl_next], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    // (read after the flag: if the flag shows the frame, its time index,
    // written before it, is seen too; otherwise it is read again after the wait)
    next_t = __hip_atomic_load(&frame_t[sl_next], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ring[(f % kRing) * kWave + lane] =
        make_int2(w.valid ? ((w.k << 16) | w.c) : -1, w.valid ? w.len_k : 0);
    PROF_MARK(7);
    last_t = t;
    // the ring entry is written by LDS operations of this wave, which the LDS
    // performs in issue order: the flag written after them is seen only after
    // them, with no wait for their completion
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_store(wpub, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    step++;
    sl = sl_next;
    ek = ek + 1 == nrk ? 0 : ek + 1;
  }
  // every published step stored (bounded wait that the abort flag does not cut
  // short: the store wave drains what was published before it stops)
  if (!spin_wait(tdone, step - 1, false, nullptr)) aborted = true;
  if (aborted) atomicOr(&C.scal[kScalStatus], kStatusAborted);
#ifdef CTCPB_PHASE_PROF
  if (lane == 0 && nframes > 0) {
    uint64_t* dst = reinterpret_cast<uint64_t*>(C.hdr + kProfBase);
    for (int i = 0; i < 10; i++)   // 2, 8, 10, 11: store-wave counters
      if (i != 2 && i != 8) dst[i] = C.prof[i];
    if (!STREAM) C.hdr[kFrames] = (int)C.stat_multi;   // diagnostics only (offline)
  }
#endif
  lds_sync();

  if (STREAM) {
    beam_store(C, b);
    if (L.paged) paged_meta_io(C, false);
    scal_to_header(C, step, last_t, STREAM ? frame0 + P.T : -1);
  } else {
    wave_sync();
    const int parity = step > 0 ? (step - 1) & 1 : 0;
    write_outputs(C, b, parity, C.tab, srow);
    scal_to_header(C, step, last_t, STREAM ? frame0 + P.T : -1);
  }
}

// Fresh streams (stream_init / stream_reset): one block per stream.
__global__ __launch_bounds__(64) void stream_fresh_kernel(Params P) {
  const Layout L = P.L;
  const int lane = lane_id();
  int srow = P.rows ? P.rows[blockIdx.x] : (int)blockIdx.x;
  if (srow < 0 || srow >= P.num_rows) return;
  char* base = P.state + (int64_t)srow * L.row_bytes;
  int* hdr = reinterpret_cast<int*>(base);
  if (lane < kHdrInts) hdr[lane] = 0;
  if (lane == 0) hdr[kLastT] = -1;
  Ctx C;
  C.L = L;
  C.base = base;
  Beam b;
  beam_fresh(b, L.blank);
  beam_store(C, b);
  if (!L.paged && L.W <= kMaxBeam) {
    // the token store's kept state: no lineage, all-zero common-prefix bounds
    int* a = reinterpret_cast<int*>(base + L.o_sst);
    for (int i = lane; i < (int)(StoreArrays::bytes / 4); i += kWave)
      a[i] = i < (int)(StoreArrays::mat / 4) ? -1 : 0;
  }
  if (L.W > kMaxBeam) {
    // the wide decoder's kept state: the empty hypothesis in slot 0, every
    // other slot dead, no token rows written yet
    float* wf = reinterpret_cast<float*>(base + L.o_wide);
    int* wi = reinterpret_cast<int*>(base + L.o_wide);
    for (int i = lane; i < kMaxBeamWide; i += kWave) {
      wf[kWPb * kMaxBeamWide + i] = i == 0 ? 0.0f : kNeg;
      wf[kWPnb * kMaxBeamWide + i] = kNeg;
      wf[kWSc * kMaxBeamWide + i] = i == 0 ? 0.0f : kNeg;
      wi[kWLast * kMaxBeamWide + i] = L.blank;
      wi[kWLen * kMaxBeamWide + i] = 0;
      wi[kWPar * kMaxBeamWide + i] = -1;
      wi[kWH * kMaxBeamWide + i] = (int)kHashEmpty;
      wi[kWHp * kMaxBeamWide + i] = (int)kHashEmpty;
      wi[kWLive * kMaxBeamWide + i] = i == 0 ? 1 : 0;
      wi[kWSrc0 * kMaxBeamWide + i] = -1;
      wi[kWSrc1 * kMaxBeamWide + i] = -1;
      wi[kWFlen0 * kMaxBeamWide + i] = -1;
      wi[kWFlen1 * kMaxBeamWide + i] = -1;
      wi[kWNp0 * kMaxBeamWide + i] = 0;
      wi[kWNp1 * kMaxBeamWide + i] = 0;
    }
  }
  if (L.paged) {
    int* gt = reinterpret_cast<int*>(base + L.o_tab);
    int* gr = reinterpret_cast<int*>(base + L.o_ref);
    for (int i = lane; i < 2 * L.W * L.max_lp; i += kWave) gt[i] = kInvalidPage;
    for (int i = lane; i < L.npages; i += kWave) gr[i] = 0;
    int* gn = reinterpret_cast<int*>(base + L.o_tlen);
    for (int i = lane; i < 2 * kMaxBeam; i += kWave) gn[i] = 0;
  }
}

// read_state: report the N best of each listed stream without changing it.
__global__ __launch_bounds__(64) void read_state_kernel(Params P) {
  extern __shared__ __align__(16) char smem[];
  const Layout L = P.L;
  int srow = P.rows ? P.rows[blockIdx.x] : (int)blockIdx.x;
  if (srow < 0 || srow >= P.num_rows) return;
  char* base = P.state + (int64_t)srow * L.row_bytes;
  Ctx C = make_ctx(L, P.S, P.N, P.max_out_len, P.out_tokens, P.out_lengths, P.out_scores, base,
                   smem);
  C.clist = reinterpret_cast<int*>(base + L.o_clist);  // the persisted copy
  Beam b;
  beam_load(C, b);
  const int step = C.hdr[kStep];
  if (step == 0) beam_fresh(b, L.blank);
  const int parity = step > 0 ? (step - 1) & 1 : 0;
  const int* tab = reinterpret_cast<const int*>(base + L.o_tab);
  write_outputs(C, b, parity, tab, (int)blockIdx.x);
}

// Diagnostics: copy per-row header counters out (one thread per row).
__global__ __launch_bounds__(64) void row_stats_kernel(Params P) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= P.num_rows) return;
  const int* h = reinterpret_cast<const int*>(P.state + (int64_t)i * P.L.row_bytes);
  int* o = P.out_lengths + (int64_t)i * 8;
  o[0] = h[kStep];
  o[1] = P.L.cap_sel > 0 ? h[kNSel] : h[kFrames];
  o[2] = h[kStatus];
  o[3] = h[kPagesHigh];
  o[4] = h[kFallbacks];
  o[5] = h[kVerifies];
  o[6] = max(h[kCpl0], h[kCpl1]);
  o[7] = max(h[kPcp0], h[kPcp1]);
}

}  // namespace ctcpb

// ==================================================================== host ==
namespace {

using namespace ctcpb;

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int ok() {
  g_err.clear();
  return CTCPB_OK;
}

struct Resolved {
  int W, N, V, blank, space, mol, paged, ps, npages_cfg, cap_stream;
  float threshold;
};

int resolve(const ctcpb_config* cfg, Resolved& R) {
  if (!cfg) return fail(CTCPB_ERR_INVALID, "config is NULL");
  if (cfg->beam < 1 || cfg->beam > 128)
    return fail(CTCPB_ERR_INVALID, "beam must be in [1, 128], got " + std::to_string(cfg->beam));
  if (cfg->nbest < 1 || cfg->nbest > cfg->beam)
    return fail(CTCPB_ERR_INVALID, "nbest must be in [1, beam]");
  if (cfg->vocab < 2) return fail(CTCPB_ERR_INVALID, "vocab must be >= 2");
  if (cfg->vocab > kMaxVocab)
    return fail(CTCPB_ERR_UNSUPPORTED, "vocab > 16384 is not supported");
  if (cfg->blank_id < 0 || cfg->blank_id >= cfg->vocab)
    return fail(CTCPB_ERR_INVALID, "blank_id must be in [0, vocab)");
  if (cfg->max_out_len < 0) return fail(CTCPB_ERR_INVALID, "max_out_len must be >= 0");
  if (cfg->storage != CTCPB_STORAGE_FLAT && cfg->storage != CTCPB_STORAGE_PAGED)
    return fail(CTCPB_ERR_INVALID, "storage must be CTCPB_STORAGE_FLAT or CTCPB_STORAGE_PAGED");
  if (std::isnan(cfg->blank_threshold)) return fail(CTCPB_ERR_INVALID, "blank_threshold is NaN");
  const int ps = cfg->page_size == 0 ? 16 : cfg->page_size;
  if (cfg->storage == CTCPB_STORAGE_PAGED && (ps < 4 || ps > 64 || (ps & (ps - 1)) != 0))
    return fail(CTCPB_ERR_INVALID, "page_size must be a power of two in [4, 64]");
  if (cfg->num_pages < 0) return fail(CTCPB_ERR_INVALID, "num_pages must be >= 0");
  if (cfg->capacity < 0) return fail(CTCPB_ERR_INVALID, "capacity must be >= 0");
  if (cfg->space_id >= cfg->vocab)
    return fail(CTCPB_ERR_INVALID, "space_id must be < vocab (or -1 for no space slot)");
  R.W = cfg->beam;
  R.N = cfg->nbest;
  R.V = cfg->vocab;
  R.blank = cfg->blank_id;
  // the space slot exists for a space label other than the blank (sec. 3.4.2)
  R.space = (cfg->space_id >= 0 && cfg->space_id != cfg->blank_id) ? cfg->space_id : -1;
  R.mol = cfg->max_out_len;
  R.paged = cfg->storage == CTCPB_STORAGE_PAGED;
  R.ps = ps;
  R.npages_cfg = cfg->num_pages;
  R.cap_stream = cfg->capacity == 0 ? kDefaultCapacity : cfg->capacity;
  R.threshold = cfg->blank_threshold;
  return CTCPB_OK;
}

int align16(int x) { return (x + 15) & ~15; }

// Beams above 32 run on the wide kernel, which keeps flat token lists: paged
// storage needs the narrow decoder.
LdsPlan plan_lds_with(const Layout& L, int nprod, int spare, bool clist_lds) {
  LdsPlan S{};
  int off = lds::end;
  auto take = [&](int bytes) {
    const int at = off;
    off += align16(bytes);
    return at;
  };
  // ring of frame slots from lds::end: row, then the label -> rank map
  S.nprod = nprod;
  S.nslot = nprod + spare;
  S.slot_rank = align16(L.V * 4);
  S.slot_stride = S.slot_rank + align16(L.V);
  take(S.nslot * S.slot_stride);
  S.nrk = S.nslot + nprod;
  S.rk = take(S.nrk * 2 * lds::slot_k);
  S.scr = take(nprod * kBuf * 8);
  // paged token metadata, or the flat token lists when they fit
  S.tab = take(L.paged ? 2 * L.W * L.max_lp * 2 : 0);   // 16-bit page ids
  S.ref = take(L.paged ? L.npages * 4 : 0);             // 32-bit: updated atomically
  S.fstk = take(L.paged ? L.npages * 2 : 0);
  // paged: the tail mirrors; flat: the store wave's two matrices of pairwise
  // common-prefix lengths (int16, W x W each)
  S.tail = take(L.paged ? 2 * L.W * L.ps * 4 : 2 * L.W * L.W * 2);
  S.tlen = take(L.paged ? 2 * kMaxBeam * 4 : 0);
  S.clist_lds = (!L.paged && clist_lds) ? 1 : 0;
  S.clist = take(S.clist_lds ? 2 * L.W * L.ldc * 4 : 0);
  S.total = off;
  return S;
}

// More producer waves for wider vocabularies (the ranking pass grows with
// V while the beam recursion does not), as many as the LDS budget allows, and
// up to three frame slots beyond one per producer so that the loader can run
// ahead (a slot is held from its load until the beam wave has used it).
// Flat token lists go to LDS only for offline decodes (`lists_in_lds`): a
// stream's lists persist in its state, and copying the live rows in and out
// around every chunk costs more than the faster copies inside it save.
LdsPlan plan_lds(const Layout& L, bool lists_in_lds) {
  // four producer waves whenever they fit: ranking costs about the same per
  // frame at any vocabulary (its threshold search and sort are fixed work),
  // so small vocabularies need as many producers as large ones
  const int pref = 4;
  // flat token lists in LDS if they fit next to at least one producer
  for (int lds_clist = 1; lds_clist >= 0; lds_clist--) {
    if (lds_clist && (L.paged || !lists_in_lds)) continue;
    for (int nprod = pref; nprod >= 1; nprod--) {
      for (int spare = 3; spare >= 1; spare--) {
        if (nprod + spare > kMaxSlots) continue;
        const LdsPlan S = plan_lds_with(L, nprod, spare, lds_clist != 0);
        if (S.total <= kLdsLimit) return S;
      }
    }
  }
  return plan_lds_with(L, 1, 1, false);  // too large: check_lds reports it
}

Layout layout_for(const Resolved& R, int cap, int cap_sel) {
  Layout L = make_layout(R.W, R.V, R.blank, cap, R.paged, R.ps, R.npages_cfg, cap_sel);
  L.space = R.space;
  return L;
}

int check_lds(const Layout& L, const LdsPlan& S) {
  if (L.paged && L.npages > kMaxPages)
    return fail(CTCPB_ERR_UNSUPPORTED,
                "num_pages " + std::to_string(L.npages) + " exceeds " + std::to_string(kMaxPages));
  if (S.total > kLdsLimit)
    return fail(CTCPB_ERR_UNSUPPORTED,
                "decoder state needs " + std::to_string(S.total) +
                    " bytes of LDS per row, more than the 160 KiB of a CU (smaller vocab, "
                    "beam, capacity or num_pages)");
  return CTCPB_OK;
}

// The decode kernel whose sorting network fits the beam: 16, 32 or 64 lanes
// for beams up to 8, 16 or 32.
template <bool STREAM>
void (*decode_kernel_for(int W))(Params) {
  if (W <= 8) return decode_kernel<STREAM, 16>;
  if (W <= 16) return decode_kernel<STREAM, 32>;
  return decode_kernel<STREAM, 64>;
}

template <typename K>
int launch(K kernel, int blocks, int threads, int lds, hipStream_t st, const Params& P,
           const char* what) {
  if (blocks <= 0) return CTCPB_OK;
  if (lds > 64 * 1024) {
    // raised once per kernel to the CU's whole LDS (not a stream operation, but
    // kept out of repeated calls so that launches under stream capture are
    // plain kernel nodes)
    static std::mutex mu;
    static const void* raised[32];
    static int nraised = 0;
    const void* k = reinterpret_cast<const void*>(kernel);
    std::lock_guard<std::mutex> lock(mu);
    bool done = false;
    for (int i = 0; i < nraised; i++) done = done || raised[i] == k;
    if (!done) {
      if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit) !=
          hipSuccess)
        return fail(CTCPB_ERR_DEVICE, std::string("hipFuncSetAttribute failed for ") + what);
      if (nraised < 32) raised[nraised++] = k;
    }
  }
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), lds, st, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(CTCPB_ERR_DEVICE, std::string(what) + " launch failed: " + hipGetErrorString(e));
  return CTCPB_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the decoder can hold a row of this layout on one CU (the checks the
// decode and stream calls make before launching).
int check_fits(const Resolved& R, const Layout& L, bool stream) {
  if (R.W > kMaxBeam) {
    if (wide::lds_bytes(R.V, 1) > kLdsLimit)
      return fail(CTCPB_ERR_UNSUPPORTED, "vocabulary too wide for the wide-beam decoder");
    return CTCPB_OK;
  }
  return check_lds(L, plan_lds(L, !stream));
}

}  // namespace

extern "C" {

const char* ctcpb_last_error(void) { return g_err.c_str(); }

const char* ctcpb_version(void) { return "ctcpb 0.1 gfx950"; }

int ctcpb_workspace_size(const ctcpb_config* cfg, int32_t batch, int32_t max_T,
                         size_t* out_bytes) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (!out_bytes) return fail(CTCPB_ERR_INVALID, "out_bytes is NULL");
  if (batch < 0 || max_T < 0) return fail(CTCPB_ERR_INVALID, "batch and max_T must be >= 0");
  const Layout L = layout_for(R, max_T > 0 ? max_T : 1, max_T);
  if (int rc = check_fits(R, L, false)) return rc;
  *out_bytes = (size_t)batch * (size_t)L.row_bytes;
  return ok();
}

int ctcpb_state_size(const ctcpb_config* cfg, int32_t num_streams, size_t* out_bytes) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (!out_bytes) return fail(CTCPB_ERR_INVALID, "out_bytes is NULL");
  if (num_streams < 0) return fail(CTCPB_ERR_INVALID, "num_streams must be >= 0");
  const Layout L = layout_for(R, R.cap_stream, 0);
  if (int rc = check_fits(R, L, true)) return rc;
  *out_bytes = (size_t)num_streams * (size_t)L.row_bytes;
  return ok();
}

}  // extern "C"

namespace {

// The offline decode with a workspace of `workspace_bytes` bytes.  With
// `scratch_ws`, the workspace is the library's fixed device scratch array and
// is resolved only after every host-side check has passed (its address is
// taken from `get_ws`, which may fail).
template <typename GetWs>
int decode_offline_impl(const ctcpb_config* cfg, const float* log_prob, int64_t stride_b,
                        int64_t stride_t, int32_t batch, int32_t max_T,
                        const int32_t* seq_lengths, void* workspace, size_t workspace_bytes,
                        bool scratch_ws, GetWs get_ws, int32_t* out_tokens, int32_t* out_lengths,
                        float* out_scores, void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (batch < 0 || max_T < 0) return fail(CTCPB_ERR_INVALID, "batch and max_T must be >= 0");
  if (batch == 0) return ok();
  if (!log_prob || !seq_lengths || (!workspace && !scratch_ws) || !out_lengths || !out_scores ||
      (!out_tokens && R.mol > 0))
    return fail(CTCPB_ERR_INVALID, "a required pointer is NULL");
  if (max_T > 0 && stride_t < R.V) return fail(CTCPB_ERR_INVALID, "stride_t must be >= vocab");
  if (stride_b < 0)
    return fail(CTCPB_ERR_INVALID, "stride_b must be >= 0 (0: every row reads the same frames)");
  if (!scratch_ws && !aligned16(workspace))
    return fail(CTCPB_ERR_INVALID, "workspace must be 16-byte aligned");
  const Layout L = layout_for(R, max_T > 0 ? max_T : 1, max_T);
  const size_t need = (size_t)batch * (size_t)L.row_bytes;
  if (workspace_bytes < need) {
    if (scratch_ws)
      return fail(CTCPB_ERR_TOO_SMALL,
                  "this decode needs " + std::to_string(need) +
                      " bytes of workspace, more than the fixed scratch of " +
                      std::to_string(workspace_bytes) + " bytes (fewer rows per call)");
    return fail(CTCPB_ERR_TOO_SMALL, "workspace smaller than ctcpb_workspace_size");
  }
  const bool wide_path = R.W > kMaxBeam;
  Params P{};
  P.L = L;
  if (!wide_path) {
    P.S = plan_lds(L, true);
    if (int rc = check_lds(P.L, P.S)) return rc;
  } else {
    // two frame rows in LDS when they fit (the next frame is fetched ahead)
    P.S.nslot = wide::lds_bytes(R.V, 2) <= kLdsLimit ? 2 : 1;
    if (wide::lds_bytes(R.V, P.S.nslot) > kLdsLimit)
      return fail(CTCPB_ERR_UNSUPPORTED, "vocabulary too wide for the wide-beam decoder");
  }
  P.N = R.N;
  P.max_out_len = R.mol;
  if (R.threshold >= 1.0f) {
    P.sel_mode = 0;
  } else if (R.threshold <= 0.0f) {
    P.sel_mode = 1;
  } else {
    P.sel_mode = 2;
    P.log_thr = (float)std::log((double)R.threshold);
  }
  if (scratch_ws) {
    if (int rc = get_ws(&workspace)) return rc;
  }
  P.lp = log_prob;
  P.stride_b = stride_b;
  P.stride_t = stride_t;
  P.T = max_T;
  P.num_rows = batch;
  P.seq_lengths = seq_lengths;
  P.rows = nullptr;
  P.state = static_cast<char*>(workspace);
  P.out_tokens = out_tokens;
  P.out_lengths = out_lengths;
  P.out_scores = out_scores;
  P.vec4 = aligned16(log_prob) && (R.V % 4 == 0) && (stride_b % 4 == 0) && (stride_t % 4 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (int rc = launch(select_kernel, batch, 256, 0, st, P, "select_kernel")) return rc;
  if (wide_path) {
    // the ranked labels of every selected frame first, in parallel over frames
    const int groups = wide::rank_groups(P.T);
    if ((int64_t)batch * groups > INT_MAX)
      return fail(CTCPB_ERR_UNSUPPORTED, "too many rows for one wide-beam launch");
    if (int rc = launch(wide::rank_wide_kernel, batch * groups, wide::kNT,
                        wide::rank_lds_bytes(R.V), st, P, "rank_wide_kernel"))
      return rc;
    // paged: the page tables, refcounts and free stack in LDS when they fit
    // (S.tab / S.ref / S.fstk: their LDS offsets; 0: in the workspace)
    int wlds = wide::lds_bytes(R.V, P.S.nslot);
    if (L.paged && wlds + wide::pager_lds_bytes(L) <= kLdsLimit) {
      P.S.tab = wlds;
      P.S.ref = P.S.tab + align16(2 * L.W * L.max_lp * 4);
      P.S.fstk = P.S.ref + align16(L.npages * 4);
      wlds += wide::pager_lds_bytes(L);
    }
    if (int rc = launch(wide::decode_wide_kernel<false>, batch, wide::kNT, wlds, st, P,
                        "decode_wide_kernel"))
      return rc;
    return ok();
  }
  if (int rc = launch(decode_kernel_for<false>(R.W), batch, 64 * (3 + P.S.nprod), P.S.total,
                      st, P, "decode_kernel"))
    return rc;
  return ok();
}

}  // namespace

// ------------------------------------------------------- allocation-free --
// The workspace of ctcpb_decode_offline_noalloc: one fixed device array.  Each
// GPU that runs the call holds its own copy for the life of the process.  In
// host code `scratch` names a host-side stand-in, not the device memory: its
// device address is taken once per device with hipGetSymbolAddress and only
// that address is used.
namespace ctcpb {
__device__ __align__(256) char scratch[CTCPB_NOALLOC_SCRATCH_BYTES];
}  // namespace ctcpb

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (resolved on the device's
// first call, with that device current).
int scratch_for_current_device(void** out, void* stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(CTCPB_ERR_DEVICE, "no current HIP device");
  if (dev >= kMaxDevices)
    return fail(CTCPB_ERR_UNSUPPORTED, "device index " + std::to_string(dev) + " >= 64");
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return fail(CTCPB_ERR_INVALID, "stream is not a valid HIP stream");
    if (sdev != dev)
      return fail(CTCPB_ERR_INVALID, "stream belongs to device " + std::to_string(sdev) +
                                         ", not the current device " + std::to_string(dev));
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CTCPB_ERR_DEVICE,
                  std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CTCPB_OK;
}

}  // namespace

extern "C" {

int ctcpb_decode_offline(const ctcpb_config* cfg, const float* log_prob, int64_t stride_b,
                         int64_t stride_t, int32_t batch, int32_t max_T,
                         const int32_t* seq_lengths, void* workspace, size_t workspace_bytes,
                         int32_t* out_tokens, int32_t* out_lengths, float* out_scores,
                         void* stream) {
  return decode_offline_impl(cfg, log_prob, stride_b, stride_t, batch, max_T, seq_lengths,
                             workspace, workspace_bytes, false, [](void**) { return 0; },
                             out_tokens, out_lengths, out_scores, stream);
}

int ctcpb_decode_offline_noalloc(const ctcpb_config* cfg, const float* log_prob,
                                 int64_t stride_b, int64_t stride_t, int32_t batch,
                                 int32_t max_T, const int32_t* seq_lengths, int32_t* out_tokens,
                                 int32_t* out_lengths, float* out_scores, void* stream) {
  return decode_offline_impl(
      cfg, log_prob, stride_b, stride_t, batch, max_T, seq_lengths, nullptr,
      (size_t)CTCPB_NOALLOC_SCRATCH_BYTES, true,
      [stream](void** ws) { return scratch_for_current_device(ws, stream); }, out_tokens,
      out_lengths, out_scores, stream);
}

int ctcpb_stream_init(const ctcpb_config* cfg, void* state, size_t state_bytes,
                      int32_t num_streams, void* stream) {
  return ctcpb_stream_reset(cfg, state, state_bytes, num_streams, nullptr, num_streams, stream);
}

int ctcpb_stream_reset(const ctcpb_config* cfg, void* state, size_t state_bytes,
                       int32_t num_streams, const int32_t* rows, int32_t n_rows, void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (num_streams < 0 || n_rows < 0 || n_rows > num_streams)
    return fail(CTCPB_ERR_INVALID, "need 0 <= n_rows <= num_streams");
  if (n_rows == 0) return ok();
  if (!state) return fail(CTCPB_ERR_INVALID, "state is NULL");
  if (!aligned16(state)) return fail(CTCPB_ERR_INVALID, "state must be 16-byte aligned");
  const Layout L = layout_for(R, R.cap_stream, 0);
  if (state_bytes < (size_t)num_streams * (size_t)L.row_bytes)
    return fail(CTCPB_ERR_TOO_SMALL, "state smaller than ctcpb_state_size");
  Params P{};
  P.L = L;
  P.num_rows = num_streams;
  P.rows = rows;
  P.state = static_cast<char*>(state);
  if (int rc = launch(stream_fresh_kernel, n_rows, 64, 0, static_cast<hipStream_t>(stream), P,
                      "stream_fresh_kernel"))
    return rc;
  return ok();
}

int ctcpb_stream_chunk_ex(const ctcpb_config* cfg, void* state, size_t state_bytes,
                          int32_t num_streams, const float* log_prob_chunk, int64_t stride_row,
                          int64_t stride_t, int32_t chunk_T, const uint8_t* is_speech,
                          const int32_t* start_frame, const int32_t* rows, int32_t n_rows,
                          void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (num_streams < 0 || n_rows < 0 || n_rows > num_streams || chunk_T < 0)
    return fail(CTCPB_ERR_INVALID, "need 0 <= n_rows <= num_streams and chunk_T >= 0");
  if (n_rows == 0 || chunk_T == 0) return ok();
  if (!state || !log_prob_chunk) return fail(CTCPB_ERR_INVALID, "a required pointer is NULL");
  if (stride_t < R.V) return fail(CTCPB_ERR_INVALID, "stride_t must be >= vocab");
  if (stride_row < 0)
    return fail(CTCPB_ERR_INVALID, "stride_row must be >= 0 (0: every row reads the same frames)");
  if (!aligned16(state)) return fail(CTCPB_ERR_INVALID, "state must be 16-byte aligned");
  const Layout L = layout_for(R, R.cap_stream, 0);
  if (state_bytes < (size_t)num_streams * (size_t)L.row_bytes)
    return fail(CTCPB_ERR_TOO_SMALL, "state smaller than ctcpb_state_size");
  Params P{};
  P.L = L;
  const bool wide_path = R.W > kMaxBeam;
  if (!wide_path) {
    P.S = plan_lds(L, false);
    if (int rc = check_lds(P.L, P.S)) return rc;
  } else {
    P.S.nslot = wide::lds_bytes(R.V, 2) <= kLdsLimit ? 2 : 1;
    if (wide::lds_bytes(R.V, P.S.nslot) > kLdsLimit)
      return fail(CTCPB_ERR_UNSUPPORTED, "vocabulary too wide for the wide-beam decoder");
  }
  P.N = R.N;
  P.max_out_len = R.mol;
  P.lp = log_prob_chunk;
  P.stride_b = stride_row;
  P.stride_t = stride_t;
  P.T = chunk_T;
  P.num_rows = num_streams;
  P.rows = rows;
  P.speech = is_speech;
  P.start_frame = start_frame;
  P.state = static_cast<char*>(state);
  P.vec4 = aligned16(log_prob_chunk) && (R.V % 4 == 0) && (stride_row % 4 == 0) &&
           (stride_t % 4 == 0);
  if (wide_path) {
    if (int rc = launch(wide::decode_wide_kernel<true>, n_rows, wide::kNT,
                        wide::lds_bytes(R.V, P.S.nslot), static_cast<hipStream_t>(stream), P,
                        "decode_wide_kernel<stream>"))
      return rc;
    return ok();
  }
  if (int rc = launch(decode_kernel_for<true>(R.W), n_rows, 64 * (3 + P.S.nprod), P.S.total,
                      static_cast<hipStream_t>(stream), P, "decode_kernel<stream>"))
    return rc;
  return ok();
}

int ctcpb_stream_chunk(const ctcpb_config* cfg, void* state, size_t state_bytes,
                       int32_t num_streams, const float* log_prob_chunk, int64_t stride_row,
                       int64_t stride_t, int32_t chunk_T, const int32_t* rows, int32_t n_rows,
                       void* stream) {
  return ctcpb_stream_chunk_ex(cfg, state, state_bytes, num_streams, log_prob_chunk, stride_row,
                               stride_t, chunk_T, nullptr, nullptr, rows, n_rows, stream);
}

int ctcpb_stream_step(const ctcpb_config* cfg, void* state, size_t state_bytes,
                      int32_t num_streams, const float* log_prob_frame, int64_t stride_row,
                      const int32_t* frame_index, const int32_t* rows, int32_t n_rows,
                      void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  return ctcpb_stream_chunk_ex(cfg, state, state_bytes, num_streams, log_prob_frame, stride_row,
                               R.V, 1, nullptr, frame_index, rows, n_rows, stream);
}

int ctcpb_read_state(const ctcpb_config* cfg, const void* state, size_t state_bytes,
                     int32_t num_streams, const int32_t* rows, int32_t n_rows,
                     int32_t* out_tokens, int32_t* out_lengths, float* out_scores,
                     void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (num_streams < 0 || n_rows < 0 || n_rows > num_streams)
    return fail(CTCPB_ERR_INVALID, "need 0 <= n_rows <= num_streams");
  if (n_rows == 0) return ok();
  if (!state || !out_lengths || !out_scores || (!out_tokens && R.mol > 0))
    return fail(CTCPB_ERR_INVALID, "a required pointer is NULL");
  if (!aligned16(state)) return fail(CTCPB_ERR_INVALID, "state must be 16-byte aligned");
  const Layout L = layout_for(R, R.cap_stream, 0);
  if (state_bytes < (size_t)num_streams * (size_t)L.row_bytes)
    return fail(CTCPB_ERR_TOO_SMALL, "state smaller than ctcpb_state_size");
  Params P{};
  P.L = L;
  P.S = plan_lds(L, false);
  P.N = R.N;
  P.max_out_len = R.mol;
  P.num_rows = num_streams;
  P.rows = rows;
  P.state = static_cast<char*>(const_cast<void*>(state));
  P.out_tokens = out_tokens;
  P.out_lengths = out_lengths;
  P.out_scores = out_scores;
  if (R.W > kMaxBeam) {
    if (int rc = launch(wide::read_state_wide_kernel, n_rows, wide::kNT, 0,
                        static_cast<hipStream_t>(stream), P, "read_state_wide_kernel"))
      return rc;
    return ok();
  }
  // only the small per-row scratch is needed: rows/ranks, no frame buffers
  const int lds = lds::scal + kScalCount * 4;
  if (int rc = launch(read_state_kernel, n_rows, 64, lds, static_cast<hipStream_t>(stream), P,
                      "read_state_kernel"))
    return rc;
  return ok();
}

int ctcpb_row_stats(const ctcpb_config* cfg, const void* buf, size_t buf_bytes, int32_t num_rows,
                    int32_t max_T, int32_t* out, void* stream) {
  Resolved R;
  if (int rc = resolve(cfg, R)) return rc;
  if (num_rows < 0 || max_T < 0) return fail(CTCPB_ERR_INVALID, "num_rows and max_T must be >= 0");
  if (num_rows == 0) return ok();
  if (!buf || !out) return fail(CTCPB_ERR_INVALID, "a required pointer is NULL");
  const Layout L = max_T > 0 ? layout_for(R, max_T, max_T) : layout_for(R, R.cap_stream, 0);
  if (buf_bytes < (size_t)num_rows * (size_t)L.row_bytes)
    return fail(CTCPB_ERR_TOO_SMALL, "buffer smaller than the rows it should hold");
  Params P{};
  P.L = L;
  P.num_rows = num_rows;
  P.state = static_cast<char*>(const_cast<void*>(buf));
  P.out_lengths = out;
  if (int rc = launch(row_stats_kernel, (num_rows + 63) / 64, 64, 0,
                      static_cast<hipStream_t>(stream), P, "row_stats_kernel"))
    return rc;
  return ok();
}

}  // extern "C"
