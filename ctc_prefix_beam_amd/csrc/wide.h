// wide.h -- offline decode for beams of 33 to 128 slots (included by ctcpb.hip).
//
// The page runs beams above 32 through its multi-kernel pipeline (sec. 3.4.1 -
// 3.4.5) rather than the fused single-block step.  Here they get their own
// kernel, one workgroup of 256 threads per row with the whole frame loop in one
// launch, and the same results as the narrow decoder:
//   - the frame row is staged in LDS and its best K = min(V-1, 2W+2) non-blank
//     labels are found by a block-wide radix select (sec. 3.4.6: with each
//     beam's blank and repeated-label slots they contain the global top W);
//   - every beam's candidates are its blank slot, its repeated-label slot and
//     its ordinary ranked labels minus the ones merged away (sec. 3.4.3); a
//     candidate behind h + i - 2 larger ones (h: the rank of its beam's best
//     candidate among the beams' bests, i: its place in its beam's list) cannot
//     be in the top W, which leaves about W^2/2 candidates;
//   - those are held in registers, and a radix select over their 64-bit
//     (score, id) keys gives the W-th; the winners are ranked by counting;
//   - tokens are double-buffered flat lists in the workspace (sec. 3.1), or
//     pages with reference-counted sharing (sec. 3.4.5 paged variant, sec.
//     4.2; see WidePager); merge parents are tracked structurally, with a
//     hash lookup and an exact token comparison where a parent prefix may have
//     been re-created.
#pragma once

namespace ctcpb {
namespace wide {

constexpr int kNT = 256;                  // threads per row
constexpr int kMaxW = 128;
constexpr int kMaxK = 2 * kMaxW + 2;      // ranked labels per frame
constexpr int kExw = (kMaxK + 31) / 32;   // exclusion words per beam
constexpr int kItems = 36;                // candidates per thread (>= (W(W+1)/2 + 4W) / kNT)
constexpr int kCBuf = 1024;               // candidates at or above the sample bound

// LDS: fixed part at compile-time offsets, then the row and the label map.
namespace off {
constexpr int a16(int x) { return (x + 15) & ~15; }
constexpr int Rc = 0;                                   // int [kMaxK]
constexpr int Rl = Rc + a16(kMaxK * 4);                 // float [kMaxK]
constexpr int kb64 = Rl + a16(kMaxK * 4);               // u64 [kMaxK + 8]: gathered keys
constexpr int win = kb64 + a16((kMaxK + 8) * 8);        // u64 [kMaxW]: winners in rank order
constexpr int f_pb = win + a16(kMaxW * 8);              // per beam, float
constexpr int f_pnb = f_pb + kMaxW * 4;
constexpr int f_sc = f_pnb + kMaxW * 4;
constexpr int f_A = f_sc + kMaxW * 4;
constexpr int f_pb1 = f_A + kMaxW * 4;                  // pb after the gap collapse
constexpr int f_ptb = f_pb1 + kMaxW * 4;                // blank slot: pt
constexpr int f_stay = f_ptb + kMaxW * 4;               // blank slot: ptn after the merge fold
constexpr int f_kb = f_stay + kMaxW * 4;                // blank slot key
constexpr int f_kc = f_kb + kMaxW * 4;                  // repeated-label slot key
constexpr int f_lpc = f_kc + kMaxW * 4;                 // lp of the beam's last label
constexpr int i_live = f_lpc + kMaxW * 4;               // per beam, int
constexpr int i_last = i_live + kMaxW * 4;
constexpr int i_len = i_last + kMaxW * 4;
constexpr int i_par = i_len + kMaxW * 4;                // merge parent for this step
constexpr int i_h = i_par + kMaxW * 4;                  // prefix hash
constexpr int i_hp = i_h + kMaxW * 4;                   // hash of the prefix minus its last label
constexpr int i_exc = i_hp + kMaxW * 4;                 // repeated-label slot merged away
constexpr int i_lim = i_exc + kMaxW * 4;                // candidates considered
constexpr int i_bslot = i_lim + kMaxW * 4;              // slot of winner (k, blank)
constexpr int i_src = i_bslot + kMaxW * 4;              // [2][kMaxW] copy source per parity
constexpr int i_flen = i_src + 2 * kMaxW * 4;           // [2][kMaxW] row length per parity
constexpr int i_offs = i_flen + 2 * kMaxW * 4;          // [kMaxW + 1] prefix sums
constexpr int u64_head = i_offs + a16((kMaxW + 1) * 4); // u64 [kMaxW]: each beam's best
constexpr int tag = u64_head + kMaxW * 8;               // u64 [kMaxW]: (length, hash) of live slots
constexpr int exm = tag + kMaxW * 8;                    // u32 [kMaxW][kExw]
constexpr int cbuf = exm + a16(kMaxW * kExw * 4);       // u64 [kCBuf]: candidates
constexpr int hist = cbuf + kCBuf * 8;                  // int [256]
constexpr int sh = hist + 256 * 4;                      // int [16] block scalars
constexpr int khist = sh + 16 * 4;                      // int [2][256]: kth_largest, kept zero
constexpr int ksh = khist + 2 * 256 * 4;                // int [8]: kth_largest's scalars
constexpr int pg = ksh + 8 * 4;                         // int [8]: pager scalars
constexpr int pgP = pg + 8 * 4;                         // int [kMaxW]: page a slot appends into
constexpr int np = pgP + kMaxW * 4;                     // int [2][kMaxW]: pages held per row
constexpr int end = np + 2 * kMaxW * 4;
}  // namespace off

// Bytes of LDS for vocabulary V: nbuf rows of floats (2: the next frame is
// fetched while this one is decoded), then a 16-bit label -> rank map.
inline int lds_bytes(int V, int nbuf) {
  return off::end + nbuf * off::a16(V * 4) + off::a16(V * 2);
}

// Bytes of LDS for an offline row's page tables, refcounts and free stack
// (int32, laid out after the lds_bytes part when they fit).
inline int pager_lds_bytes(const Layout& L) {
  return off::a16(2 * L.W * L.max_lp * 4) + 2 * off::a16(L.npages * 4);
}

// Block-wide: the kth largest (1-based) nonzero 64-bit key of the items, by
// radix select over 8-bit digits; 0 when fewer than kth keys are nonzero.
// gen(i) gives item i's key for i in [0, n): the keys of items tid + j kNT,
// j < R, are generated once and kept in registers, any further ones are
// generated again in every pass.  khist holds two 256-bin histograms used by alternate passes; both are zero
// on entry and again on return (wave 0 clears the bins it has read), so a
// pass needs two barriers: after the counts, and after the digit is chosen
// (ksh holds one set of the chosen digit's scalars per histogram, and a set
// is written again only two passes later, after everyone has read it).
template <int R, typename Gen>
__device__ __forceinline__ uint64_t kth_largest(int n, int kth, Gen gen, int* khist, int* ksh) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint64_t kr[R];
#pragma unroll
  for (int j = 0; j < R; j++) kr[j] = tid + j * kNT < n ? gen(tid + j * kNT) : 0ull;
  uint64_t prefix = 0ull;
  int need = kth;
  for (int pass = 0, shift = 56; shift >= 0; pass++, shift -= 8) {
    int* hist = khist + (pass & 1) * 256;
    int* sv = ksh + (pass & 1) * 4;
    const uint64_t hmask = shift == 56 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
    for (int j = 0; j < R; j++) {
      const uint64_t x = kr[j];
      if (x != 0ull && (x & hmask) == prefix) atomicAdd(&hist[(int)((x >> shift) & 255u)], 1);
    }
    for (int i = tid + R * kNT; i < n; i += kNT) {
      const uint64_t x = gen(i);
      if (x != 0ull && (x & hmask) == prefix) atomicAdd(&hist[(int)((x >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l (descending)
      const int d0 = 255 - 4 * lane;
      const int c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
      hist[d0] = 0;
      hist[d0 - 1] = 0;
      hist[d0 - 2] = 0;
      hist[d0 - 3] = 0;
      const int s = c0 + c1 + c2 + c3;
      const int incl = wave_incl_scan(s);
      const int ex = incl - s;
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (ex < need && incl >= need) {
        int d, above, in;
        if (ex + c0 >= need) { d = d0; above = ex; in = c0; }
        else if (ex + c0 + c1 >= need) { d = d0 - 1; above = ex + c0; in = c1; }
        else if (ex + c0 + c1 + c2 >= need) { d = d0 - 2; above = ex + c0 + c1; in = c2; }
        else { d = d0 - 3; above = ex + c0 + c1 + c2; in = c3; }
        sv[0] = d;
        sv[1] = above;
        sv[2] = in;
      }
      if (lane == 0 && total < need) sv[0] = -1;
    }
    __syncthreads();
    const int d = sv[0], above = sv[1], in = sv[2];
    if (d < 0) return 0ull;
    prefix |= (uint64_t)d << shift;
    need -= above;
    // once the score half is fixed, a group of keys sharing it that is needed
    // whole ends the search: every key at or above prefix is taken
    if (shift == 32 && in == need) return prefix;
  }
  return prefix;
}

// Ranks the n keys of keys[0, n) (n <= 64 * kRankChunks; the nonzero ones
// pairwise distinct) in descending order and calls out(rank, key) once per
// nonzero key; zero keys rank below all others and are skipped.  keys may be
// tmp itself.
// Each wave sorts chunks of 64 keys in registers into tmp[0, 64 * chunks);
// a key's rank is its place in its own chunk plus, for every other chunk, the
// number of that chunk's keys above it (a binary search of the sorted chunk).
constexpr int kRankChunks = 5;
template <typename Out>
__device__ __forceinline__ void rank_keys(const uint64_t* keys, int n, uint64_t* tmp, Out out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (n + 63) >> 6;
  for (int c = wave; c < nch; c += kNT / 64) {   // wave-uniform: every lane sorts
    const int i = c * 64 + lane;
    tmp[i] = wave_sort64_desc<uint64_t>(i < n ? keys[i] : 0ull);
  }
  __syncthreads();
  for (int i = tid; i < nch * 64; i += kNT) {
    const uint64_t x = tmp[i];
    const int own = i >> 6;
    int r = i & 63;
    if (nch > 1) {
#pragma unroll
    for (int c = 0; c < kRankChunks; c++) {
      const uint64_t* a = tmp + (c < nch ? c : 0) * 64;
      int lo = 0;   // keys of chunk c above x: a leading run (descending, zero-padded)
#pragma unroll
      for (int st = 32; st >= 1; st >>= 1) lo += a[lo + st - 1] > x ? st : 0;
      lo += a[lo] > x ? 1 : 0;   // lo <= 63 before this
      r += (c < nch && c != own) ? lo : 0;
    }
    }
    if (x != 0ull) out(r, x);
  }
}

// The run of ranks whose score A + Rl[r] rounds to that of rank r (the
// scores do not increase with the rank): its first rank, and one past its last
// (at most `end`), by binary search.
__device__ __forceinline__ int tie_run_start(float A, const float* Rl, int r) {
  const float key = A + Rl[r];
  int lo = 0, hi = r;   // first rank in [0, r] whose score is not above key
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A + Rl[mid] > key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int tie_run_end(float A, const float* Rl, int r, int end) {
  const float key = A + Rl[r];
  int lo = r + 1, hi = end;   // first rank in (r, end) whose score is below key
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A + Rl[mid] < key) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// The 64 largest of the keys keys[0, n) (n <= 256; missing ones count as 0)
// in descending order, returned in wave 0's lanes (other waves: unspecified).
// Each of the first ceil(n / 64) waves sorts a chunk of 64 (odd chunks
// ascending) into tmp[0, 256); with more than two chunks waves 0 and 1 merge
// the pairs into tmp[256, 384) (wave 1's run stored ascending); wave 0 merges
// the last pair.  Block-wide: every thread calls it; tmp must not overlap
// keys.  Ends with wave 0 holding the result (no barrier after the merge).
__device__ __forceinline__ uint64_t block_top64(const uint64_t* keys, int n, uint64_t* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (n + 63) >> 6;
  if (wave < nch) {
    const uint64_t x = tid < n ? keys[tid] : 0ull;
    tmp[tid] = (wave & 1) ? wave_sort64_asc(x) : wave_sort64_desc<uint64_t>(x);
  } else if (wave < (nch > 2 ? 4 : 2)) {
    tmp[tid] = 0ull;   // empty chunks up to the end of the last pair
  }
  __syncthreads();
  const uint64_t* pair = tmp;
  if (nch > 2) {
    if (wave < 2) {
      const uint64_t m = wave_top64_merge(tmp[128 * wave + lane], tmp[128 * wave + 64 + lane]);
      tmp[256 + 64 * wave + (wave ? 63 - lane : lane)] = m;
    }
    __syncthreads();
    pair = tmp + 256;
  }
  uint64_t top = 0ull;
  if (wave == 0) top = wave_top64_merge(pair[lane], pair[64 + lane]);
  return top;
}

// A bitonic sequence of 64 keys (one per lane) into descending order.
__device__ __forceinline__ uint64_t wave_bitonic64_desc(uint64_t v) {
  v = bitonic_stage<64, 32>(v);
  v = bitonic_stage<64, 16>(v);
  v = bitonic_stage<64, 8>(v);
  v = bitonic_stage<64, 4>(v);
  v = bitonic_stage<64, 2>(v);
  return bitonic_stage<64, 1>(v);
}
// A bitonic sequence of 128 keys (h: the first 64, l: the rest) into
// descending order.
__device__ __forceinline__ void order128(uint64_t& h, uint64_t& l) {
  const uint64_t a = h > l ? h : l, b = h > l ? l : h;
  h = wave_bitonic64_desc(a);
  l = wave_bitonic64_desc(b);
}
// The 128 largest of keys[0, n) (n <= 512; missing ones count as 0) in
// descending order, in wave 0's lanes: hi holds ranks 0-63, lo ranks 64-127
// (other waves: unspecified).  Each wave orders a chunk of 128 (two keys per
// lane: a run of 64 each way, which together are bitonic, then the merge's
// cross stage and the last six stages on each half); waves 1 and 3 hand
// their runs to waves 0 and 2 through tmp, which keep the 128 largest of the
// two (the merge's first half-cleaner against the partner's run reversed,
// then the same ordering); wave 2 hands its result to wave 0 for the last
// merge.  Block-wide: every thread calls it; tmp (384 keys) must not overlap
// keys.  Ends with wave 0 holding the result (no barrier after the merge).
__device__ __forceinline__ void block_top128(const uint64_t* keys, int n, uint64_t* tmp,
                                             uint64_t& hi, uint64_t& lo) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = 128 * wave;
  uint64_t h = base + lane < n ? keys[base + lane] : 0ull;
  uint64_t l = base + 64 + lane < n ? keys[base + 64 + lane] : 0ull;
  h = wave_sort64_desc<uint64_t>(h);
  l = wave_sort64_asc(l);
  order128(h, l);
  // the 128 largest of (h, l) and a descending run y of 128 held in tmp:
  // element i against y[127 - i]
  auto keep128 = [&](const uint64_t* y) {
    const uint64_t yh = y[127 - lane], yl = y[63 - lane];
    uint64_t mh = h > yh ? h : yh, ml = l > yl ? l : yl;
    order128(mh, ml);
    h = mh;
    l = ml;
  };
  if (wave & 1) {
    tmp[(wave >> 1) * 128 + lane] = h;
    tmp[(wave >> 1) * 128 + 64 + lane] = l;
  }
  __syncthreads();
  if (!(wave & 1)) keep128(tmp + (wave >> 1) * 128);
  if (wave == 2) {
    tmp[256 + lane] = h;
    tmp[256 + 64 + lane] = l;
  }
  __syncthreads();
  if (wave == 0) {
    keep128(tmp + 256);
    hi = h;
    lo = l;
  }
}

// The best K non-blank labels of a frame row by (lp desc, label asc) (sec.
// 3.4.6): out(rank, label) once per rank r < K (K <= V - 1: at least K labels
// have a nonzero key).  kb64: the gathered keys (kMaxK + 8); tmp: rank_keys'
// chunks; khist / ksh as kth_largest; cnt: one int.  Ends without a barrier
// (out's writes come last).
template <typename Out>
__device__ __forceinline__ void rank_frame_wide(const float* row, int V, int blank, int K,
                                                uint64_t* kb64, uint64_t* tmp, int* khist,
                                                int* ksh, int* cnt, Out out) {
  const int tid = threadIdx.x;
  auto lkey = [&](int c) -> uint64_t {
    return c == blank ? 0ull : compose(row[c], (uint32_t)c);
  };
  const uint64_t xk = kth_largest<8>(V, K, lkey, khist, ksh);
  if (tid == 0) *cnt = 0;
  __syncthreads();
  for (int c = tid; c < V; c += kNT) {
    const uint64_t x = lkey(c);
    if (x != 0ull && x >= xk) kb64[atomicAdd(cnt, 1)] = x;
  }
  __syncthreads();
  rank_keys(kb64, K, tmp, [&](int r, uint64_t x) { out(r, (int)comp_id(x)); });
}

// Offline: the ranked labels of every selected frame are independent of the
// beams, so a pre-pass ranks all of them in parallel (the page hoists its
// vocabulary ranking out of the fused step the same way, sec. 3.4.6) into
// the row's list region, [max_T][K] labels in rank order; the decode reads
// one list per step.  Block i ranks frames g, g + G, ... of row i / G (g =
// i % G, G = rank_groups(max_T)) with the decode's own ranking.
constexpr int kRankGroups = 256;
__host__ __device__ inline int rank_groups(int max_T) {
  return max_T < 1 ? 1 : (max_T < kRankGroups ? max_T : kRankGroups);
}
inline int rank_lds_bytes(int V) {
  return off::a16(V * 4) + off::a16((kMaxK + 8) * 8) + 64 * kRankChunks * 8 + 2 * 256 * 4 + 16 * 4;
}
__device__ __forceinline__ int* rank_lists(const Layout& L, char* base, int K) {
  const int64_t bytes = ((int64_t)L.cap_sel * K * 4 + 255) & ~(int64_t)255;   // align256
  return reinterpret_cast<int*>(base + L.row_bytes - bytes);
}

__global__ __launch_bounds__(kNT) void rank_wide_kernel(Params P) {
  extern __shared__ __align__(16) char smem[];
  const Layout L = P.L;
  const int G = rank_groups(P.T);
  const int V = L.V, blank = L.blank, W = L.W;
  const int b = blockIdx.x / G, g = blockIdx.x % G;
  char* base = P.state + (int64_t)b * L.row_bytes;
  const int* hdr = reinterpret_cast<const int*>(base);
  const int* sel = reinterpret_cast<const int*>(base + L.o_sel);
  const int nsel = hdr[kNSel];
  const int K = min(V - 1, 2 * W + 2);
  int* lists = rank_lists(L, base, K);
  float* row = reinterpret_cast<float*>(smem);
  uint64_t* kb64 = reinterpret_cast<uint64_t*>(smem + off::a16(V * 4));
  uint64_t* tmp = kb64 + (kMaxK + 8);
  int* khist = reinterpret_cast<int*>(tmp + 64 * kRankChunks);
  int* ksh = khist + 2 * 256;
  int* cnt = ksh + 8;
  for (int i = threadIdx.x; i < 2 * 256; i += kNT) khist[i] = 0;
  const float* lp_row = P.lp + (int64_t)b * P.stride_b;
  for (int f = g; f < nsel; f += G) {
    const float* gr = lp_row + (int64_t)sel[f] * P.stride_t;
    if (P.vec4) {
      for (int i = threadIdx.x; i < (V >> 2); i += kNT)
        reinterpret_cast<float4*>(row)[i] = reinterpret_cast<const float4*>(gr)[i];
    } else {
      for (int i = threadIdx.x; i < V; i += kNT) row[i] = gr[i];
    }
    __syncthreads();
    int* out = lists + (int64_t)f * K;
    rank_frame_wide(row, V, blank, K, kb64, tmp, khist, ksh, cnt,
                    [&](int r, int c) { out[r] = c; });
    __syncthreads();   // the row and the scratch are reused by the next frame
  }
}

// Paged token storage (sec. 3.4.5 paged variant, sec. 4.2) in the row region:
// block tables [2][W][max_lp] of page ids (-1 none; the pages a row holds are
// the leading entries of its table row), a reference count per page, a LIFO
// stack of freed pages and a bump pointer over the row's pool of npages.
// Each step forks every new row onto its source's pages, then appends the new
// label in slot order: a label that starts a page takes a fresh one; one that
// goes into a partial page shared with another row (its reference count,
// less the slots before it that already copied it away, is above 1) copies
// the page first; otherwise it writes in place.  A pop with nothing left
// gives no page: the beam keeps its prefix without appending and the row's
// status sets bit 0 (its outputs are then unspecified).
struct WidePager {
  int* tab;
  int* ref;
  int* fstk;
  int* pages;
  int W, ps, psh, mlp, npages;
  __device__ int* row(int par, int s) const { return tab + (int64_t)(par * W + s) * mlp; }
  // token pos of row (par, s), -1 where the row holds no page
  __device__ int tok(int par, int s, int pos) const {
    const int e = row(par, s)[pos >> psh];
    return e >= 0 ? pages[(int64_t)e * ps + (pos & (ps - 1))] : -1;
  }
};

__device__ __forceinline__ WidePager wide_pager(const Layout& L, char* base) {
  WidePager G;
  G.tab = reinterpret_cast<int*>(base + L.o_tab);
  G.ref = reinterpret_cast<int*>(base + L.o_ref);
  G.fstk = reinterpret_cast<int*>(base + L.o_free);
  G.pages = reinterpret_cast<int*>(base + L.o_pages);
  G.W = L.W;
  G.ps = L.ps;
  G.psh = L.ps_log2;
  G.mlp = L.max_lp;
  G.npages = L.npages;
  return G;
}

// The N best of one row (sec. 3.6): live slots by (score desc, slot asc),
// tokens from the flat lists (or the pages) of the last step's parity.
// out_rank: LDS scratch of at least kNT ints.  Ends with a block barrier.
__device__ __forceinline__ void wide_nbest(const Params& P, int out_row, int W, int step, int ldc,
                                           const int* clist, bool paged, const WidePager G,
                                           const int* s_live, const float* s_sc,
                                           const int* s_len, int* out_rank) {
  const int tid = threadIdx.x;
  const int parity = step > 0 ? (step - 1) & 1 : 0;
  const int N = P.N, mol = P.max_out_len;
  out_rank[tid] = -1;
  __syncthreads();
  if (tid < W && s_live[tid]) {
    const float sc = s_sc[tid];
    int r = 0;
    for (int j = 0; j < W; j++) {
      if (!s_live[j]) continue;
      const float sj = s_sc[j];
      r += (sj > sc || (sj == sc && j < tid)) ? 1 : 0;
    }
    if (r < N) out_rank[r] = tid;
  }
  __syncthreads();
  if (tid < N) {
    const int s = out_rank[tid];
    P.out_lengths[(int64_t)out_row * N + tid] = s < 0 ? 0 : s_len[s];
    P.out_scores[(int64_t)out_row * N + tid] = s < 0 ? kNeg : s_sc[s];
  }
  int* ot = P.out_tokens + (int64_t)out_row * N * mol;
  for (int i = tid; i < N * mol; i += kNT) {
    const int n = i / mol, pos = i - n * mol;
    const int s = out_rank[n];
    int v = -1;
    if (s >= 0 && pos < s_len[s] && step > 0)
      v = paged ? G.tok(parity, s, pos) : clist[(int64_t)(parity * W + s) * ldc + pos];
    ot[i] = v;
  }
  __syncthreads();
}

// Offline rows (STREAM = false) or streaming chunk rows (STREAM = true: the
// beam state is loaded from the stream's region at the start and stored back
// at the end; frames come from the chunk, optionally gated by a speech mask).
template <bool STREAM>
__global__ __launch_bounds__(kNT, 1) void decode_wide_kernel(Params P) {
  extern __shared__ __align__(16) char smem[];
  const Layout L = P.L;
  const int W = L.W, V = L.V, blank = L.blank;
  const int tid = threadIdx.x;
  const int row_i = blockIdx.x;
  int srow = row_i;
  if (STREAM) {
    srow = P.rows ? P.rows[row_i] : row_i;
    if (srow < 0 || srow >= P.num_rows) return;
  }
  char* base = P.state + (int64_t)srow * L.row_bytes;
  int* hdr = reinterpret_cast<int*>(base);
  const int* sel = reinterpret_cast<const int*>(base + L.o_sel);
  int* clist = reinterpret_cast<int*>(base + L.o_clist);
  const float* lp_row = P.lp + (int64_t)row_i * P.stride_b;
  const bool paged = L.paged != 0;
  WidePager G = wide_pager(L, base);
  if (!STREAM && paged && P.S.tab > 0) {
    // offline, when they fit: the row's page tables, refcounts and free stack
    // in LDS (they do not outlive the launch; the pages stay in the workspace)
    G.tab = reinterpret_cast<int*>(smem + P.S.tab);
    G.ref = reinterpret_cast<int*>(smem + P.S.ref);
    G.fstk = reinterpret_cast<int*>(smem + P.S.fstk);
  }

  int* Rc = reinterpret_cast<int*>(smem + off::Rc);
  float* Rl = reinterpret_cast<float*>(smem + off::Rl);
  uint64_t* kb64 = reinterpret_cast<uint64_t*>(smem + off::kb64);
  uint64_t* win = reinterpret_cast<uint64_t*>(smem + off::win);
  float* s_pb = reinterpret_cast<float*>(smem + off::f_pb);
  float* s_pnb = reinterpret_cast<float*>(smem + off::f_pnb);
  float* s_sc = reinterpret_cast<float*>(smem + off::f_sc);
  float* s_A = reinterpret_cast<float*>(smem + off::f_A);
  float* s_pb1 = reinterpret_cast<float*>(smem + off::f_pb1);
  float* s_ptb = reinterpret_cast<float*>(smem + off::f_ptb);
  float* s_stay = reinterpret_cast<float*>(smem + off::f_stay);
  float* s_kb = reinterpret_cast<float*>(smem + off::f_kb);
  float* s_kc = reinterpret_cast<float*>(smem + off::f_kc);
  float* s_lpc = reinterpret_cast<float*>(smem + off::f_lpc);
  int* s_live = reinterpret_cast<int*>(smem + off::i_live);
  int* s_last = reinterpret_cast<int*>(smem + off::i_last);
  int* s_len = reinterpret_cast<int*>(smem + off::i_len);
  int* s_par = reinterpret_cast<int*>(smem + off::i_par);
  uint32_t* s_h = reinterpret_cast<uint32_t*>(smem + off::i_h);
  uint32_t* s_hp = reinterpret_cast<uint32_t*>(smem + off::i_hp);
  int* s_exc = reinterpret_cast<int*>(smem + off::i_exc);
  int* s_lim = reinterpret_cast<int*>(smem + off::i_lim);
  int* s_bslot = reinterpret_cast<int*>(smem + off::i_bslot);
  int* s_src = reinterpret_cast<int*>(smem + off::i_src);
  int* s_flen = reinterpret_cast<int*>(smem + off::i_flen);
  int* s_offs = reinterpret_cast<int*>(smem + off::i_offs);
  uint64_t* s_head = reinterpret_cast<uint64_t*>(smem + off::u64_head);
  uint64_t* s_tag = reinterpret_cast<uint64_t*>(smem + off::tag);
  uint32_t* s_exm = reinterpret_cast<uint32_t*>(smem + off::exm);
  uint64_t* cbuf = reinterpret_cast<uint64_t*>(smem + off::cbuf);
  int* hist = reinterpret_cast<int*>(smem + off::hist);
  int* sh = reinterpret_cast<int*>(smem + off::sh);
  int* khist = reinterpret_cast<int*>(smem + off::khist);
  int* ksh = reinterpret_cast<int*>(smem + off::ksh);
  int* pgs = reinterpret_cast<int*>(smem + off::pg);      // free-stack depth, bump, high, counts
  int* s_pgP = reinterpret_cast<int*>(smem + off::pgP);
  int* s_np = reinterpret_cast<int*>(smem + off::np);
  const int nbuf = P.S.nslot;   // frame rows in LDS: 1 or 2
  float* rows = reinterpret_cast<float*>(smem + off::end);
  const int rstride = off::a16(V * 4) / 4;
  int16_t* rmap = reinterpret_cast<int16_t*>(smem + off::end + nbuf * off::a16(V * 4));
  const int wave = tid >> 6;

  const int K = min(V - 1, 2 * W + 2);
  const int ldc = L.ldc;
  // streaming: chunk frame c is frame number frame0 + c; with a speech mask
  // only the frames it flags are decoded (sec. 9 is_speech_mask,
  // start_frame_idx).  next_frame(c) is the first chunk frame >= c to decode
  // (the scan is the same on every thread).
  const int step_in = STREAM ? hdr[kStep] : 0;
  const int frame0 = STREAM ? (P.start_frame ? P.start_frame[row_i] : hdr[kFrames]) : 0;
  const uint8_t* speech = STREAM && P.speech ? P.speech + (int64_t)row_i * P.T : nullptr;
  auto next_frame = [&](int c) {
    if (speech)
      while (c < P.T && speech[c] == 0) c++;
    return c;
  };
  int nframes;
  if (STREAM) {
    int avail = P.T;
    if (speech) {
      if (tid == 0) sh[14] = 0;
      __syncthreads();
      int cnt = 0;
      for (int c = tid; c < P.T; c += kNT) cnt += speech[c] != 0;
      if (cnt) atomicAdd(&sh[14], cnt);
      __syncthreads();
      avail = sh[14];
    }
    nframes = L.cap - step_in;
    nframes = nframes < 0 ? 0 : (nframes > avail ? avail : nframes);
  } else {
    nframes = hdr[kNSel];
  }
  // the row of frame f: offline, frame sel[f] of the row; streaming, chunk row
  // cf (the f-th frame to decode)
  int cf = STREAM ? next_frame(0) : 0;
  auto frame_src = [&](int f, int c) {
    return lp_row + (int64_t)(STREAM ? c : sel[f]) * P.stride_t;
  };

  for (int c = tid; c < V; c += kNT) rmap[c] = -1;
  float* wst = reinterpret_cast<float*>(base + L.o_wide);   // streaming: kept beam state
  int* wsti = reinterpret_cast<int*>(base + L.o_wide);
  if (tid < kMaxW) {
    if (STREAM) {
      s_pb[tid] = wst[kWPb * kMaxW + tid];
      s_pnb[tid] = wst[kWPnb * kMaxW + tid];
      s_sc[tid] = wst[kWSc * kMaxW + tid];
      s_last[tid] = wsti[kWLast * kMaxW + tid];
      s_len[tid] = wsti[kWLen * kMaxW + tid];
      s_par[tid] = wsti[kWPar * kMaxW + tid];
      s_h[tid] = (uint32_t)wsti[kWH * kMaxW + tid];
      s_hp[tid] = (uint32_t)wsti[kWHp * kMaxW + tid];
      s_live[tid] = wsti[kWLive * kMaxW + tid];
      s_src[tid] = wsti[kWSrc0 * kMaxW + tid];
      s_src[kMaxW + tid] = wsti[kWSrc1 * kMaxW + tid];
      s_flen[tid] = wsti[kWFlen0 * kMaxW + tid];
      s_flen[kMaxW + tid] = wsti[kWFlen1 * kMaxW + tid];
      s_np[tid] = wsti[kWNp0 * kMaxW + tid];
      s_np[kMaxW + tid] = wsti[kWNp1 * kMaxW + tid];
    } else {
      // fresh row: the empty hypothesis in slot 0 (sec. 13), every other slot dead
      s_live[tid] = tid == 0 ? 1 : 0;
      s_pb[tid] = tid == 0 ? 0.0f : kNeg;
      s_pnb[tid] = kNeg;
      s_sc[tid] = tid == 0 ? 0.0f : kNeg;
      s_last[tid] = blank;
      s_len[tid] = 0;
      s_par[tid] = -1;
      s_h[tid] = kHashEmpty;
      s_hp[tid] = kHashEmpty;
      s_src[tid] = s_src[kMaxW + tid] = -1;
      s_flen[tid] = s_flen[kMaxW + tid] = -1;
      s_np[tid] = s_np[kMaxW + tid] = 0;
    }
  }
  if (!STREAM && paged) {
    // a fresh row's pager: no page held, none in use
    for (int i = tid; i < 2 * W * G.mlp; i += kNT) G.tab[i] = kInvalidPage;
    for (int i = tid; i < G.npages; i += kNT) G.ref[i] = 0;
    __threadfence();
  }
  // with two row buffers, wave 3 fetches frame f + 1 while frame f is decoded
  if (nbuf == 2 && wave == 3 && nframes > 0) row_fetch_async(frame_src(0, cf), rows, V, P.vec4);
  int last_t = STREAM ? hdr[kLastT] : -1, step = step_in, prevK = 0, nver = 0;
  for (int i = tid; i < 2 * 256; i += kNT) khist[i] = 0;
  // offline: the pre-pass's lists (rank_wide_kernel); this thread's entries
  // r = tid and tid + kNT of the next frame's list are loaded one step ahead
  const int* lists = STREAM ? nullptr : rank_lists(L, base, K);
  int lst0 = 0, lst1 = 0;
  if (!STREAM && nframes > 0) {
    lst0 = tid < K ? lists[tid] : 0;
    lst1 = tid + kNT < K ? lists[tid + kNT] : 0;
  }
  if (tid == 0) {
    // common token prefix of the live rows of parity 0 / 1
    sh[6] = STREAM ? hdr[kCpl0] : 0;
    sh[7] = STREAM ? hdr[kCpl1] : 0;
    sh[9] = 0;    // exact token comparisons
    sh[10] = STREAM ? hdr[kStatus] : 0;   // status bits
    pgs[0] = STREAM ? hdr[kFreeTop] : 0;
    pgs[1] = STREAM ? hdr[kNextFree] : 0;
    pgs[2] = STREAM ? hdr[kPagesHigh] : 0;
  }
  __syncthreads();

  for (int f = 0; f < nframes; f++) {
    const int t = STREAM ? frame0 + cf : sel[f];
    const int cnext = STREAM && f + 1 < nframes ? next_frame(cf + 1) : 0;
    const bool g = t > last_t + 1;    // frames skipped before t (step 0: t > 0)
    const int p = step & 1, q = p ^ 1;
    // ---- stage the row; clear the previous list's label map entries
    float* row = rows + (nbuf == 2 ? (f & 1) * rstride : 0);
    if (nbuf == 2) {
      if (wave == 3) row_fetch_wait();
    } else {
      const float* gr = frame_src(f, cf);
      if (P.vec4) {
        for (int i = tid; i < (V >> 2); i += kNT)
          reinterpret_cast<float4*>(row)[i] = reinterpret_cast<const float4*>(gr)[i];
      } else {
        for (int i = tid; i < V; i += kNT) row[i] = gr[i];
      }
    }
    for (int r = tid; r < prevK; r += kNT) rmap[Rc[r]] = -1;
    __syncthreads();
    // the other buffer was last read in the previous step: fetch the next frame
    if (nbuf == 2 && wave == 3 && f + 1 < nframes)
      row_fetch_async(frame_src(f + 1, cnext), rows + ((f + 1) & 1) * rstride, V, P.vec4);

    // ---- the frame's best K non-blank labels, (lp desc, label asc)
    if (STREAM) {
      rank_frame_wide(row, V, blank, K, kb64, cbuf, khist, ksh, &sh[2], [&](int r, int c) {
        Rc[r] = c;
        Rl[r] = row[c];
        rmap[c] = (int16_t)r;
      });
    } else {
      // ranked by the pre-pass
      if (tid < K) {
        Rc[tid] = lst0;
        Rl[tid] = row[lst0];
        rmap[lst0] = (int16_t)tid;
      }
      if (tid + kNT < K) {
        Rc[tid + kNT] = lst1;
        Rl[tid + kNT] = row[lst1];
        rmap[lst1] = (int16_t)(tid + kNT);
      }
      if (f + 1 < nframes) {
        const int* nl = lists + (int64_t)(f + 1) * K;
        lst0 = tid < K ? nl[tid] : 0;
        lst1 = tid + kNT < K ? nl[tid + kNT] : 0;
      }
    }
    prevK = K;
    if (tid < kMaxW) {
      for (int w = 0; w < kExw; w++) s_exm[tid * kExw + w] = 0u;
      s_exc[tid] = 0;
      s_bslot[tid] = -1;
    }
    __syncthreads();

    if (step == 0) {
      // ---- step 0 (sec. 3.3): the best W-1 labels (W = 1: the best one) and
      // the empty prefix in the last slot
      const int nb = W > 1 ? W - 1 : 1;
      const int m = min(nb, K);
      if (tid < W) {
        const int r = tid;
        int live = 0, len = 0, last = blank;
        float pb = kNeg, pnb = kNeg, sc = kNeg;
        uint32_t h = kHashEmpty;
        int par = -1;
        if (r < m) {
          const float key = Rl[r];
          live = 1;
          len = 1;
          last = Rc[r];
          pb = g ? key : kNeg;
          pnb = g ? kNeg : key;
          sc = key;
          h = hash_push(kHashEmpty, last);
          par = W > 1 ? W - 1 : -1;
          if (!paged) {
            clist[(int64_t)(0 * W + r) * ldc] = last;
          } else {
            // a page per seeded slot, taken in slot order from a fresh row's pool
            const int top = pgs[0], nf = pgs[1];
            const int pid = r < top ? G.fstk[top - 1 - r]
                                    : (nf + r - top < G.npages ? nf + r - top : kInvalidPage);
            if (pid >= 0) {
              G.row(0, r)[0] = pid;
              atomicExch(&G.ref[pid], 1);
              G.pages[(int64_t)pid * G.ps] = last;
              s_np[r] = 1;
            } else {
              atomicOr(&sh[10], kStatusOutOfPages);
            }
          }
        } else if (W > 1 && r == W - 1) {
          live = 1;
          pb = row[blank];
          sc = row[blank];
        }
        s_live[r] = live;
        s_len[r] = len;
        s_last[r] = last;
        s_pb[r] = pb;
        s_pnb[r] = pnb;
        s_sc[r] = sc;
        s_h[r] = h;
        s_hp[r] = kHashEmpty;
        s_par[r] = par;
        s_src[r] = -1;
        s_flen[r] = len;
      }
      __syncthreads();
      if (paged && tid == 0) {
        const int m0 = min(W > 1 ? W - 1 : 1, K);
        const int from = min(pgs[0], m0);
        pgs[0] -= from;
        pgs[1] = min(G.npages, pgs[1] + (m0 - from));
        pgs[2] = max(pgs[2], pgs[1] - pgs[0]);
      }
      last_t = t;
      step++;
      cf = cnext;
      continue;
    }

    // ---- per beam (sec. 3.4, 3.4.1 - 3.4.3): gap collapse, blank and
    // repeated-label slots, merge fold into the child's blank slot
    if (tid < W) {
      const int k = tid;
      const bool lv = s_live[k] != 0;
      const float pb = s_pb[k], pnb = s_pnb[k];
      const float A = lv ? lse(pb, pnb) : kNeg;
      const float pb1 = g ? A : pb, pnb1 = g ? kNeg : pnb;
      const int last = s_last[k];
      const bool has_last = lv && last != blank;
      // a beam ending in the space label (sec. 3.4.2) extends by it like by
      // any other label and has no repeated-label slot and no stay term
      const bool rep_last = has_last && last != L.space;
      const float lpc = has_last ? row[last] : kNeg;
      float stay = (rep_last && !g) ? lpc + pnb1 : kNeg;
      const int par = lv ? s_par[k] : -1;
      if (par >= 0) {
        // the parent's extension by this beam's last label joins this beam's
        // blank slot and leaves the parent's candidates
        const int lastp = s_last[par];
        const float Ap = lse(s_pb[par], s_pnb[par]);
        const float pb1p = g ? Ap : s_pb[par];
        const bool same = rep_last && last == lastp;
        const float from = same ? lpc + pb1p : lpc + Ap;
        stay = lse(stay, from);
        if (same) {
          s_exc[par] = 1;
        } else {
          const int r = rmap[last];
          if (r >= 0) atomicOr(&s_exm[par * kExw + (r >> 5)], 1u << (r & 31));
        }
      }
      // the beam's own last label is its repeated-label slot, not an ordinary one
      if (rep_last) {
        const int r = rmap[last];
        if (r >= 0) atomicOr(&s_exm[k * kExw + (r >> 5)], 1u << (r & 31));
      }
      const float ptb = lv ? row[blank] + A : kNeg;
      s_A[k] = A;
      s_pb1[k] = pb1;
      s_ptb[k] = ptb;
      s_stay[k] = stay;
      s_kb[k] = lv ? lse(ptb, stay) : kNeg;
      s_kc[k] = rep_last ? lpc + pb1 : kNeg;
      s_lpc[k] = lpc;
    }
    __syncthreads();
    // each beam's best candidate, its first two open ranks, and the sample
    // (both slots and those two ranks of every beam) whose W-th largest key
    // bounds the W-th largest candidate from below; n3: the score of the
    // beam's third open rank (no later label of the beam scores above it)
    float n3 = kNeg;
    uint64_t t1k = 0ull, t2k = 0ull;   // the beam's best and second best sample key
    if (tid < W) {
      const int k = tid;
      const bool lv = s_live[k] != 0;
      if (s_exc[k]) s_kc[k] = kNeg;
      const float kb = s_kb[k], kc = s_exc[k] ? kNeg : s_kc[k];
      uint64_t cb = 0ull, cc = 0ull, o0 = 0ull, o1 = 0ull, ob = 0ull;
      if (lv) {
        cb = kb > kNeg ? compose(kb, (uint32_t)((k << kIdShift) | blank)) : 0ull;
        cc = kc > kNeg ? compose(kc, (uint32_t)((k << kIdShift) | s_last[k])) : 0ull;
        int r0 = -1, r1 = -1, r2 = -1;
        for (int w = 0; w < kExw && r2 < 0; w++) {
          uint32_t open = ~s_exm[k * kExw + w];
          while (open && r2 < 0) {
            const int r = w * 32 + __ffs((int)open) - 1;
            open &= open - 1u;
            if (r >= K) break;
            if (r0 < 0) r0 = r;
            else if (r1 < 0) r1 = r;
            else r2 = r;
          }
        }
        if (r2 >= 0) n3 = s_A[k] + Rl[r2];
        // the beam's best ordinary candidate (for its place among the beams'
        // bests): the first open rank, unless a later open rank whose score
        // rounds to the same value has a smaller label and outranks it (only
        // where the run of that score holds different log-probabilities: in a
        // run of equal ones the labels already ascend)
        int rb = r0;
        if (r0 >= 0) {
          const float A = s_A[k], kr0 = A + Rl[r0];
          if (r0 + 1 < K && A + Rl[r0 + 1] == kr0) {
            const int re = tie_run_end(A, Rl, r0, K);
            if (Rl[re - 1] != Rl[r0]) {
              for (int r = r0 + 1; r < re; r++) {
                const bool ex = (s_exm[k * kExw + (r >> 5)] >> (r & 31)) & 1u;
                if (!ex && Rc[r] < Rc[rb]) rb = r;
              }
            }
          }
          ob = kr0 > kNeg ? compose(kr0, (uint32_t)((k << kIdShift) | Rc[rb])) : 0ull;
        }
        if (r0 >= 0) {
          const float key = s_A[k] + Rl[r0];
          o0 = key > kNeg ? compose(key, (uint32_t)((k << kIdShift) | Rc[r0])) : 0ull;
        }
        if (r1 >= 0) {
          const float key = s_A[k] + Rl[r1];
          o1 = key > kNeg ? compose(key, (uint32_t)((k << kIdShift) | Rc[r1])) : 0ull;
        }
      }
      const uint64_t b1 = cb > cc ? cb : cc;
      s_head[k] = b1 > ob ? b1 : ob;
      cbuf[4 * k + 0] = cb;
      cbuf[4 * k + 1] = cc;
      cbuf[4 * k + 2] = o0;
      cbuf[4 * k + 3] = o1;
      const uint64_t m1 = cb > cc ? cb : cc, m2 = cb > cc ? cc : cb;
      const uint64_t q1 = o0 > o1 ? o0 : o1, q2 = o0 > o1 ? o1 : o0;
      t1k = m1 > q1 ? m1 : q1;
      const uint64_t r1 = m1 > q1 ? q1 : m1, r2 = m2 > q2 ? m2 : q2;
      t2k = r1 > r2 ? r1 : r2;
    }
    constexpr uint64_t kScoreBits = 0xffffffff00000000ull;
    if (tid == 0) {
      sh[4] = 0;
      sh[15] = 0;
      if (W > 64) sh[1] = 1;
    }
    if (W > 64) {   // for the test below across two waves
      if (tid == 64) kb64[0] = t1k;
      if (tid == W - 1) kb64[1] = t1k;
    }
    if (W <= 64 && wave == 0) {
      // (beams up to 64, one per lane of this wave) as in the fused decoder:
      // when every beam's best ranks in beam order and every beam's second
      // scores strictly below the last beam's best, the beams' bests are the
      // winners, in rank order (every later candidate scores no higher than
      // its beam's second), and no sort is needed
      const uint64_t nxt = wave_shl1_u64(t1k);
      const uint64_t c1W = readlane_u64(t1k, W - 1);
      const bool in_order = __ballot(t1k < nxt) == 0ull;
      const bool no_second = __ballot((t2k != 0ull) & (t2k >= (c1W & kScoreBits))) == 0ull;
      const bool ok = in_order && no_second;
      if (ok) {
        if (tid < W) win[tid] = t1k;
        const int cnt = __popcll(__ballot(tid < W && t1k != 0ull));
        if (tid == 0) sh[4] = cnt;
      }
      if (tid == 0) sh[1] = ok ? 1 : 0;
    }
    __syncthreads();
    if (W > 64) {
      // the same test with the beams in two waves (the beam after a wave's
      // last and the last beam's best from LDS); the winners are written in
      // advance, and the paths below overwrite them
      if (wave < 2) {
        uint64_t nxt = wave_shl1_u64(t1k);
        if (tid == 63) nxt = kb64[0];
        const uint64_t c1W = kb64[1];
        const bool bad = __ballot(t1k < nxt) != 0ull ||
                         __ballot((t2k != 0ull) & (t2k >= (c1W & kScoreBits))) != 0ull;
        if (bad && (tid & 63) == 0) sh[1] = 0;
        if (tid < W) win[tid] = t1k;
        const int cnt = __popcll(__ballot(tid < W && t1k != 0ull));
        if ((tid & 63) == 0 && cnt) atomicAdd(&sh[4], cnt);
      }
      __syncthreads();
    }
    const bool in_order_fast = sh[1] != 0;
    // tau: the W-th largest of the 4W sample keys (0 when fewer are nonzero)
    uint64_t tau = 1ull;
    bool fast = in_order_fast;   // set when the winners are known without the survivors
    if (in_order_fast) {
    } else if (W <= 64) {
      const uint64_t top = block_top64(cbuf, 4 * W, cbuf + kCBuf - 384);
      if (wave == 0) {
        // (beams up to 64: all in this wave) when every beam's third open rank
        // scores strictly below the W-th sample key, so does every candidate
        // outside the sample (a later label whose score rounds to the same
        // value may outrank it by id, hence the strict score bound), and the
        // sample's best W, sorted, are the winners
        const uint64_t tw = readlane_u64(top, W - 1);
        const float twk = tw != 0ull ? comp_key(tw) : -__builtin_inff();
        const bool exact = __ballot(tid < W && n3 > kNeg && !(n3 < twk)) == 0ull;
        if (exact) {
          if (tid < W) win[tid] = top;
          const int cnt = __popcll(__ballot(tid < W && top != 0ull));
          if (tid == 0) sh[4] = cnt;
        }
        if (tid == 0) {
          reinterpret_cast<unsigned long long*>(sh + 12)[0] = tw;
          sh[15] = exact ? 0 : 1;
        }
      }
      __syncthreads();
      tau = reinterpret_cast<unsigned long long*>(sh + 12)[0];
      fast = sh[15] == 0;
    } else {
      // beams of 65-128: the sample's best 128 in order, handed to the winners
      // in advance (the slow path below overwrites them); the same test with
      // the beams in two waves
      uint64_t th = 0ull, tl = 0ull;
      block_top128(cbuf, 4 * W, cbuf + kCBuf - 384, th, tl);
      if (wave == 0) {
        const uint64_t tw = readlane_u64(tl, W - 65);
        win[tid] = th;   // (wave 0: tid is the lane)
        if (64 + tid < W) win[64 + tid] = tl;
        const int cnt = __popcll(__ballot(th != 0ull)) + __popcll(__ballot(64 + tid < W && tl != 0ull));
        if (tid == 0) {
          reinterpret_cast<unsigned long long*>(sh + 12)[0] = tw;
          sh[4] = cnt;
        }
      }
      __syncthreads();
      tau = reinterpret_cast<unsigned long long*>(sh + 12)[0];
      const float twk = tau != 0ull ? comp_key(tau) : -__builtin_inff();
      if (tid < W && n3 > kNeg && !(n3 < twk)) sh[15] = 1;
      __syncthreads();
      fast = sh[15] == 0;
    }
    int nw;
    bool ranked = false;   // win[0, nw) already holds the winners in rank order
    if (fast) {
      nw = sh[4];
      ranked = true;
    } else {
    // each live beam's place h - 1 among the beams' bests (in s_lim until the
    // beam overwrites it below)
    rank_keys(s_head, W, kb64, [&](int r, uint64_t x) { s_lim[comp_id(x) >> kIdShift] = r; });
    __syncthreads();
    if (tau == 0ull) tau = 1ull;   // fewer than W in the sample: no bound
    const float tau_key = comp_key(tau);
    // per beam: open ranks considered (at most W - h + 1 open ones when its
    // best is the h-th best of the beams), and the leading ones whose key
    // reaches the bound
    if (tid < W) {
      const int k = tid;
      const uint64_t mine = s_head[k];
      int lim = 0, reach = 0;
      if (mine != 0ull) {
        const int h = 1 + s_lim[k];
        // the (W - h + 1)-th open rank: every exclusion word loaded at once,
        // the word holding it found by running popcounts, the bit inside it by
        // halving (all ranks below K when fewer are open)
        const int want = W - h + 1;
        uint32_t wd[kExw];
#pragma unroll
        for (int w = 0; w < kExw; w++) {
          const int nb = K - w * 32;
          const uint32_t valid = nb >= 32 ? ~0u : (nb <= 0 ? 0u : ((1u << nb) - 1u));
          wd[w] = ~s_exm[k * kExw + w] & valid;
        }
        lim = K;
        int acc = 0, fr = 0, fbase = -1;
        uint32_t fv = 0u;
#pragma unroll
        for (int w = 0; w < kExw; w++) {
          const int c = __popc(wd[w]);
          if (fbase < 0 && acc + c >= want) {
            fbase = w * 32;
            fv = wd[w];
            fr = want - acc;   // 1-based among the word's set bits
          }
          acc += c;
        }
        if (fbase >= 0) {
          int pos = 0;
#pragma unroll
          for (int sh2 = 16; sh2 >= 1; sh2 >>= 1) {
            const int c = __popc(fv & ((1u << sh2) - 1u));
            if (c < fr) {
              fr -= c;
              pos += sh2;
              fv >>= sh2;
            }
          }
          lim = fbase + pos + 1;
        }
        const float A = s_A[k];
        // a label past the last one considered whose score rounds to the same
        // value outranks the considered labels of that score with larger ids:
        // the limit moves past the last such label (in a run of equal
        // log-probabilities the ids already ascend, and nothing moves)
        if (lim < K) {
          const float kl = A + Rl[lim - 1];
          if (kl > kNeg && A + Rl[lim] == kl) {
            const int rs = tie_run_start(A, Rl, lim - 1), re = tie_run_end(A, Rl, lim - 1, K);
            if (Rl[rs] != Rl[re - 1]) {
              int lmax = Rc[lim - 1];
              for (int i = rs; i < lim - 1; i++) lmax = max(lmax, Rc[i]);
              int nl = lim;
              for (int i = lim; i < re; i++)
                if (Rc[i] < lmax) nl = i + 1;
              lim = nl;
            }
          }
        }
        // keys A + Rl[r] do not increase with r: binary search of the first
        // rank below the bound
        int lo = 0, hi = lim;
        if (tau > 1ull) {
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (A + Rl[mid] >= tau_key) lo = mid + 1;
            else hi = mid;
          }
          reach = lo;
        } else {
          reach = lim;
        }
      }
      s_lim[k] = lim;
      s_bslot[k] = mine != 0ull ? 2 + reach : 0;   // (reused: survivor items of the beam)
    }
    __syncthreads();
    if (tid < 64) {
      const int k0 = 2 * tid, k1 = 2 * tid + 1;
      const int n0 = k0 < W ? s_bslot[k0] : 0;
      const int n1 = k1 < W ? s_bslot[k1] : 0;
      const int incl = wave_incl_scan(n0 + n1);
      const int ex = incl - n0 - n1;
      if (k0 < W) s_offs[k0] = ex;
      if (k1 < W) s_offs[k1] = ex + n0;
      if (tid == 63) {
        sh[3] = incl;
        s_offs[W] = incl;   // end sentinel
      }
    }
    __syncthreads();
    const int nsurv = sh[3];
    if (nsurv <= kCBuf) {
      // ---- top W (sec. 3.4.4 / 3.4.5) among the candidates at or above the
      // bound, each beam writing its own
      for (int i = tid; i < nsurv; i += kNT) {
        // the beam of item i: the last k with s_offs[k] <= i
        int lo = 0, hi = W - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_offs[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        const int k = lo, j = i - s_offs[k];
        // every read is made and the values selected: selecting between the
        // reads would turn into a load through a selected generic pointer,
        // with `blank` spilled to scratch memory
        const int r = j >= 2 ? j - 2 : 0;
        const float kbv = s_kb[k], kcv = s_kc[k], lkey = s_A[k] + Rl[r];
        const int lastv = s_last[k], rcv = Rc[r];
        const uint32_t exw = s_exm[k * kExw + (r >> 5)];
        const float key = j == 0 ? kbv : (j == 1 ? kcv : lkey);
        const int c = j == 0 ? blank : (j == 1 ? lastv : rcv);
        const bool ex = j >= 2 && ((exw >> (r & 31)) & 1u);
        const uint64_t x =
            (!ex && key > kNeg) ? compose(key, (uint32_t)((k << kIdShift) | c)) : 0ull;
        cbuf[i] = x >= tau ? x : 0ull;
      }
      if (tid == 0) sh[4] = 0;
      __syncthreads();
      if (W <= 64 && nsurv <= 256) {
        // at most 256 survivors (the usual case for beams up to 64): their 64
        // largest in order (zeros, the candidates below the bound, come last)
        const uint64_t top = block_top64(cbuf, nsurv, cbuf + kCBuf - 384);
        if (wave == 0) {
          if (tid < W) win[tid] = top;
          const int cnt = __popcll(__ballot(tid < W && top != 0ull));
          if (tid == 0) sh[4] = cnt;
        }
        __syncthreads();
        nw = sh[4];
        ranked = true;
      } else if (nsurv <= 64 * kRankChunks) {
        // few survivors (the usual case): rank them all, in place, and keep
        // the first W (zeros, the candidates below the bound, rank last and
        // are skipped)
        rank_keys(cbuf, nsurv, cbuf, [&](int r, uint64_t x) {
          if (r < W) {
            win[r] = x;
            atomicMax(&sh[4], r + 1);
          }
        });
        __syncthreads();
        nw = sh[4];
        ranked = true;
      } else {
        uint64_t xw = kth_largest<4>(nsurv, W, [&](int i) { return cbuf[i]; }, khist, ksh);
        if (xw == 0ull) xw = 1ull;   // fewer than W candidates: all of them win
        for (int i = tid; i < nsurv; i += kNT) {
          const uint64_t x = cbuf[i];
          if (x != 0ull && x >= xw) kb64[atomicAdd(&sh[4], 1)] = x;
        }
        __syncthreads();
        nw = sh[4];
      }
    } else {
      // many candidates at the bound (exact ties): every considered candidate,
      // held in registers, through a radix select
      if (tid < 64) {
        const int k0 = 2 * tid, k1 = 2 * tid + 1;
        const int n0 = k0 < W ? (s_head[k0] != 0ull ? 2 + s_lim[k0] : 0) : 0;
        const int n1 = k1 < W ? (s_head[k1] != 0ull ? 2 + s_lim[k1] : 0) : 0;
        const int incl = wave_incl_scan(n0 + n1);
        const int ex = incl - n0 - n1;
        if (k0 < W) s_offs[k0] = ex;
        if (k1 < W) s_offs[k1] = ex + n0;
        if (tid == 63) {
          sh[3] = incl;
          s_offs[W] = incl;   // end sentinel of the walk below
        }
      }
      __syncthreads();
      const int ntot = sh[3];
      if (tid == 0 && ntot > kItems * kNT) sh[10] |= kStatusAborted;   // cannot happen (bound above)
      // this thread's candidates, kept in registers
      uint64_t ck[kItems];
      {
        int k = 0;
  #pragma unroll
        for (int u = 0; u < kItems; u++) {
          const int qi = tid + u * kNT;
          uint64_t x = 0ull;
          if (qi < ntot) {
            while (s_offs[k + 1] <= qi) k++;
            const int j = qi - s_offs[k];
            // (reads made, values selected: see the sampled gather above)
            const int r = j >= 2 ? j - 2 : 0;
            const float kbv = s_kb[k], kcv = s_kc[k], lkey = s_A[k] + Rl[r];
            const int lastv = s_last[k], rcv = Rc[r];
            const uint32_t exw = s_exm[k * kExw + (r >> 5)];
            const bool ex = j >= 2 && ((exw >> (r & 31)) & 1u);
            const float key = j == 0 ? kbv : (j == 1 ? kcv : (ex ? kNeg : lkey));
            const int c = j == 0 ? blank : (j == 1 ? lastv : rcv);
            x = key > kNeg ? compose(key, (uint32_t)((k << kIdShift) | c)) : 0ull;
          }
          ck[u] = x;
        }
      }
      // ---- top W (sec. 3.4.4 / 3.4.5): radix select over the register keys
      uint64_t prefix = 0ull;
      int need = W;
      bool few = false;
      for (int shift = 56; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        const uint64_t hmask = shift == 56 ? 0ull : (~0ull << (shift + 8));
  #pragma unroll
        for (int u = 0; u < kItems; u++) {
          const uint64_t x = ck[u];
          if (x != 0ull && (x & hmask) == prefix) atomicAdd(&hist[(int)((x >> shift) & 255u)], 1);
        }
        __syncthreads();
        if (tid < 64) {
          const int lane = tid;
          const int d0 = 255 - 4 * lane;
          const int c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
          const int s = c0 + c1 + c2 + c3;
          const int incl = wave_incl_scan(s);
          const int ex = incl - s;
          const int total = __shfl(incl, 63, 64);
          if (ex < need && incl >= need) {
            int d, above;
            if (ex + c0 >= need) { d = d0; above = ex; }
            else if (ex + c0 + c1 >= need) { d = d0 - 1; above = ex + c0; }
            else if (ex + c0 + c1 + c2 >= need) { d = d0 - 2; above = ex + c0 + c1; }
            else { d = d0 - 3; above = ex + c0 + c1 + c2; }
            sh[0] = d;
            sh[1] = above;
          }
          if (lane == 0 && total < need) sh[0] = -1;
        }
        __syncthreads();
        const int d = sh[0], above = sh[1];
        __syncthreads();
        if (d < 0) {
          few = true;   // fewer than W candidates: all of them win
          break;
        }
        prefix |= (uint64_t)d << shift;
        need -= above;
      }
      const uint64_t xw = few ? 1ull : prefix;
      if (tid == 0) sh[4] = 0;
      __syncthreads();
  #pragma unroll
      for (int u = 0; u < kItems; u++) {
        const uint64_t x = ck[u];
        if (x != 0ull && x >= xw) kb64[atomicAdd(&sh[4], 1)] = x;
      }
      __syncthreads();
      nw = sh[4];
    }
    }   // (not fast)
    if (!ranked) rank_keys(kb64, nw, cbuf, [&](int r, uint64_t x) { win[r] = x; });
    if (tid < kMaxW) s_bslot[tid] = -1;
    __syncthreads();

    // ---- new state of slot r <- winner (k, c) (sec. 3.4.5)
    int k = -1, c = blank, nlen = 0, nlast = blank, nlive = 0;
    float npb = kNeg, npnb = kNeg, nsc = kNeg;
    uint32_t nh = kHashEmpty, nhp = kHashEmpty;
    if (tid < W && tid < nw) {
      const uint64_t wc = win[tid];
      const uint32_t id = comp_id(wc);
      k = (int)(id >> kIdShift);
      c = (int)(id & ((1u << kIdShift) - 1u));
      const float key = comp_key(wc);
      const int lastk = s_last[k];
      if (c == blank) {
        npb = s_ptb[k];
        npnb = s_stay[k];
      } else if (c == lastk && c != L.space) {
        npb = kNeg;
        npnb = s_lpc[k] + s_pb1[k];
      } else {
        npb = kNeg;
        npnb = row[c] + s_A[k];
      }
      if (g) {
        npb = key;
        npnb = kNeg;
      }
      nsc = key;
      nlive = 1;
      nlen = s_len[k] + (c != blank ? 1 : 0);
      nlast = c == blank ? lastk : c;
      nh = c == blank ? s_h[k] : hash_push(s_h[k], c);
      nhp = c == blank ? s_hp[k] : s_h[k];
      if (c == blank) s_bslot[k] = tid;
    }
    if (!paged) {
      // ---- tokens: row tid of parity p <- row k of parity q (+ c).  If row k
      // was itself forked from slot tid one step earlier, slot tid's row of
      // parity p already holds row k's tokens but (at most) the label that
      // fork appended, the last one of row k: it is written directly, nothing
      // is copied.  Otherwise, if slot tid was live two steps ago, its row
      // already holds the tokens that every live row then shared.
      int start = 0, dlab = -1;
      bool direct = false;
      const int klen = k >= 0 ? s_len[k] : 0;
      if (k >= 0) {
        const int oldlen = s_flen[p * kMaxW + tid];
        if (oldlen >= 0) {
          direct = s_src[q * kMaxW + k] == tid;   // then klen is oldlen or oldlen + 1
          start = min(direct ? oldlen : sh[6 + p], klen);
          if (direct && klen > oldlen) dlab = s_last[k];
        }
      }
      const int s4 = start >> 2;
      const int e4 = (klen + 3) >> 2;
      const int cnt = (k >= 0 && !direct) ? e4 - s4 : 0;
      __syncthreads();   // s_bslot complete; every read of the old state done
      // copy counts (int4 units) -> prefix sums; per destination its source
      // slot and first int4
      if (tid < kMaxW) hist[tid] = tid < W ? cnt : 0;
      if (tid < W) {
        hist[128 + tid] = k;
        s_lim[tid] = s4;
      }
      __syncthreads();
      if (tid < 64) {
        const int a = hist[2 * tid], b = hist[2 * tid + 1];
        const int incl = wave_incl_scan(a + b);
        s_offs[2 * tid] = incl - a - b;
        s_offs[2 * tid + 1] = incl - b;
        if (tid == 63) sh[5] = incl;
      }
      __syncthreads();
      {
        const int ntok4 = sh[5];
        int4* c4 = reinterpret_cast<int4*>(clist);
        const int64_t ld4 = ldc >> 2;
        // destination of this thread's first item by binary search, later ones
        // by walking forward
        int a = 0;
        if (tid < ntok4) {
          int lo = 0, hi = W - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_offs[mid] <= tid) lo = mid;
            else hi = mid - 1;
          }
          a = lo;
        }
        auto where = [&](int i, int64_t& dst, int64_t& src) {
          while (a + 1 < W && s_offs[a + 1] <= i) a++;
          const int64_t pos4 = s_lim[a] + (i - s_offs[a]);
          dst = (int64_t)(p * W + a) * ld4 + pos4;
          src = (int64_t)(q * W + hist[128 + a]) * ld4 + pos4;
        };
        // four copies per round: the loads are issued before the stores
        for (int i = tid; i < ntok4; i += 4 * kNT) {
          int64_t d0, s0, d1 = 0, s1 = 0, d2 = 0, s2 = 0, d3 = 0, s3 = 0;
          int4 v1, v2, v3;
          where(i, d0, s0);
          const int4 v0 = c4[s0];
          const bool b1 = i + kNT < ntok4, b2 = i + 2 * kNT < ntok4, b3 = i + 3 * kNT < ntok4;
          if (b1) {
            where(i + kNT, d1, s1);
            v1 = c4[s1];
          }
          if (b2) {
            where(i + 2 * kNT, d2, s2);
            v2 = c4[s2];
          }
          if (b3) {
            where(i + 3 * kNT, d3, s3);
            v3 = c4[s3];
          }
          c4[d0] = v0;
          if (b1) c4[d1] = v1;
          if (b2) c4[d2] = v2;
          if (b3) c4[d3] = v3;
        }
      }
      __syncthreads();
      if (dlab >= 0) clist[(int64_t)(p * W + tid) * ldc + klen - 1] = dlab;
      if (tid < W && k >= 0 && c != blank) clist[(int64_t)(p * W + tid) * ldc + klen] = c;
      __threadfence_block();
      __syncthreads();
    } else {
      // ---- tokens, paged (sec. 3.4.5 paged variant).  Pass 1: row tid of
      // parity p takes the pages of row k of parity q and releases the ones it
      // held; every reference is taken before any is released, so that a
      // page held by both an old and a new row never drops to zero in between.
      const int klen = k >= 0 ? s_len[k] : 0;
      const int npo = tid < W ? s_np[p * kMaxW + tid] : 0;
      const int nps = k >= 0 ? s_np[q * kMaxW + k] : 0;
      int* drow = G.row(p, tid < W ? tid : 0);
      const int* srow_k = G.row(q, k >= 0 ? k : 0);
      __syncthreads();   // s_bslot complete; every read of the old state done
      // (table entries are read eight at a time, all loads issued before any
      // is used: the tables live in global memory)
      constexpr int kB = 8;
      for (int j0 = 0; j0 < nps; j0 += kB) {
        int e[kB], o[kB];
#pragma unroll
        for (int u = 0; u < kB; u++) {
          e[u] = j0 + u < nps ? srow_k[j0 + u] : kInvalidPage;
          o[u] = j0 + u < npo ? drow[j0 + u] : kInvalidPage;
        }
#pragma unroll
        for (int u = 0; u < kB; u++)
          if (e[u] >= 0 && (j0 + u >= npo || o[u] != e[u])) atomicAdd(&G.ref[e[u]], 1);
      }
      __threadfence_block();
      __syncthreads();
      const int nmax = max(npo, nps);
      for (int j0 = 0; j0 < nmax; j0 += kB) {
        int e[kB], o[kB], left[kB];
#pragma unroll
        for (int u = 0; u < kB; u++) {
          o[u] = j0 + u < npo ? drow[j0 + u] : kInvalidPage;
          e[u] = j0 + u < nps ? srow_k[j0 + u] : kInvalidPage;
        }
        // the releases are issued together, then their old counts checked
#pragma unroll
        for (int u = 0; u < kB; u++)
          left[u] = (o[u] >= 0 && o[u] != e[u]) ? atomicSub(&G.ref[o[u]], 1) : 0;
#pragma unroll
        for (int u = 0; u < kB; u++) {
          if (j0 + u >= nmax || o[u] == e[u]) continue;
          if (left[u] == 1) {
            const int at = atomicAdd(&pgs[0], 1);
            if (at < G.npages) G.fstk[at] = o[u];
          }
          drow[j0 + u] = e[u];
        }
      }
      // Pass 2: the new label, in slot order.  It goes to offset klen mod
      // page_size of page klen / page_size: a fresh page at offset 0, else the
      // row's last page, copied first when another row still holds it.
      const bool ext = tid < W && k >= 0 && c != blank;
      const int po = klen & (G.ps - 1), pi = klen >> G.psh;
      bool fresh = false;
      int pshared = -1;
      if (ext) {
        if (po == 0) fresh = pi == nps && pi < G.mlp;
        else if (pi == nps - 1) pshared = srow_k[pi];
      }
      if (tid < W) s_pgP[tid] = pshared;
      __threadfence_block();
      __syncthreads();
      bool cow = false;
      if (pshared >= 0) {
        int before = 0;   // earlier slots appending into the same page copy it away first
        for (int s2 = 0; s2 < tid; s2++) before += s_pgP[s2] == pshared ? 1 : 0;
        const int rc = __hip_atomic_load(&G.ref[pshared], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        cow = rc - before > 1;
      }
      const bool need = fresh || cow;
      const uint64_t bm = __ballot(need);
      if ((tid & 63) == 0) pgs[4 + wave] = __popcll(bm);
      __syncthreads();
      const int ord = (wave > 0 ? pgs[4] : 0) + (wave > 1 ? pgs[5] : 0) +
                      (wave > 2 ? pgs[6] : 0) + lanes_below(bm);
      const int top = min(pgs[0], G.npages), nf = pgs[1];
      const int nalloc = pgs[4] + pgs[5] + pgs[6] + pgs[7];
      int npn = nps;
      if (need) {
        // pops in slot order: the free stack from its top, then the bump pointer
        const int pid = ord < top ? G.fstk[top - 1 - ord]
                                  : (nf + ord - top < G.npages ? nf + ord - top : kInvalidPage);
        if (pid >= 0) {
          __hip_atomic_store(&G.ref[pid], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          int* dst = G.pages + (int64_t)pid * G.ps;
          if (cow) {
            const int* src = G.pages + (int64_t)pshared * G.ps;
            for (int j = 0; j < po; j++) dst[j] = src[j];
            atomicSub(&G.ref[pshared], 1);   // stays >= 1: another row holds it
          }
          dst[po] = c;
          drow[pi] = pid;
          if (fresh) npn = nps + 1;
        } else {
          atomicOr(&sh[10], kStatusOutOfPages);   // keeps its prefix (sec. 4.2)
        }
      } else if (pshared >= 0) {
        G.pages[(int64_t)pshared * G.ps + po] = c;   // the only holder left: in place
      } else if (ext) {
        atomicOr(&sh[10], kStatusOutOfPages);   // a row already short of pages
      }
      if (tid < W) s_np[p * kMaxW + tid] = npn;
      __threadfence_block();
      __syncthreads();
      if (tid == 0) {
        const int from = min(top, nalloc);
        pgs[0] = top - from;
        pgs[1] = min(G.npages, nf + (nalloc - from));
        pgs[2] = max(pgs[2], pgs[1] - pgs[0]);
      }
    }

    // ---- structural merge parents for the next step; a blank winner whose
    // source had no live parent may find its parent prefix re-created: hash
    // lookup, then an exact token comparison
    int npar = -1;
    if (tid < W && k >= 0) {
      const int kpar = s_par[k];
      if (c != blank) npar = s_bslot[k];
      else if (kpar >= 0) npar = s_bslot[kpar];
    }
    // publish the new hashes and lengths before the lookup (old values are no
    // longer read)
    __syncthreads();
    auto tag_pos = [](uint64_t tg) {
      return (int)((((uint32_t)tg ^ (uint32_t)(tg >> 32)) * 0x9e3779b1u) >> 24);
    };
    const uint64_t mytag = nlive ? (((uint64_t)(uint32_t)nlen << 32) | nh) : ~0ull;
    if (tid < W) {
      s_h[tid] = nh;
      s_hp[tid] = nhp;
      s_len[tid] = nlen;
      s_live[tid] = nlive;
      s_tag[tid] = mytag;
    }
    hist[tid] = -1;   // open-addressing table (length, hash) -> slot
    __syncthreads();
    if (tid < W && nlive) {
      int pos = tag_pos(mytag);
      while (atomicCAS(&hist[pos], -1, tid) != -1) pos = (pos + 1) & 255;
    }
    __syncthreads();
    if (tid < W && k >= 0 && c == blank && npar < 0 && nlen >= 1) {
      const uint64_t want = ((uint64_t)(uint32_t)(nlen - 1) << 32) | nhp;
      // at most W of the 256 entries are used, so every probe ends at an empty one
      for (int pos = tag_pos(want); hist[pos] >= 0 && npar < 0; pos = (pos + 1) & 255) {
        {
          const int i = hist[pos];
          if (s_tag[i] != want || i == tid) continue;
          const int n = nlen - 1;
          bool eq = true;
          if (paged) {
            // the first nlen - 1 tokens, page by page; a page both rows hold is equal
            const int* ta = G.row(p, tid);
            const int* tb = G.row(p, i);
            for (int b0 = 0; b0 < n && eq; b0 += G.ps) {
              const int ea = ta[b0 >> G.psh], eb = tb[b0 >> G.psh];
              if (ea == eb && ea >= 0) continue;
              if (ea < 0 || eb < 0) {
                eq = false;
                break;
              }
              const int m = min(G.ps, n - b0);
              for (int j = 0; j < m && eq; j++)
                eq = G.pages[(int64_t)ea * G.ps + j] == G.pages[(int64_t)eb * G.ps + j];
            }
          }
          // flat: the first nlen - 1 tokens of both rows, 16 per round (rows are
          // 16-byte aligned: ldc is a multiple of 4)
          const int4* ra = reinterpret_cast<const int4*>(clist + (int64_t)(p * W + tid) * ldc);
          const int4* rb = reinterpret_cast<const int4*>(clist + (int64_t)(p * W + i) * ldc);
          for (int x4 = 0; !paged && x4 * 4 < n && eq; x4 += 4) {
#pragma unroll
            for (int u2 = 0; u2 < 4; u2++) {
              const int b = (x4 + u2) * 4;
              if (b < n) {
                const int4 va = ra[x4 + u2], vb = rb[x4 + u2];
                eq = eq && (va.x == vb.x) && (b + 1 >= n || va.y == vb.y) &&
                     (b + 2 >= n || va.z == vb.z) && (b + 3 >= n || va.w == vb.w);
              }
            }
          }
          nver++;
          if (eq) npar = i;
        }
      }
    }
    __syncthreads();
    if (tid < W) {
      s_pb[tid] = npb;
      s_pnb[tid] = npnb;
      s_sc[tid] = nsc;
      s_last[tid] = nlast;
      s_par[tid] = npar;
      s_src[p * kMaxW + tid] = k;
      s_flen[p * kMaxW + tid] = nlive ? nlen : -1;
    }
    if (!paged && (step & 15) == 15) {
      // grow the common prefix of the live rows of parity p by up to 64
      // positions (it never shrinks: every row extends a row of the step before)
      if (tid < 64) {
        const int r0 = 2 * tid, r1 = 2 * tid + 1;
        const bool l0 = r0 < W && s_live[r0], l1 = r1 < W && s_live[r1];
        int mn = min(l0 ? s_len[r0] : 0x7fffffff, l1 ? s_len[r1] : 0x7fffffff);
#pragma unroll
        for (int m = 32; m > 0; m >>= 1) mn = min(mn, __shfl_xor(mn, m, 64));
        const uint64_t lm = __ballot(l0 || l1);
        if (tid == 0) {
          sh[8] = mn;
          int first = -1;
          if (lm) {
            const int ln = __ffsll((long long)lm) - 1;
            first = s_live[2 * ln] ? 2 * ln : 2 * ln + 1;
          }
          sh[11] = first;
          reinterpret_cast<unsigned long long*>(sh + 12)[0] = ~0ull;
        }
      }
      __syncthreads();
      const int first = sh[11];
      if (first >= 0) {
        const int c0 = max(sh[6], sh[7]);
        const int pos = c0 + (tid & 63);
        bool ok = pos < sh[8];
        if (ok) {
          const int ref = clist[(int64_t)(p * W + first) * ldc + pos];
          for (int r = tid >> 6; r < W; r += 4)
            if (s_live[r]) ok = ok && clist[(int64_t)(p * W + r) * ldc + pos] == ref;
        }
        const uint64_t okm = __ballot(ok);
        if ((tid & 63) == 0)
          atomicAnd(reinterpret_cast<unsigned long long*>(sh + 12), (unsigned long long)okm);
        __syncthreads();
        if (tid == 0) {
          const uint64_t all = reinterpret_cast<unsigned long long*>(sh + 12)[0];
          sh[6 + p] = c0 + (all == ~0ull ? 64 : __ffsll((long long)~all) - 1);
        }
      }
    }
    __syncthreads();
    last_t = t;
    step++;
    cf = cnext;
  }

  if (STREAM) {
    // keep the beam state for the stream's next chunk
    if (nver) atomicAdd(&sh[9], nver);
    if (tid < kMaxW) {
      wst[kWPb * kMaxW + tid] = s_pb[tid];
      wst[kWPnb * kMaxW + tid] = s_pnb[tid];
      wst[kWSc * kMaxW + tid] = s_sc[tid];
      wsti[kWLast * kMaxW + tid] = s_last[tid];
      wsti[kWLen * kMaxW + tid] = s_len[tid];
      wsti[kWPar * kMaxW + tid] = s_par[tid];
      wsti[kWH * kMaxW + tid] = (int)s_h[tid];
      wsti[kWHp * kMaxW + tid] = (int)s_hp[tid];
      wsti[kWLive * kMaxW + tid] = s_live[tid];
      wsti[kWSrc0 * kMaxW + tid] = s_src[tid];
      wsti[kWSrc1 * kMaxW + tid] = s_src[kMaxW + tid];
      wsti[kWFlen0 * kMaxW + tid] = s_flen[tid];
      wsti[kWFlen1 * kMaxW + tid] = s_flen[kMaxW + tid];
      wsti[kWNp0 * kMaxW + tid] = s_np[tid];
      wsti[kWNp1 * kMaxW + tid] = s_np[kMaxW + tid];
    }
    __syncthreads();
    if (tid == 0) {
      hdr[kStep] = step;
      hdr[kLastT] = last_t;
      hdr[kFrames] = frame0 + P.T;
      hdr[kStatus] = sh[10];
      hdr[kVerifies] += sh[9];
      hdr[kCpl0] = sh[6];
      hdr[kCpl1] = sh[7];
      hdr[kFreeTop] = pgs[0];
      hdr[kNextFree] = pgs[1];
      hdr[kPagesHigh] = pgs[2];
    }
    return;
  }

  wide_nbest(P, row_i, W, step, ldc, clist, paged, G, s_live, s_sc, s_len, hist);
  if (nver) atomicAdd(&sh[9], nver);
  __syncthreads();
  if (tid == 0) {
    hdr[kStep] = step;
    hdr[kLastT] = last_t;
    hdr[kStatus] = sh[10];
    hdr[kVerifies] = sh[9];
    hdr[kPagesHigh] = paged ? pgs[2] : 0;
    hdr[kFallbacks] = 0;
    hdr[kCpl0] = hdr[kCpl1] = hdr[kPcp0] = hdr[kPcp1] = 0;
    hdr[kFrames] = 0;
  }
}

// read_state for streams of beams above kMaxBeam: the N best of each listed
// stream from its kept beam state, without changing it.
__global__ __launch_bounds__(kNT) void read_state_wide_kernel(Params P) {
  __shared__ int out_rank[kNT];
  __shared__ int s_live[kMaxW];
  __shared__ int s_len[kMaxW];
  __shared__ float s_sc[kMaxW];
  const Layout L = P.L;
  const int tid = threadIdx.x;
  const int srow = P.rows ? P.rows[blockIdx.x] : (int)blockIdx.x;
  if (srow < 0 || srow >= P.num_rows) return;
  const char* base = P.state + (int64_t)srow * L.row_bytes;
  const int step = reinterpret_cast<const int*>(base)[kStep];
  const float* wst = reinterpret_cast<const float*>(base + L.o_wide);
  const int* wsti = reinterpret_cast<const int*>(base + L.o_wide);
  if (tid < kMaxW) {
    // a stream that has decoded nothing holds the empty hypothesis (sec. 13)
    s_live[tid] = step > 0 ? wsti[kWLive * kMaxW + tid] : (tid == 0 ? 1 : 0);
    s_len[tid] = step > 0 ? wsti[kWLen * kMaxW + tid] : 0;
    s_sc[tid] = step > 0 ? wst[kWSc * kMaxW + tid] : (tid == 0 ? 0.0f : kNeg);
  }
  __syncthreads();
  const WidePager G = wide_pager(L, const_cast<char*>(base));
  wide_nbest(P, (int)blockIdx.x, L.W, step, L.ldc, reinterpret_cast<const int*>(base + L.o_clist),
             L.paged != 0, G, s_live, s_sc, s_len, out_rank);
}

}  // namespace wide
}  // namespace ctcpb
