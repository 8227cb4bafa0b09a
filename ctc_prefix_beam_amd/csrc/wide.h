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
//   - tokens are double-buffered flat lists in the workspace (sec. 3.1); merge
//     parents are tracked structurally, with a hash lookup and an exact token
//     comparison where a parent prefix may have been re-created.
#pragma once

namespace ctcpb {
namespace wide {

constexpr int kNT = 256;                  // threads per row
constexpr int kMaxW = 128;
constexpr int kMaxK = 2 * kMaxW + 2;      // ranked labels per frame
constexpr int kExw = (kMaxK + 31) / 32;   // exclusion words per beam
constexpr int kItems = 36;                // candidates per thread (>= (W(W+1)/2 + 4W) / kNT)

// LDS: fixed part at compile-time offsets, then the row and the label map.
namespace off {
constexpr int a16(int x) { return (x + 15) & ~15; }
constexpr int Rc = 0;                                   // int [kMaxK]
constexpr int Rl = Rc + a16(kMaxK * 4);                 // float [kMaxK]
constexpr int kb64 = Rl + a16(kMaxK * 4);               // u64 [kMaxK]: gathered keys
constexpr int win = kb64 + a16(kMaxK * 8);              // u64 [kMaxW]: winners in rank order
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
constexpr int exm = u64_head + kMaxW * 8;               // u32 [kMaxW][kExw]
constexpr int hist = exm + a16(kMaxW * kExw * 4);       // int [256]
constexpr int sh = hist + 256 * 4;                      // int [16] block scalars
constexpr int end = sh + 16 * 4;
}  // namespace off

// Bytes of LDS for vocabulary V (row of floats, then a 16-bit label -> rank map).
inline int lds_bytes(int V) { return off::end + off::a16(V * 4) + off::a16(V * 2); }

// Block-wide: the kth largest (1-based) nonzero 64-bit key of the items, by
// radix select over 8-bit digits; 0 when fewer than kth keys are nonzero.
// gen(i) gives item i's key for i in [0, n) (called once per item and pass).
template <typename Gen>
__device__ uint64_t kth_largest(int n, int kth, Gen gen, int* hist, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint64_t prefix = 0ull;
  int need = kth;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    const uint64_t hmask = shift == 56 ? 0ull : (~0ull << (shift + 8));
    for (int i = tid; i < n; i += kNT) {
      const uint64_t x = gen(i);
      if (x != 0ull && (x & hmask) == prefix) atomicAdd(&hist[(int)((x >> shift) & 255u)], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l (descending)
      const int d0 = 255 - 4 * lane;
      const int c0 = hist[d0], c1 = hist[d0 - 1], c2 = hist[d0 - 2], c3 = hist[d0 - 3];
      const int s = c0 + c1 + c2 + c3;
      const int incl = wave_incl_scan(s);
      const int ex = incl - s;
      const int total = __shfl(incl, 63, 64);
      int d = -1, above = 0;
      if (ex < need && incl >= need) {
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
    if (d < 0) return 0ull;
    prefix |= (uint64_t)d << shift;
    need -= above;
  }
  return prefix;
}

// Rank of buf[i] among the n distinct keys of buf (0 = largest), by counting.
__device__ __forceinline__ int rank_of(const uint64_t* buf, int n, int i) {
  const uint64_t x = buf[i];
  int r = 0;
  for (int j = 0; j < n; j++) r += buf[j] > x ? 1 : 0;
  return r;
}

__global__ __launch_bounds__(kNT, 1) void decode_wide_kernel(Params P) {
  extern __shared__ __align__(16) char smem[];
  const Layout L = P.L;
  const int W = L.W, V = L.V, blank = L.blank;
  const int tid = threadIdx.x;
  const int row_i = blockIdx.x;
  char* base = P.state + (int64_t)row_i * L.row_bytes;
  int* hdr = reinterpret_cast<int*>(base);
  const int* sel = reinterpret_cast<const int*>(base + L.o_sel);
  int* clist = reinterpret_cast<int*>(base + L.o_clist);
  const float* lp_row = P.lp + (int64_t)row_i * P.stride_b;

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
  uint32_t* s_exm = reinterpret_cast<uint32_t*>(smem + off::exm);
  int* hist = reinterpret_cast<int*>(smem + off::hist);
  int* sh = reinterpret_cast<int*>(smem + off::sh);
  float* row = reinterpret_cast<float*>(smem + off::end);
  int16_t* rmap = reinterpret_cast<int16_t*>(smem + off::end + off::a16(V * 4));

  const int nframes = hdr[kNSel];
  const int K = min(V - 1, 2 * W + 2);
  const int ldc = L.ldc;

  // fresh row: the empty hypothesis in slot 0 (sec. 13), every other slot dead
  for (int c = tid; c < V; c += kNT) rmap[c] = -1;
  if (tid < kMaxW) {
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
  }
  int last_t = -1, step = 0, prevK = 0, nver = 0;
  if (tid == 0) {
    sh[9] = 0;    // exact token comparisons
    sh[10] = 0;   // status bits
  }
  __syncthreads();

  for (int f = 0; f < nframes; f++) {
    const int t = sel[f];
    const bool g = t > last_t + 1;    // frames skipped before t (step 0: t > 0)
    const int p = step & 1, q = p ^ 1;
    // ---- stage the row; clear the previous list's label map entries
    const float* gr = lp_row + (int64_t)t * P.stride_t;
    if (P.vec4) {
      for (int i = tid; i < (V >> 2); i += kNT)
        reinterpret_cast<float4*>(row)[i] = reinterpret_cast<const float4*>(gr)[i];
    } else {
      for (int i = tid; i < V; i += kNT) row[i] = gr[i];
    }
    for (int r = tid; r < prevK; r += kNT) rmap[Rc[r]] = -1;
    __syncthreads();

    // ---- the frame's best K non-blank labels, (lp desc, label asc)
    auto lkey = [&](int c) -> uint64_t {
      return c == blank ? 0ull : compose(row[c], (uint32_t)c);
    };
    const uint64_t xk = kth_largest(V, K, lkey, hist, sh);
    if (tid == 0) sh[2] = 0;
    __syncthreads();
    for (int c = tid; c < V; c += kNT) {
      const uint64_t x = lkey(c);
      if (x != 0ull && x >= xk) kb64[atomicAdd(&sh[2], 1)] = x;
    }
    __syncthreads();
    for (int i = tid; i < K; i += kNT) {
      const int r = rank_of(kb64, K, i);
      const int c = (int)comp_id(kb64[i]);
      Rc[r] = c;
      Rl[r] = row[c];
      rmap[c] = (int16_t)r;
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
          clist[(int64_t)(0 * W + r) * ldc] = last;
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
      last_t = t;
      step++;
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
      const float lpc = has_last ? row[last] : kNeg;
      float stay = (has_last && !g) ? lpc + pnb1 : kNeg;
      const int par = lv ? s_par[k] : -1;
      if (par >= 0) {
        // the parent's extension by this beam's last label joins this beam's
        // blank slot and leaves the parent's candidates
        const int lastp = s_last[par];
        const float Ap = lse(s_pb[par], s_pnb[par]);
        const float pb1p = g ? Ap : s_pb[par];
        const float from = last == lastp ? lpc + pb1p : lpc + Ap;
        stay = lse(stay, from);
        if (last == lastp) {
          s_exc[par] = 1;
        } else {
          const int r = rmap[last];
          if (r >= 0) atomicOr(&s_exm[par * kExw + (r >> 5)], 1u << (r & 31));
        }
      }
      // the beam's own last label is its repeated-label slot, not an ordinary one
      if (has_last) {
        const int r = rmap[last];
        if (r >= 0) atomicOr(&s_exm[k * kExw + (r >> 5)], 1u << (r & 31));
      }
      const float ptb = lv ? row[blank] + A : kNeg;
      s_A[k] = A;
      s_pb1[k] = pb1;
      s_ptb[k] = ptb;
      s_stay[k] = stay;
      s_kb[k] = lv ? lse(ptb, stay) : kNeg;
      s_kc[k] = has_last ? lpc + pb1 : kNeg;
      s_lpc[k] = lpc;
    }
    __syncthreads();
    // each beam's best candidate
    if (tid < W) {
      const int k = tid;
      const bool lv = s_live[k] != 0;
      if (s_exc[k]) s_kc[k] = kNeg;
      const float kb = s_kb[k], kc = s_exc[k] ? kNeg : s_kc[k];
      uint64_t best = 0ull;
      if (lv) {
        const uint64_t cb = kb > kNeg ? compose(kb, (uint32_t)((k << kIdShift) | blank)) : 0ull;
        const uint64_t cc =
            kc > kNeg ? compose(kc, (uint32_t)((k << kIdShift) | s_last[k])) : 0ull;
        best = cb > cc ? cb : cc;
        int r0 = -1;
        for (int w = 0; w < kExw && r0 < 0; w++) {
          const uint32_t open = ~s_exm[k * kExw + w];
          if (open) r0 = w * 32 + __ffs((int)open) - 1;
        }
        if (r0 >= 0 && r0 < K) {
          const float key = s_A[k] + Rl[r0];
          const uint64_t co = key > kNeg ? compose(key, (uint32_t)((k << kIdShift) | Rc[r0])) : 0ull;
          best = best > co ? best : co;
        }
      }
      s_head[k] = best;
    }
    __syncthreads();
    // candidates considered: at most W - h + 1 open ranks of a beam whose best
    // is the h-th best of the beams, plus its two slots
    if (tid < W) {
      const int k = tid;
      const uint64_t mine = s_head[k];
      int lim = 0;
      if (mine != 0ull) {
        int h = 1;
        for (int j = 0; j < W; j++) h += s_head[j] > mine ? 1 : 0;
        int want = W - h + 1;
        int r = 0;
        while (r < K && want > 0) {
          if (!((s_exm[k * kExw + (r >> 5)] >> (r & 31)) & 1u)) want--;
          r++;
        }
        lim = r;
      }
      s_lim[k] = lim;
    }
    __syncthreads();
    if (tid < 64) {
      // prefix sums of the per-beam item counts (2 slots + lim ranks)
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
          float key;
          int c;
          if (j == 0) {
            key = s_kb[k];
            c = blank;
          } else if (j == 1) {
            key = s_kc[k];
            c = s_last[k];
          } else {
            const int r = j - 2;
            const bool ex = (s_exm[k * kExw + (r >> 5)] >> (r & 31)) & 1u;
            key = ex ? kNeg : s_A[k] + Rl[r];
            c = Rc[r];
          }
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
    const int nw = sh[4];   // <= W
    for (int i = tid; i < nw; i += kNT) win[rank_of(kb64, nw, i)] = kb64[i];
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
      } else if (c == lastk) {
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
    // ---- tokens: row tid of parity p <- row k of parity q (+ c).  If row k
    // was itself copied from slot tid one step earlier, slot tid's row of
    // parity p already holds its first s_flen[p][tid] tokens.
    int start = 0;
    const int klen = k >= 0 ? s_len[k] : 0;
    if (k >= 0 && s_src[q * kMaxW + k] == tid && s_flen[p * kMaxW + tid] >= 0)
      start = min(s_flen[p * kMaxW + tid], klen);
    const int s4 = start >> 2;
    const int e4 = (klen + 3) >> 2;
    const int cnt = k >= 0 ? e4 - s4 : 0;
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
      int a = 0;
      for (int i = tid; i < ntok4; i += kNT) {
        while (a + 1 < W && s_offs[a + 1] <= i) a++;
        const int64_t pos4 = s_lim[a] + (i - s_offs[a]);
        c4[(int64_t)(p * W + a) * ld4 + pos4] = c4[(int64_t)(q * W + hist[128 + a]) * ld4 + pos4];
      }
    }
    __syncthreads();
    if (tid < W && k >= 0 && c != blank) clist[(int64_t)(p * W + tid) * ldc + klen] = c;
    __threadfence_block();
    __syncthreads();

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
    if (tid < W) {
      s_h[tid] = nh;
      s_hp[tid] = nhp;
      s_len[tid] = nlen;
      s_live[tid] = nlive;
    }
    __syncthreads();
    if (tid < W && k >= 0 && c == blank && npar < 0 && nlen >= 1) {
      for (int i = 0; i < W; i++) {
        if (i == tid || !s_live[i] || s_len[i] != nlen - 1 || s_h[i] != nhp) continue;
        const int* ra = clist + (int64_t)(p * W + tid) * ldc;
        const int* rb = clist + (int64_t)(p * W + i) * ldc;
        bool eq = true;
        for (int x = 0; x < nlen - 1 && eq; x++) eq = ra[x] == rb[x];
        nver++;
        if (eq) {
          npar = i;
          break;
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
    __syncthreads();
    last_t = t;
    step++;
  }

  // ---- N best (sec. 3.6): live slots by (score desc, slot asc)
  const int parity = step > 0 ? (step - 1) & 1 : 0;
  const int N = P.N, mol = P.max_out_len;
  int* out_rank = hist;   // rank -> slot
  if (tid < 256) out_rank[tid] = -1;
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
    P.out_lengths[(int64_t)row_i * N + tid] = s < 0 ? 0 : s_len[s];
    P.out_scores[(int64_t)row_i * N + tid] = s < 0 ? kNeg : s_sc[s];
  }
  int* ot = P.out_tokens + (int64_t)row_i * N * mol;
  for (int i = tid; i < N * mol; i += kNT) {
    const int n = i / mol, pos = i - n * mol;
    const int s = out_rank[n];
    int v = -1;
    if (s >= 0 && pos < s_len[s]) v = step > 0 ? clist[(int64_t)(parity * W + s) * ldc + pos] : -1;
    ot[i] = v;
  }
  if (nver) atomicAdd(&sh[9], nver);
  __syncthreads();
  if (tid == 0) {
    hdr[kStep] = step;
    hdr[kLastT] = last_t;
    hdr[kStatus] = sh[10];
    hdr[kVerifies] = sh[9];
    hdr[kPagesHigh] = 0;
    hdr[kFallbacks] = 0;
    hdr[kCpl0] = hdr[kCpl1] = hdr[kPcp0] = hdr[kPcp1] = 0;
    hdr[kFrames] = 0;
  }
}

}  // namespace wide
}  // namespace ctcpb
