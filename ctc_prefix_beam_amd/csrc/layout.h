// layout.h -- per-row (offline) / per-stream (streaming) state region.
//
// Offline workspaces and streaming state blobs are arrays of identical row
// regions whose layout is a pure function of the configuration and the token
// capacity, so the host rebuilds every pointer from the dimensions and never
// reads device memory (the page's StreamingState idea, sec. 4.3 / 5).
//
//   header      64 x int32   step, last frame, counters, parity bookkeeping
//   beam arrays kMaxBeam x {pb, pnb, score, len, last token, parent slot,
//               second-to-last token, live, prefix hash, parent-prefix hash}
//   wide        beams above kMaxBeam: kWideArrays x kMaxBeamWide words of the
//               wide decoder's beam state
//   sel         cap_sel x int32     offline: selected frame indices
//   flat:       clist[2][beam][ldc] int32 tokens, double-buffered by parity
//               (ldc = cap rounded up to a multiple of 4); beams up to 32: the
//               token store's lineage and common-prefix bounds (StoreArrays)
//   paged:      table[2][beam][max_lp] int32 page ids (-1 none),
//               refcount[num_pages], free stack[num_pages],
//               pages[num_pages][page_size] int32 tokens,
//               tail[2][beam][page_size] int32: each beam's partial last page,
//               tlen[2][32] int32: valid leading entries of each table row
#pragma once
#include <stdint.h>

namespace ctcpb {

constexpr int kMaxBeam = 32;     // widest beam of the fused decoder
constexpr int kMaxBeamWide = 128;   // widest beam of the wide decoder

// Beam state of the wide decoder (beams above kMaxBeam) kept between the
// chunks of a stream: arrays of kMaxBeamWide entries, in this order.
enum WideArray {
  kWPb = 0, kWPnb, kWSc, kWLast, kWLen, kWPar, kWH, kWHp, kWLive, kWSrc0, kWSrc1, kWFlen0,
  kWFlen1, kWNp0, kWNp1, kWideArrays
};
constexpr int kHdrInts = 64;
constexpr int kInvalidPage = -1;

enum HeaderField {
  kStep = 0,      // frames decoded so far (steps)
  kLastT,         // frame index of the last decoded frame, -1 before any
  kNSel,          // offline: number of selected frames
  kStatus,        // bit 0: a paged row ran out of pages
  kCpl0,          // common token prefix of all live beams, parity 0 / 1
  kCpl1,
  kPcp0,          // leading full pages shared by all live beams, parity 0 / 1
  kPcp1,
  kNextFree,      // paged: bump pointer
  kFreeTop,       // paged: free-stack depth
  kLive0,         // live-slot bitmask written at parity 0 / 1
  kLive1,
  kPagesHigh,     // paged: high-water mark of pages in use
  kFallbacks,     // steps that needed the full beam x vocab selection
  kVerifies,      // exact token comparisons made for the merge test
  kFrames,        // streaming: frames given so far, decoded or not (the next frame's index)
  // words 32..47: optional per-phase cycle counters of a diagnostics build
};

enum Status { kStatusOutOfPages = 1, kStatusAborted = 2 };

struct Layout {
  int W;          // beam
  int V;          // vocabulary
  int blank;
  int space;      // label of the space slot, -1 none (not part of the sizes)
  int cap;        // token (and frame) capacity of a row
  int ldc;        // flat: row stride of clist (cap rounded up to 4)
  int paged;      // 0 flat; paged: 1 the default pool, 2 a pool the caller sized
                  // (appends follow the page's copy-on-write rule exactly, see store_paged)
  int ps;         // page size (a power of two)
  int ps_log2;    // log2(page size)
  int max_lp;     // pages per block-table row
  int npages;     // pages per row
  int cap_sel;    // entries of sel (offline: max_T; streaming: 0)
  int64_t row_bytes;
  int64_t o_beam, o_sel, o_clist, o_tab, o_ref, o_free, o_pages, o_tail, o_tlen;
  int64_t o_wide;   // beams above kMaxBeam: the wide decoder's beam state (WideArray)
  int64_t o_sst;    // flat lists, beams up to kMaxBeam: the store wave's kept state (StoreArrays)
};

// Beam arrays inside a row region (offsets from o_beam).
struct BeamArrays {
  static constexpr int64_t pb = 0, pnb = 128, score = 256, len = 384, last = 512,
                           parent = 640, last2 = 768, live = 896, hash = 1024, phash = 1152,
                           bytes = 1280;
};

// The token store's state kept between the chunks of a stream (flat lists,
// beams up to kMaxBeam), offsets from o_sst: per parity and slot the row's
// length (-1 unknown), the source slot of its last fork and the label that
// fork appended (-1 none), as int arrays [2][kMaxBeam]; then per parity the
// W x W matrix of lower bounds on the common prefix of two rows (int16, row
// stride W, kMaxBeam^2 entries reserved each).
struct StoreArrays {
  static constexpr int64_t len = 0, src = 2 * kMaxBeam * 4, lab = 4 * kMaxBeam * 4,
                           mat = 6 * kMaxBeam * 4, mat_bytes = kMaxBeam * kMaxBeam * 2,
                           bytes = mat + 2 * mat_bytes;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

inline Layout make_layout(int W, int V, int blank, int cap, int paged, int ps, int npages_cfg,
                          int cap_sel) {
  Layout L{};
  L.W = W;
  L.V = V;
  L.blank = blank;
  L.space = -1;
  L.cap = cap;
  L.ldc = (cap + 3) & ~3;
  L.paged = paged ? (npages_cfg > 0 ? 2 : 1) : 0;
  L.ps = paged ? ps : 0;
  L.ps_log2 = 0;
  while (paged && (1 << L.ps_log2) < ps) L.ps_log2++;
  L.max_lp = paged ? (cap + ps - 1) / ps : 0;
  L.npages = paged ? (npages_cfg > 0 ? npages_cfg : W * (L.max_lp + 1)) : 0;
  L.cap_sel = cap_sel;
  int64_t off = kHdrInts * 4;
  L.o_beam = off;
  off += BeamArrays::bytes;
  L.o_wide = off;
  if (W > kMaxBeam) off += align256((int64_t)kWideArrays * kMaxBeamWide * 4);
  L.o_sel = off;
  off += align256((int64_t)cap_sel * 4);
  if (!paged) {
    L.o_clist = off;
    off += align256((int64_t)2 * W * L.ldc * 4);
    L.o_sst = off;
    if (W <= kMaxBeam) off += align256(StoreArrays::bytes);
  } else {
    L.o_tab = off;
    off += align256((int64_t)2 * W * L.max_lp * 4);
    L.o_ref = off;
    off += align256((int64_t)L.npages * 4);
    L.o_free = off;
    off += align256((int64_t)L.npages * 4);
    L.o_pages = off;
    off += align256((int64_t)L.npages * ps * 4);
    L.o_tail = off;
    off += align256((int64_t)2 * W * ps * 4);
    L.o_tlen = off;
    off += align256((int64_t)2 * kMaxBeam * 4);
  }
  // offline beams above kMaxBeam: the ranked labels of every selected frame,
  // [cap_sel][K] with K = min(V - 1, 2W + 2), at the end of the region
  if (W > kMaxBeam && cap_sel > 0) {
    const int K = V - 1 < 2 * W + 2 ? V - 1 : 2 * W + 2;
    off += align256((int64_t)cap_sel * K * 4);
  }
  L.row_bytes = align256(off);
  return L;
}

}  // namespace ctcpb
