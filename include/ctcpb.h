/*
 * ctcpb.h -- C ABI of libctcpb.so, a batched CTC prefix beam search decoder
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the page "GPU CTC Prefix Beam Search Decoder"
 * (OASR documentation): from log_prob[B, T, V] it returns, per utterance, the
 * N best collapsed label sequences with their CTC prefix scores, offline
 * (sec. 3.7) or streaming chunk by chunk with the decoder state kept on the
 * device (sec. 8).  The calls follow the page's public API (sec. 9, 12.5, 16):
 * size queries, an offline decode, and a streaming init / chunk / read-state
 * lifecycle.
 *
 * Conventions for every call:
 *   - Pointers documented "device" are HIP device memory owned by the caller;
 *     the library never allocates, frees or keeps device memory, and keeps no
 *     host state between calls.  The configuration is passed on every call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns without synchronising; results are
 *     ready when the stream reaches that point.
 *   - Return value: CTCPB_OK (0) or an error code; ctcpb_last_error() then
 *     describes the failure (thread-local, valid until the next call on the
 *     same thread).  There is no partial success: on error nothing was
 *     enqueued, except CTCPB_ERR_DEVICE, reported when a launch fails.
 *   - Scores are float32 natural-log probabilities.  A reported slot with no
 *     hypothesis has length 0, score -FLT_MAX and tokens -1.
 */
#ifndef CTCPB_H
#define CTCPB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  CTCPB_OK = 0,
  CTCPB_ERR_INVALID = 1,     /* an argument is out of range or inconsistent */
  CTCPB_ERR_TOO_SMALL = 2,   /* workspace / state buffer smaller than required */
  CTCPB_ERR_UNSUPPORTED = 3, /* valid but not supported by this library (LDS budget, vocab
                                above 16384) */
  CTCPB_ERR_DEVICE = 4       /* a HIP launch failed */
};

enum { CTCPB_STORAGE_FLAT = 0, CTCPB_STORAGE_PAGED = 1 };

/* Decoder configuration (sec. 10 GpuDecoderConfig, sec. 11 options). */
typedef struct {
  int32_t beam;            /* beam width W, 1..128 (sec. 10); beams above 32 (the page's
                              multi-kernel path) run on a separate decoder, offline and
                              streaming, flat or paged (whose pager always follows
                              the page's copy-on-write rule, see num_pages). */
  int32_t nbest;           /* hypotheses reported per row, 1..beam */
  int32_t vocab;           /* V >= 2, at most 16384.  Beams of 1..32 keep a ring of
                              frame rows (4V bytes each) and, paged, the page tables,
                              refcounts and free stack in one CU's 160 KB of LDS;
                              configurations that do not fit return
                              CTCPB_ERR_UNSUPPORTED.  Flat storage fits up to
                              V = 14616 / 14540 / 14232 for beams 8 / 16 / 32;
                              paged storage at 1500 frames (offline max_T,
                              streaming capacity) up to 13756 / 12896 / 11180 for
                              beams 8 / 16 / 32, at 4096 frames and beam 32 up to
                              5996 (a larger page_size shrinks the tables).  Beams
                              above 32 fit every V. */
  int32_t blank_id;        /* 0 <= blank_id < vocab */
  float blank_threshold;   /* offline frame skip (sec. 3.5): frame t is decoded iff
                              log_prob[t, blank] < log(blank_threshold); >= 1 keeps
                              every frame, <= 0 keeps none.  Streaming ignores it. */
  int32_t max_out_len;     /* tokens copied per hypothesis; longer ones are truncated,
                              lengths still report the full count (sec. 13) */
  int32_t capacity;        /* streaming: frames (hence tokens) per stream, 0 = 4096;
                              later frames are ignored (sec. 13).  Offline: unused,
                              the capacity is max_T so nothing is ever cut. */
  int32_t storage;         /* CTCPB_STORAGE_FLAT: double-buffered token lists
                              (sec. 3.1, 7); CTCPB_STORAGE_PAGED: pages with
                              reference-counted prefix sharing (sec. 3.4.5, 4.2) */
  int32_t page_size;       /* paged: tokens per page, a power of two in 4..64 (0 = 16) */
  int32_t num_pages;       /* paged: pages per row/stream (0 = beam * (ceil(cap /
                              page_size) + 1), the bound of sec. 4.2), at most 32767
                              for beams up to 32 (16-bit page ids on chip).
                              A pool given here (> 0) is handed out exactly as the
                              page's allocator does (sec. 3.4.5 fork, then appends
                              in ascending slot order with copy-on-write of a page
                              another row holds; sec. 4.2 freed pages first, then
                              the bump pointer), so it runs out where the page's
                              would.  A row that runs out sets status bit 0
                              (ctcpb_row_stats [2]); the beam keeps its prefix
                              without the label, the row's outputs are then
                              unspecified (all accesses stay in its own pool) and
                              the other rows are unaffected.  With such a pool, the
                              high-water mark (ctcpb_row_stats [3]) is the smallest
                              pool that decodes the row.  The default pool (0)
                              cannot run out; beams up to 32 then also append in
                              place to a partial page that only the source row of
                              the previous step holds (same outputs, fewer pages
                              and copies), so its marks are lower. */
  int32_t space_id;        /* the space label of the optional space slot (sec. 3.4.1,
                              3.4.2), or -1 for none (the page's default); the blank
                              label also means none.  With a space label, every beam's
                              space extension scores lp[space] + logsumexp(pb, pnb),
                              also after a beam that ends in the space label, and a
                              beam ending in the space label has no non-blank stay
                              term: every space frame emits a new space token.
                              Zero-initialised configs get space_id 0, which is a
                              space slot unless blank_id is 0: set it to -1. */
} ctcpb_config;

/* Bytes of device workspace ctcpb_decode_offline needs for `batch` rows of up
 * to `max_T` frames (sec. 5 calculate_[paged_]workspace_size).  Returns
 * CTCPB_ERR_UNSUPPORTED, with nothing written, when a row of this
 * configuration does not fit one CU's LDS (see ctcpb_config.vocab). */
int ctcpb_workspace_size(const ctcpb_config* cfg, int32_t batch, int32_t max_T,
                         size_t* out_bytes);

/* Offline batch decode (sec. 3.7).
 *   log_prob     device, float32; element (b, t, c) at
 *                log_prob[b*stride_b + t*stride_t + c] (unit stride over the
 *                vocabulary, stride_t >= vocab, stride_b >= 0; 0 makes every
 *                row read the same frames); only frames t < seq_lengths[b] are
 *                read, so padding may hold anything (even NaN).  Values must
 *                be finite.  Rows are read with 16-byte loads when log_prob,
 *                stride_b and stride_t are multiples of 4 floats and vocab %
 *                4 == 0, else 4 bytes at a time.
 *   seq_lengths  device, int32 [batch]; clamped to [0, max_T] on the device.
 *   workspace    device, >= ctcpb_workspace_size bytes, 16-byte aligned; its
 *                contents on entry do not matter.  It holds the decode's
 *                state until the call completes (and its counters afterwards,
 *                see ctcpb_row_stats): calls that share a workspace must not
 *                overlap.
 *   out_tokens   device, int32 [batch][nbest][max_out_len], -1 padded
 *   out_lengths  device, int32 [batch][nbest], full hypothesis lengths
 *   out_scores   device, float32 [batch][nbest]
 * Hypotheses are reported in (score descending, slot ascending) order.  A row
 * with no decodable frame reports the empty hypothesis at score 0 (sec. 13).
 * No host synchronisation happens inside the call.  Per-row status bits
 * (ctcpb_row_stats [2]) flag rows whose outputs are not a complete decode:
 * value 1, a paged row ran out of pages; value 2, the row's decode was abandoned
 * (a bounded internal wait between the kernel's wave roles gave up, which a
 * correct launch never reaches) and its outputs hold the hypotheses of the
 * last completed step or are unspecified. */
int ctcpb_decode_offline(const ctcpb_config* cfg, const float* log_prob, int64_t stride_b,
                         int64_t stride_t, int32_t batch, int32_t max_T,
                         const int32_t* seq_lengths, void* workspace, size_t workspace_bytes,
                         int32_t* out_tokens, int32_t* out_lengths, float* out_scores,
                         void* stream);

/* Size of the fixed device scratch of ctcpb_decode_offline_noalloc. */
#define CTCPB_NOALLOC_SCRATCH_BYTES (64u << 20)

/* ctcpb_decode_offline without a caller workspace and without any device
 * memory allocation, for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a fixed array of CTCPB_NOALLOC_SCRATCH_BYTES bytes of device
 * memory inside the library, one per GPU, held until the process ends.
 *   - Runs on the calling thread's current device; `stream` (NULL = the
 *     default stream) must belong to that device (CTCPB_ERR_INVALID otherwise).
 *   - A decode whose ctcpb_workspace_size exceeds the scratch is refused with
 *     CTCPB_ERR_TOO_SMALL before anything is enqueued (decode fewer rows per
 *     call).
 *   - Every call on one GPU uses that GPU's one array: calls that may overlap
 *     in time on one GPU (other streams, other threads) race and must be
 *     ordered by the caller.  ctcpb_row_stats cannot read this scratch.
 * Arguments, outputs and errors otherwise as ctcpb_decode_offline. */
int ctcpb_decode_offline_noalloc(const ctcpb_config* cfg, const float* log_prob,
                                 int64_t stride_b, int64_t stride_t, int32_t batch,
                                 int32_t max_T, const int32_t* seq_lengths, int32_t* out_tokens,
                                 int32_t* out_lengths, float* out_scores, void* stream);

/* Bytes of a streaming state blob holding `num_streams` independent streams
 * (sec. 5 calculate_[paged_]state_buffer_size).  Returns
 * CTCPB_ERR_UNSUPPORTED, with nothing written, when a stream of this
 * configuration does not fit one CU's LDS (see ctcpb_config.vocab). */
int ctcpb_state_size(const ctcpb_config* cfg, int32_t num_streams, size_t* out_bytes);

/* Put every stream of the blob in the fresh state (no frame decoded; reads
 * back the empty hypothesis).  state: device, >= ctcpb_state_size bytes,
 * 16-byte aligned (every call that takes the blob checks this). */
int ctcpb_stream_init(const ctcpb_config* cfg, void* state, size_t state_bytes,
                      int32_t num_streams, void* stream);

/* Reset the listed streams to the fresh state.  rows: device int32[n_rows]
 * stream indices in [0, num_streams) (duplicates not allowed), or NULL for
 * streams 0..n_rows-1. */
int ctcpb_stream_reset(const ctcpb_config* cfg, void* state, size_t state_bytes,
                       int32_t num_streams, const int32_t* rows, int32_t n_rows, void* stream);

/* Decode one chunk of frames for n_rows streams at once (sec. 3.4.8 / 3.4.9):
 * row i of log_prob_chunk (element (i, t, c) at i*stride_row + t*stride_t + c,
 * device float32, finite; stride_t >= vocab, stride_row >= 0) continues stream
 * rows[i] (NULL: stream i; distinct indices required).  Every frame is decoded (no skipping); frames past a
 * stream's capacity are ignored.  The state stays on the device; nothing is
 * read back.  Same as ctcpb_stream_chunk_ex with no mask and no start frame. */
int ctcpb_stream_chunk(const ctcpb_config* cfg, void* state, size_t state_bytes,
                       int32_t num_streams, const float* log_prob_chunk, int64_t stride_row,
                       int64_t stride_t, int32_t chunk_T, const int32_t* rows, int32_t n_rows,
                       void* stream);

/* ctcpb_stream_chunk gated by a speech mask and/or numbered from caller-given
 * frame indices (sec. 9 ctc_beam_search_chunk with is_speech_mask and
 * start_frame_idx; sec. 12: skipped frames bypass the decoder).
 *   is_speech    device uint8 [n_rows][chunk_T] (row i for stream rows[i]), or
 *                NULL: frame t of row i is decoded iff is_speech[i*chunk_T + t]
 *                is nonzero; other frames are skipped but counted.
 *   start_frame  device int32 [n_rows] (>= 0), or NULL: frame t of row i is
 *                frame number start_frame[i] + t of its stream; NULL uses the
 *                stream's own count of frames given so far.
 * A decoded frame whose number exceeds the previous decoded one by more than
 * one takes the gap rule of an offline skip (sec. 3.3 / 3.4 need_add_blank).
 * Afterwards a stream's frame count is its chunk's first frame number plus
 * chunk_T.  Frames past a stream's capacity (in decoded frames) are ignored.
 * Other arguments and errors as ctcpb_stream_chunk. */
int ctcpb_stream_chunk_ex(const ctcpb_config* cfg, void* state, size_t state_bytes,
                          int32_t num_streams, const float* log_prob_chunk, int64_t stride_row,
                          int64_t stride_t, int32_t chunk_T, const uint8_t* is_speech,
                          const int32_t* start_frame, const int32_t* rows, int32_t n_rows,
                          void* stream);

/* One frame for n_rows streams (sec. 9 ctc_beam_search_step with
 * actual_frame_index): row i of log_prob_frame (device float32, element
 * (i, c) at i*stride_row + c) is decoded as frame number frame_index[i] of
 * stream rows[i] (device int32 [n_rows], >= 0; NULL: the stream's own frame
 * count).  Equivalent to ctcpb_stream_chunk_ex with chunk_T = 1,
 * is_speech = NULL and start_frame = frame_index. */
int ctcpb_stream_step(const ctcpb_config* cfg, void* state, size_t state_bytes,
                      int32_t num_streams, const float* log_prob_frame, int64_t stride_row,
                      const int32_t* frame_index, const int32_t* rows, int32_t n_rows,
                      void* stream);

/* Report the current N best of the listed streams (sec. 8 read_state) without
 * changing them.  Outputs as in ctcpb_decode_offline with batch = n_rows. */
int ctcpb_read_state(const ctcpb_config* cfg, const void* state, size_t state_bytes,
                     int32_t num_streams, const int32_t* rows, int32_t n_rows,
                     int32_t* out_tokens, int32_t* out_lengths, float* out_scores,
                     void* stream);

/* Per-row counters a decode left in an offline workspace (max_T = the max_T
 * of that decode) or in a streaming state blob (max_T = 0), for diagnostics:
 * out (device int32 [num_rows][8]) receives per row
 *   [0] frames decoded  [1] offline: frames selected; streaming: frames
 *   given so far (the next frame's number)  [2] status bits (value 1: a
 *   paged row ran out of pages; value 2: the row's decode was abandoned
 *   when a bounded wait inside the kernel gave up, so its outputs are not a
 *   complete decode; stream_reset clears both)  [3] paged: most pages in use at once
 *   [4] steps that needed the full beam x vocab selection  [5] exact token
 *   comparisons made for the merge test  [6] common token prefix of the live
 *   beams (flat)  [7] leading pages shared by every live beam (paged). */
int ctcpb_row_stats(const ctcpb_config* cfg, const void* buf, size_t buf_bytes, int32_t num_rows,
                    int32_t max_T, int32_t* out, void* stream);

/* Human-readable description of the last error on this thread ("" if none). */
const char* ctcpb_last_error(void);

/* Library build identifier, e.g. "ctcpb 0.1 gfx950". */
const char* ctcpb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CTCPB_H */
