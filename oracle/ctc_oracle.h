/* ctc_oracle.h -- interface of the CPU reference decoder (test infrastructure
 * only; see ctc_oracle.c).  All buffers are host memory owned by the caller. */
#ifndef CTC_ORACLE_H
#define CTC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

float oracle_exp(float x);     /* x in [-80, 0] */
float oracle_log1p(float x);   /* x in [0, 1]   */
float oracle_lse(float a, float b);
float oracle_log_threshold(float threshold);

/* exp (op 0), log1p (op 1) or the quotient x / (2 + x) (op 2) of the floats
 * with bit patterns first_bits .. first_bits + n - 1, or lse(a[i], b[i])
 * (op 3), into out[0 .. n). */
void oracle_math_sweep(int op, uint32_t first_bits, int64_t n, const float *a, const float *b,
                       float *out);

/* Frame selection of one row: writes the selected frame indices (ascending)
 * to sel and returns their count. */
int oracle_select_frames(const float *lp_row, int64_t stride_t, int len, int blank,
                         float threshold, int *sel);

/* Offline decode.  log_prob[b, t, c] at b*stride_b + t*stride_t + c.
 * Outputs: out_tokens[batch][nbest][max_out_len] (-1 padded),
 * out_lengths[batch][nbest], out_scores[batch][nbest].  Returns 0, or 1 on
 * an invalid argument. */
int oracle_decode(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                  int max_T, const int *seq_lengths, int beam, int nbest, int vocab,
                  int blank, float threshold, int max_out_len, int *out_tokens,
                  int *out_lengths, float *out_scores);

/* The same with a space slot for label `space` (-1 or the blank: none). */
int oracle_decode_sp(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                     int max_T, const int *seq_lengths, int beam, int nbest, int vocab,
                     int blank, float threshold, int max_out_len, int *out_tokens,
                     int *out_lengths, float *out_scores, int space);

/* Streaming: one stream, frames fed in chunks (optionally gated by a speech
 * mask, and from a caller-given frame index). */
typedef struct OracleStream OracleStream;
OracleStream *oracle_stream_new(int beam, int vocab, int blank, int capacity);
OracleStream *oracle_stream_new_sp(int beam, int vocab, int blank, int capacity, int space);
void oracle_stream_free(OracleStream *st);
void oracle_stream_reset(OracleStream *st);
int oracle_stream_feed(OracleStream *st, const float *frames, int64_t stride_t, int n_frames);
int oracle_stream_feed_ex(OracleStream *st, const float *frames, int64_t stride_t, int n_frames,
                          const unsigned char *is_speech, int start_frame);
int oracle_stream_frame_count(const OracleStream *st);

/* Page accounting of the paged variant (see ctc_oracle.c): a stream that
 * counts pages as the page's allocator hands them out; out[0] most pages in
 * use at once, out[1] 1 if a pop found nothing, out[2] the step of the first
 * such pop (-1).  num_pages 0: the default pool. */
OracleStream *oracle_stream_new_paged(int beam, int vocab, int blank, int capacity, int space,
                                      int page_size, int num_pages);
void oracle_stream_pages(const OracleStream *st, int *out);
int oracle_decode_pages(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                        int max_T, const int *seq_lengths, int beam, int vocab, int blank,
                        float threshold, int space, int page_size, int num_pages, int *out);
int oracle_page_model_run(int beam, int page_size, int num_pages, int cap, int blank, int nseed,
                          int nsteps, const int *src, const int *lab, int *used, int *out);
int oracle_stream_step_count(const OracleStream *st);
void oracle_stream_read(const OracleStream *st, int nbest, int max_out_len, int *out_tokens,
                        int *out_lengths, float *out_scores);

#ifdef __cplusplus
}
#endif
#endif
