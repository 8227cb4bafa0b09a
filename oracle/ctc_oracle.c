/*
 * ctc_oracle.c -- plain CPU reference ("oracle") of batched CTC prefix beam
 * search.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP decoder.  Only
 * the tests, the smoke check and the benchmark's cpu_baseline leg load it; the
 * decoder library never links, loads or calls it, and the two share no source.
 *
 * Source of the method: the page "GPU CTC Prefix Beam Search Decoder" (OASR
 * documentation, chiendb97.github.io/oasr/ctc_decoder_gpu).  Section numbers
 * below are that page's.  Everything is done the slow, obvious way: for every
 * step the full beam x vocab tables ptable / ptablen are built (sec. 3.4.1,
 * 3.4.2), every ordered beam pair is tested for the merge by comparing tokens
 * (sec. 3.4.3), and all live candidates are sorted to pick the survivors
 * (sec. 3.4.4 / 3.4.5).  Scores are float32, as the page fixes them
 * (log_prob is float32, pprev is a float2, score a float).
 *
 * Readings taken where the page is silent or ambiguous:
 *   - NEG (the page's NEG_INF) is -FLT_MAX; the 0xcc memset pattern the page
 *     mentions only pre-fills tables that are overwritten before use.
 *   - logsumexp is the page's max + log(1 + exp(-|a-b|)) written as
 *     m + log1p(exp(d)), d = min - max, with exp and log1p defined below
 *     (fixed float32 operation sequences from named published methods) and
 *     the correction dropped when d < -80 (every intermediate stays normal).
 *   - Ties in the top-K are broken by ascending flat id k*V + c (the fused
 *     path's order, sec. 3.4.6); ties in the step-0 vocabulary ranking by
 *     ascending char id.
 *   - need_add_blank at step s means "frames were skipped right before the
 *     frame of step s" (t > t_prev + 1; step 0: first_t > 0), and it is
 *     applied wherever the page names it: the collapse of pprev before the
 *     tables (sec. 3.4), the blank-slot rule (sec. 3.4.2) and the pprev reset
 *     of the winners (sec. 3.4.5), as well as the step-0 seeding (sec. 3.3).
 *     PARITY UNPINNED for decodes that skip frames: no closed form exists for
 *     this rule; it is checked against hand-worked cases only.
 *   - Slots that no candidate fills are dead: score NEG, no tokens; they never
 *     extend, never merge and are never reported.
 *   - Offline, the token capacity is the row's frame count, so no hypothesis
 *     is ever cut; max_out_len only truncates the copy into out_tokens while
 *     out_lengths reports the full count (sec. 13).  Streaming, a stream
 *     decodes at most `capacity` frames; later frames are ignored (sec. 13).
 *   - Streaming frame indices: chunk frame f is frame start + f, where start
 *     is the caller's start frame when given (sec. 9, ctc_beam_search_chunk's
 *     start_frame_idx, or the per-frame step's actual_frame_index) and the
 *     count of frames given so far otherwise.  A frame that the speech mask
 *     marks 0 is not decoded but is counted, so the next decoded frame takes
 *     the gap rule above, exactly as after an offline skip.
 *   - Final hypotheses are reported in (score desc, slot asc) order; positions
 *     past a hypothesis' length and dead hypotheses' tokens are -1.
 *   - Space slot (optional, sec. 3.4.1 / 3.4.2): the space label is skipped
 *     by the ordinary extension loop and scored as lp[space] + logsumexp(pb,
 *     pnb) for every beam, also one that already ends in it; a beam ending
 *     in the space label therefore has no non-blank stay term (NEG).  The
 *     result is prefix search under the collapse in which every space frame
 *     emits a new space token.
 *   - Paged variant, page accounting (sec. 3.4.5 paged variant, sec. 4.2):
 *     an optional model that follows the page's allocator along the decode
 *     and counts pages; tokens stay in the flat lists.  Per step, pass 1
 *     forks every new row onto its source's pages and releases the pages it
 *     held, a page being freed when no row refers to it any more (the page's
 *     per-entry release and acquire, read as never freeing a page a new row
 *     takes); pass 2 appends each new label in ascending slot order: a label
 *     that starts a page pops a page, one that goes into a partial page whose
 *     reference count is above 1 pops a page for the copy and drops one
 *     reference from the shared page, otherwise it writes in place.  Pops
 *     take the LIFO stack of freed pages first, then the bump pointer, and
 *     give nothing past the row's pool: the beam then keeps its prefix
 *     without appending (sec. 4.2), which the model records.  After the
 *     first such pop the decode's tokens are no longer the page's (the
 *     token lists here always append), so only counts up to it are compared.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "ctc_oracle.h"

#define NEG (-FLT_MAX)

/* ---------------------------------------------------------------------- */
/* Numerics.                                                                */
/* ---------------------------------------------------------------------- */

/* exp(x) for x in [-80, 0].  Cody & Waite (1980) argument reduction
 * x = n*ln2 + r with ln2 split into a 16-significant-bit high part and a
 * low part, then the degree-7 Taylor polynomial of e^r in Horner form with
 * fused multiply-adds, then the exact scaling by 2^n. */
float oracle_exp(float x)
{
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = 0x1.a01a02p-13f;          /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);    /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);     /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);     /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);     /* 1/3! */
    p = fmaf(p, r, 0x1.0p-1f);          /* 1/2! */
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* log(1 + x) for x in [0, 1]:  log1p(x) = 2 atanh(s), s = x / (2 + x), with
 * the odd series 2 (s + s^3/3 + ... + s^15/15) summed as s + s z q(z),
 * z = s^2, q in Horner form. */
float oracle_log1p(float x)
{
    float s = x / (2.0f + x);
    float z = s * s;
    float q = 0x1.111112p-4f;           /* 1/15 */
    q = fmaf(q, z, 0x1.3b13b2p-4f);     /* 1/13 */
    q = fmaf(q, z, 0x1.745d18p-4f);     /* 1/11 */
    q = fmaf(q, z, 0x1.c71c72p-4f);     /* 1/9  */
    q = fmaf(q, z, 0x1.24924ap-3f);     /* 1/7  */
    q = fmaf(q, z, 0x1.99999ap-3f);     /* 1/5  */
    q = fmaf(q, z, 0x1.555556p-2f);     /* 1/3  */
    float r = fmaf(s * z, q, s);
    return r + r;
}

/* The page's logsumexp (sec. 3): max(a,b) + log(1 + exp(-|a-b|)). */
float oracle_lse(float a, float b)
{
    float m = (a >= b) ? a : b;
    float lo = (a >= b) ? b : a;
    float d = lo - m;
    if (!(d >= -80.0f))
        return m;
    return m + oracle_log1p(oracle_exp(d));
}

/* The functions above over a range of inputs, for exhaustive comparisons:
 * element i uses the float whose bit pattern is first_bits + i (op 0 exp,
 * 1 log1p, 2 the IEEE quotient x / (2 + x) that log1p starts from), or the
 * pair (a[i], b[i]) (op 3 lse). */
void oracle_math_sweep(int op, uint32_t first_bits, int64_t n, const float *a, const float *b,
                       float *out)
{
    for (int64_t i = 0; i < n; i++) {
        float x;
        uint32_t u = first_bits + (uint32_t)i;
        memcpy(&x, &u, sizeof x);
        switch (op) {
        case 0: out[i] = oracle_exp(x); break;
        case 1: out[i] = oracle_log1p(x); break;
        case 2: out[i] = x / (2.0f + x); break;
        default: out[i] = oracle_lse(a[i], b[i]); break;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Frame selection (sec. 3.5).                                              */
/* ---------------------------------------------------------------------- */

float oracle_log_threshold(float threshold)
{
    /* computed once on the host, in double, rounded to float */
    return (float)log((double)threshold);
}

int oracle_select_frames(const float *lp_row, int64_t stride_t, int len, int blank,
                         float threshold, int *sel)
{
    int n = 0;
    if (threshold <= 0.0f)
        return 0; /* log(0) = -inf: no frame passes (sec. 13) */
    if (threshold >= 1.0f) {
        for (int t = 0; t < len; t++)
            sel[n++] = t; /* no skipping (sec. 13) */
        return n;
    }
    float log_thr = oracle_log_threshold(threshold);
    for (int t = 0; t < len; t++)
        if (lp_row[(int64_t)t * stride_t + blank] < log_thr)
            sel[n++] = t;
    return n;
}

/* ---------------------------------------------------------------------- */
/* Beam state (sec. 3.1).                                                   */
/* ---------------------------------------------------------------------- */

typedef struct {
    int live;
    int len;
    int *tok; /* capacity cap */
    float pb, pnb, score;
} Slot;

struct OracleStream {
    int beam, vocab, blank, capacity;
    int space;   /* the space label, or -1 (no space slot) */
    int step;    /* number of frames decoded so far */
    int last_t;  /* frame index of the last decoded frame */
    int frames;  /* frames given so far, decoded or not: the next frame's index */
    Slot *cur, *nxt;
    float *ptable, *ptablen; /* [beam][vocab] */
    int64_t *order;          /* candidate ids for the sort */
    const float *sort_keys;  /* keys the comparator reads */
    struct PageModel *pages; /* optional page accounting (NULL: none) */
};

/* ---------------------------------------------------------------------- */
/* Page accounting of the paged variant (sec. 3.4.5 paged variant, 4.2).    */
/* ---------------------------------------------------------------------- */

typedef struct PageModel {
    int beam, ps, npages, max_lp;
    int *tab[2];  /* [beam][max_lp] page ids of the two table parities, -1 none */
    int *held[2]; /* [beam] pages a row holds: the leading entries of its row */
    int *ref;     /* [npages] rows referring to each page */
    int *stack;   /* [npages] freed pages, LIFO */
    int top, next_free;
    int high;        /* most pages in use at once (handed out, not freed) */
    int failed;      /* a pop found nothing */
    int failed_step; /* step of the first such pop, -1 */
} PageModel;

static void pm_reset(PageModel *m)
{
    for (int i = 0; i < 2 * m->beam * m->max_lp; i++) {
        m->tab[0][i] = -1;
    }
    for (int k = 0; k < m->beam; k++) m->held[0][k] = m->held[1][k] = 0;
    for (int i = 0; i < m->npages; i++) m->ref[i] = 0;
    m->top = m->next_free = m->high = m->failed = 0;
    m->failed_step = -1;
}

static PageModel *pm_new(int beam, int ps, int npages, int cap)
{
    PageModel *m = (PageModel *)calloc(1, sizeof(PageModel));
    m->beam = beam;
    m->ps = ps;
    m->max_lp = (cap + ps - 1) / ps + 1;
    /* sec. 4.2: the default pool is beam * (max_logical_pages + 1) per row */
    m->npages = npages > 0 ? npages : beam * ((cap + ps - 1) / ps + 1);
    m->tab[0] = (int *)malloc(sizeof(int) * (size_t)(2 * beam * m->max_lp));
    m->tab[1] = m->tab[0] + beam * m->max_lp;
    m->held[0] = (int *)malloc(sizeof(int) * (size_t)(2 * beam));
    m->held[1] = m->held[0] + beam;
    m->ref = (int *)malloc(sizeof(int) * (size_t)(m->npages > 0 ? m->npages : 1));
    m->stack = (int *)malloc(sizeof(int) * (size_t)(m->npages > 0 ? m->npages : 1));
    pm_reset(m);
    return m;
}

static void pm_free(PageModel *m)
{
    if (!m) return;
    free(m->tab[0]);
    free(m->held[0]);
    free(m->ref);
    free(m->stack);
    free(m);
}

/* alloc_page: the stack of freed pages first (LIFO), then the bump pointer;
 * -1 past the row's pool */
static int pm_pop(PageModel *m)
{
    if (m->top > 0) return m->stack[--m->top];
    if (m->next_free < m->npages) return m->next_free++;
    return -1;
}

static void pm_fail(PageModel *m, int step)
{
    if (!m->failed) m->failed_step = step;
    m->failed = 1;
}

static void pm_note_use(PageModel *m)
{
    int used = m->next_free - m->top;
    if (used > m->high) m->high = used;
}

/* Step 0 (sec. 3.3): each of the first nseed slots holds one label, on a page
 * of its own, taken in slot order; the table of parity 0 is written. */
static void pm_seed(PageModel *m, int nseed)
{
    for (int r = 0; r < nseed && r < m->beam; r++) {
        int pg = pm_pop(m);
        if (pg < 0) {
            pm_fail(m, 0);
            continue;
        }
        m->ref[pg] = 1;
        m->tab[0][r * m->max_lp] = pg;
        m->held[0][r] = 1;
    }
    pm_note_use(m);
}

/* Step s >= 1: new row r (table parity s & 1) continues row src[r] of the
 * other parity (-1: a dead slot) whose hypothesis had srclen[r] labels, and
 * appends lab[r] unless it is the blank. */
static void pm_step(PageModel *m, int step, const int *src, const int *lab, const int *srclen,
                    int blank)
{
    const int W = m->beam, L = m->max_lp, p = step & 1, q = p ^ 1;
    int *newtab = (int *)malloc(sizeof(int) * (size_t)(W * L));
    int *newheld = (int *)malloc(sizeof(int) * (size_t)W);
    /* pass 1, fork: the new rows refer to their sources' pages ... */
    for (int r = 0; r < W; r++) {
        int k = src[r];
        newheld[r] = k >= 0 ? m->held[q][k] : 0;
        for (int j = 0; j < newheld[r]; j++) {
            newtab[r * L + j] = m->tab[q][k * L + j];
            m->ref[newtab[r * L + j]]++;
        }
    }
    /* ... and the pages the replaced rows held are released; one that no row
     * refers to any more goes on the stack */
    for (int r = 0; r < W; r++) {
        for (int j = 0; j < m->held[p][r]; j++) {
            int e = m->tab[p][r * L + j];
            if (--m->ref[e] == 0) m->stack[m->top++] = e;
        }
        for (int j = 0; j < L; j++) m->tab[p][r * L + j] = j < newheld[r] ? newtab[r * L + j] : -1;
        m->held[p][r] = newheld[r];
    }
    /* pass 2, append / copy-on-write, in ascending slot order */
    for (int r = 0; r < W; r++) {
        if (src[r] < 0 || lab[r] == blank) continue;
        int len = srclen[r], pi = len / m->ps, off = len % m->ps;
        int *row = m->tab[p] + r * L;
        if (off == 0) {
            /* the label starts a page */
            if (m->held[p][r] != pi) {
                pm_fail(m, step); /* a row already short of pages */
                continue;
            }
            int pg = pm_pop(m);
            if (pg < 0) {
                pm_fail(m, step);
                continue;
            }
            m->ref[pg] = 1;
            row[pi] = pg;
            m->held[p][r] = pi + 1;
        } else {
            if (m->held[p][r] != pi + 1) {
                pm_fail(m, step);
                continue;
            }
            int shared = row[pi];
            if (m->ref[shared] > 1) {
                /* shared with another row: copy it to a page of its own */
                int pg = pm_pop(m);
                if (pg < 0) {
                    pm_fail(m, step);
                    continue;
                }
                m->ref[pg] = 1;
                m->ref[shared]--; /* > 1 before: it never reaches 0 here */
                row[pi] = pg;
            }
            /* otherwise the row holds the page alone and writes in place */
        }
    }
    pm_note_use(m);
    free(newtab);
    free(newheld);
}

static int slot_clast(const Slot *s, int blank)
{
    return s->len > 0 ? s->tok[s->len - 1] : blank;
}

/* comparator context of qsort: per thread, so that independent decodes may run
 * on threads of one process (each decode itself is single-threaded) */
static _Thread_local const float *g_rank_lp;

static int cmp_vocab_rank(const void *a, const void *b)
{
    int ca = *(const int *)a, cb = *(const int *)b;
    float la = g_rank_lp[ca], lb = g_rank_lp[cb];
    if (la > lb) return -1;
    if (la < lb) return 1;
    return (ca < cb) ? -1 : (ca > cb);
}

static _Thread_local const float *g_keys;

static int cmp_candidates(const void *a, const void *b)
{
    int64_t ia = *(const int64_t *)a, ib = *(const int64_t *)b;
    float ka = g_keys[ia], kb = g_keys[ib];
    if (ka > kb) return -1;
    if (ka < kb) return 1;
    return (ia < ib) ? -1 : (ia > ib);
}

static void reset_empty(OracleStream *st)
{
    /* sec. 13: a row that never runs step 0 holds the empty hypothesis in
     * slot 0 at score 0 and dead slots elsewhere. */
    for (int k = 0; k < st->beam; k++) {
        Slot *s = &st->cur[k];
        s->live = (k == 0);
        s->len = 0;
        s->pb = (k == 0) ? 0.0f : NEG;
        s->pnb = NEG;
        s->score = (k == 0) ? 0.0f : NEG;
    }
    st->step = 0;
    st->last_t = -1;
    st->frames = 0;
    if (st->pages) pm_reset(st->pages);
}

OracleStream *oracle_stream_new_sp(int beam, int vocab, int blank, int capacity, int space)
{
    if (beam < 1 || vocab < 2 || blank < 0 || blank >= vocab || capacity < 0 || space >= vocab)
        return NULL;
    OracleStream *st = (OracleStream *)calloc(1, sizeof(OracleStream));
    /* sec. 3.4.2: the space slot exists for space_id >= 0 other than the blank */
    st->space = (space >= 0 && space != blank) ? space : -1;
    st->beam = beam;
    st->vocab = vocab;
    st->blank = blank;
    st->capacity = capacity;
    st->cur = (Slot *)calloc((size_t)beam, sizeof(Slot));
    st->nxt = (Slot *)calloc((size_t)beam, sizeof(Slot));
    for (int k = 0; k < beam; k++) {
        st->cur[k].tok = (int *)malloc(sizeof(int) * (size_t)(capacity + 1));
        st->nxt[k].tok = (int *)malloc(sizeof(int) * (size_t)(capacity + 1));
    }
    st->ptable = (float *)malloc(sizeof(float) * (size_t)beam * (size_t)vocab);
    st->ptablen = (float *)malloc(sizeof(float) * (size_t)beam * (size_t)vocab);
    st->order = (int64_t *)malloc(sizeof(int64_t) * (size_t)beam * (size_t)vocab);
    reset_empty(st);
    return st;
}

OracleStream *oracle_stream_new(int beam, int vocab, int blank, int capacity)
{
    return oracle_stream_new_sp(beam, vocab, blank, capacity, -1);
}

OracleStream *oracle_stream_new_paged(int beam, int vocab, int blank, int capacity, int space,
                                      int page_size, int num_pages)
{
    if (page_size < 1 || num_pages < 0) return NULL;
    OracleStream *st = oracle_stream_new_sp(beam, vocab, blank, capacity, space);
    if (st) st->pages = pm_new(beam, page_size, num_pages, capacity);
    return st;
}

void oracle_stream_pages(const OracleStream *st, int *out)
{
    const PageModel *m = st->pages;
    out[0] = m ? m->high : 0;
    out[1] = m ? m->failed : 0;
    out[2] = m ? m->failed_step : -1;
}

void oracle_stream_free(OracleStream *st)
{
    if (!st) return;
    for (int k = 0; k < st->beam; k++) {
        free(st->cur[k].tok);
        free(st->nxt[k].tok);
    }
    free(st->cur);
    free(st->nxt);
    free(st->ptable);
    free(st->ptablen);
    free(st->order);
    pm_free(st->pages);
    free(st);
}

void oracle_stream_reset(OracleStream *st) { reset_empty(st); }

int oracle_stream_step_count(const OracleStream *st) { return st->step; }

/* Step 0 (sec. 3.3): seed the beams from the first decoded frame. */
static void first_step(OracleStream *st, const float *lp, int t)
{
    const int W = st->beam, V = st->vocab, blank = st->blank;
    int need_add_blank = (t > 0);
    int nb = (W > 1) ? W - 1 : W;

    int *chars = (int *)malloc(sizeof(int) * (size_t)V);
    int nc = 0;
    for (int c = 0; c < V; c++)
        if (c != blank)
            chars[nc++] = c;
    g_rank_lp = lp;
    qsort(chars, (size_t)nc, sizeof(int), cmp_vocab_rank);

    for (int k = 0; k < W; k++) {
        Slot *s = &st->cur[k];
        s->live = 0;
        s->len = 0;
        s->pb = s->pnb = s->score = NEG;
    }
    int m = nb < nc ? nb : nc;
    for (int k = 0; k < m; k++) {
        Slot *s = &st->cur[k];
        float key = lp[chars[k]];
        s->live = 1;
        s->len = 1;
        s->tok[0] = chars[k];
        if (need_add_blank) {
            s->pb = key;
            s->pnb = NEG;
        } else {
            s->pb = NEG;
            s->pnb = key;
        }
        s->score = key;
    }
    if (W > 1) {
        Slot *s = &st->cur[W - 1];
        s->live = 1;
        s->len = 0;
        s->pb = lp[blank];
        s->pnb = NEG;
        s->score = lp[blank];
    }
    if (st->pages) pm_seed(st->pages, m);
    free(chars);
}

/* One step s >= 1 (sec. 3.4.1 - 3.4.5) on the frame row lp. */
static void next_step(OracleStream *st, const float *lp, int need_add_blank)
{
    const int W = st->beam, V = st->vocab, blank = st->blank, space = st->space;
    float *pt = st->ptable, *ptn = st->ptablen;

    /* sec. 3.4.1 / 3.4.2: extension tables.  Dead beams get NEG everywhere. */
    for (int k = 0; k < W; k++) {
        const Slot *s = &st->cur[k];
        float *rowb = pt + (size_t)k * V, *rown = ptn + (size_t)k * V;
        if (!s->live) {
            for (int c = 0; c < V; c++)
                rowb[c] = rown[c] = NEG;
            continue;
        }
        float prev_b, prev_nb;
        if (need_add_blank) { /* collapsed-blank correction (sec. 3.4) */
            prev_b = oracle_lse(s->pb, s->pnb);
            prev_nb = NEG;
        } else {
            prev_b = s->pb;
            prev_nb = s->pnb;
        }
        int last = slot_clast(s, blank);
        /* The non-blank "stay" below reaches the blank slot only from the
         * loop's c == last case.  The loop skips the space label (sec.
         * 3.4.1), so a beam ending in the space label has no stay term: NEG
         * (the page leaves whatever the slot held; this is the reading
         * taken). */
        rown[blank] = NEG;
        for (int c = 0; c < V; c++) {
            if (c == blank)
                continue;
            if (c == space) {
                /* sec. 3.4.2 space slot: a new label from either part, also
                 * after a beam that already ends in the space label */
                rown[c] = lp[c] + oracle_lse(prev_b, prev_nb);
                rowb[c] = NEG;
                continue;
            }
            if (c == last) {
                rown[c] = lp[c] + prev_b;        /* same label: blank path only */
                rown[blank] = lp[c] + prev_nb;   /* "stay" folds into the blank slot */
            } else {
                rown[c] = lp[c] + oracle_lse(prev_b, prev_nb);
            }
            rowb[c] = NEG;
        }
        rowb[blank] = lp[blank] + oracle_lse(prev_b, prev_nb);
        if (need_add_blank || last == blank)
            rown[blank] = NEG;
    }

    /* sec. 3.4.3: prefix merge.  i = the shorter beam (source), j = the longer. */
    for (int i = 0; i < W; i++) {
        const Slot *si = &st->cur[i];
        if (!si->live) continue;
        for (int j = 0; j < W; j++) {
            const Slot *sj = &st->cur[j];
            if (j == i || !sj->live) continue;
            if (sj->len - 1 != si->len) continue;
            if (memcmp(sj->tok, si->tok, sizeof(int) * (size_t)si->len) != 0) continue;
            size_t src = (size_t)i * V + (size_t)slot_clast(sj, blank);
            size_t dst = (size_t)j * V + (size_t)blank;
            pt[dst] = oracle_lse(pt[dst], pt[src]);
            ptn[dst] = oracle_lse(ptn[dst], ptn[src]);
            pt[src] = NEG;
            ptn[src] = NEG;
        }
    }

    /* sec. 3.4.4: key = logsumexp(ptable, ptablen); keep keys above NEG;
     * order (key desc, flat id asc). */
    const int64_t total = (int64_t)W * V;
    float *keys = (float *)malloc(sizeof(float) * (size_t)total);
    int64_t n = 0;
    for (int64_t id = 0; id < total; id++) {
        keys[id] = oracle_lse(pt[id], ptn[id]);
        if (keys[id] > NEG)
            st->order[n++] = id;
    }
    g_keys = keys;
    qsort(st->order, (size_t)n, sizeof(int64_t), cmp_candidates);

    /* sec. 3.4.5: state update from the snapshot of the source beams. */
    int nw = (n < W) ? (int)n : W;
    int *psrc = NULL, *plab = NULL, *plen = NULL;   /* the page model's view */
    if (st->pages) {
        psrc = (int *)malloc(sizeof(int) * (size_t)(3 * W));
        plab = psrc + W;
        plen = plab + W;
    }
    for (int r = 0; r < W; r++) {
        Slot *d = &st->nxt[r];
        if (psrc) {
            psrc[r] = -1;
            plab[r] = blank;
            plen[r] = 0;
        }
        if (r >= nw) {
            d->live = 0;
            d->len = 0;
            d->pb = d->pnb = d->score = NEG;
            continue;
        }
        int64_t id = st->order[r];
        int k = (int)(id / V), c = (int)(id % V);
        const Slot *s = &st->cur[k];
        if (psrc) {
            psrc[r] = k;
            plab[r] = c;
            plen[r] = s->len;
        }
        d->live = 1;
        memcpy(d->tok, s->tok, sizeof(int) * (size_t)s->len);
        d->len = s->len;
        if (c != blank)
            d->tok[d->len++] = c;
        d->score = keys[id];
        if (need_add_blank) {
            d->pb = keys[id];
            d->pnb = NEG;
        } else {
            d->pb = pt[id];
            d->pnb = ptn[id];
        }
    }
    free(keys);
    if (psrc) {
        pm_step(st->pages, st->step, psrc, plab, plen, blank);
        free(psrc);
    }
    Slot *tmp = st->cur;
    st->cur = st->nxt;
    st->nxt = tmp;
}

/* Decode one selected frame t (row lp) as the stream's next step. */
static void decode_frame(OracleStream *st, const float *lp, int t)
{
    if (st->step == 0)
        first_step(st, lp, t);
    else
        next_step(st, lp, t > st->last_t + 1);
    st->last_t = t;
    st->step++;
}

int oracle_stream_feed_ex(OracleStream *st, const float *frames, int64_t stride_t, int n_frames,
                          const unsigned char *is_speech, int start_frame)
{
    /* Streaming (sec. 8): chunk frame f is frame number start + f of the
     * stream, start being the caller's start_frame (sec. 9
     * ctc_beam_search_chunk) or, when that is negative, the count of frames
     * given so far.  It is decoded unless is_speech marks it 0 (the page's
     * is_speech_mask, sec. 12: a skipped frame bypasses the decoder) or the
     * stream has reached its capacity (sec. 13).  A frame decoded after
     * skipped ones takes the gap rule through its frame index. */
    if (start_frame >= 0)
        st->frames = start_frame;
    for (int f = 0; f < n_frames; f++) {
        if (is_speech && !is_speech[f])
            continue;
        if (st->step >= st->capacity)
            break;
        decode_frame(st, frames + (int64_t)f * stride_t, st->frames + f);
    }
    st->frames += n_frames;
    return st->step;
}

int oracle_stream_feed(OracleStream *st, const float *frames, int64_t stride_t, int n_frames)
{
    return oracle_stream_feed_ex(st, frames, stride_t, n_frames, NULL, -1);
}

int oracle_stream_frame_count(const OracleStream *st) { return st->frames; }

static int cmp_slots_score(const void *a, const void *b, const Slot *slots)
{
    int ia = *(const int *)a, ib = *(const int *)b;
    float sa = slots[ia].score, sb = slots[ib].score;
    if (sa > sb) return -1;
    if (sa < sb) return 1;
    return (ia < ib) ? -1 : (ia > ib);
}

void oracle_stream_read(const OracleStream *st, int nbest, int max_out_len,
                        int *out_tokens, int *out_lengths, float *out_scores)
{
    /* live slots in (score desc, slot asc) order, then the dead ones */
    int W = st->beam;
    int *idx = (int *)malloc(sizeof(int) * (size_t)W);
    int nl = 0;
    for (int k = 0; k < W; k++)
        if (st->cur[k].live)
            idx[nl++] = k;
    /* insertion sort: W is small and this keeps the order rule explicit */
    for (int a = 1; a < nl; a++) {
        int v = idx[a], b = a - 1;
        while (b >= 0 && cmp_slots_score(&idx[b], &v, st->cur) > 0) {
            idx[b + 1] = idx[b];
            b--;
        }
        idx[b + 1] = v;
    }
    for (int r = 0; r < nbest; r++) {
        int *ot = out_tokens + (size_t)r * max_out_len;
        for (int p = 0; p < max_out_len; p++)
            ot[p] = -1;
        if (r >= nl) {
            out_lengths[r] = 0;
            out_scores[r] = NEG;
            continue;
        }
        const Slot *s = &st->cur[idx[r]];
        out_lengths[r] = s->len;
        out_scores[r] = s->score;
        int n = s->len < max_out_len ? s->len : max_out_len;
        for (int p = 0; p < n; p++)
            ot[p] = s->tok[p];
    }
    free(idx);
}

/* Offline decode of a batch (sec. 3.7): select frames, decode every selected
 * frame in order, report the N best per row. */
int oracle_decode_sp(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                     int max_T, const int *seq_lengths, int beam, int nbest, int vocab,
                     int blank, float threshold, int max_out_len, int *out_tokens,
                     int *out_lengths, float *out_scores, int space)
{
    if (beam < 1 || nbest < 1 || nbest > beam || vocab < 2 || blank < 0 || blank >= vocab ||
        max_out_len < 0 || batch < 0 || max_T < 0 || space >= vocab)
        return 1;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(max_T > 0 ? max_T : 1));
    for (int b = 0; b < batch; b++) {
        int len = seq_lengths[b];
        if (len < 0) len = 0;
        if (len > max_T) len = max_T;
        const float *row = log_prob + (int64_t)b * stride_b;
        int n = oracle_select_frames(row, stride_t, len, blank, threshold, sel);
        OracleStream *st = oracle_stream_new_sp(beam, vocab, blank, len, space);
        for (int s = 0; s < n; s++)
            decode_frame(st, row + (int64_t)sel[s] * stride_t, sel[s]);
        oracle_stream_read(st, nbest, max_out_len,
                           out_tokens + (size_t)b * nbest * max_out_len,
                           out_lengths + (size_t)b * nbest, out_scores + (size_t)b * nbest);
        oracle_stream_free(st);
    }
    free(sel);
    return 0;
}

/* Page accounting along offline decodes (sec. 3.4.5 paged variant, 4.2):
 * per row out[3b] the most pages in use at once, out[3b+1] 1 if a pop found
 * nothing, out[3b+2] the step of the first such pop (-1).  The pool is
 * num_pages, or beam * (ceil(max_T / page_size) + 1) for 0. */
int oracle_decode_pages(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                        int max_T, const int *seq_lengths, int beam, int vocab, int blank,
                        float threshold, int space, int page_size, int num_pages, int *out)
{
    if (beam < 1 || vocab < 2 || blank < 0 || blank >= vocab || batch < 0 || max_T < 0 ||
        space >= vocab || page_size < 1 || num_pages < 0)
        return 1;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(max_T > 0 ? max_T : 1));
    const int pool = num_pages > 0 ? num_pages : beam * ((max_T + page_size - 1) / page_size + 1);
    for (int b = 0; b < batch; b++) {
        int len = seq_lengths[b];
        if (len < 0) len = 0;
        if (len > max_T) len = max_T;
        const float *row = log_prob + (int64_t)b * stride_b;
        int n = oracle_select_frames(row, stride_t, len, blank, threshold, sel);
        OracleStream *st =
            oracle_stream_new_paged(beam, vocab, blank, max_T, space, page_size, pool);
        for (int s = 0; s < n; s++)
            decode_frame(st, row + (int64_t)sel[s] * stride_t, sel[s]);
        oracle_stream_pages(st, out + 3 * b);
        oracle_stream_free(st);
    }
    free(sel);
    return 0;
}

/* The page model alone, on given winners (hand-worked cases): nseed seeded
 * slots at step 0, then for steps 1..nsteps the source slot (-1 dead) and the
 * label of every slot, src/lab[(s - 1) * beam + r].  Writes the pages in use
 * after every step to used[0..nsteps] and the summary to out[3] as above. */
int oracle_page_model_run(int beam, int page_size, int num_pages, int cap, int blank, int nseed,
                          int nsteps, const int *src, const int *lab, int *used, int *out)
{
    if (beam < 1 || page_size < 1 || num_pages < 0 || cap < 1 || nsteps < 0) return 1;
    PageModel *m = pm_new(beam, page_size, num_pages, cap);
    int *len = (int *)calloc((size_t)beam, sizeof(int));
    int *nlen = (int *)calloc((size_t)beam, sizeof(int));
    int *srclen = (int *)calloc((size_t)beam, sizeof(int));
    for (int r = 0; r < nseed && r < beam; r++) len[r] = 1;
    pm_seed(m, nseed);
    used[0] = m->next_free - m->top;
    for (int s = 1; s <= nsteps; s++) {
        const int *sr = src + (size_t)(s - 1) * beam, *lb = lab + (size_t)(s - 1) * beam;
        for (int r = 0; r < beam; r++) {
            srclen[r] = sr[r] >= 0 ? len[sr[r]] : 0;
            nlen[r] = sr[r] >= 0 ? srclen[r] + (lb[r] != blank) : 0;
        }
        pm_step(m, s, sr, lb, srclen, blank);
        memcpy(len, nlen, sizeof(int) * (size_t)beam);
        used[s] = m->next_free - m->top;
    }
    out[0] = m->high;
    out[1] = m->failed;
    out[2] = m->failed_step;
    free(len);
    free(nlen);
    free(srclen);
    pm_free(m);
    return 0;
}

int oracle_decode(const float *log_prob, int64_t stride_b, int64_t stride_t, int batch,
                  int max_T, const int *seq_lengths, int beam, int nbest, int vocab,
                  int blank, float threshold, int max_out_len, int *out_tokens,
                  int *out_lengths, float *out_scores)
{
    return oracle_decode_sp(log_prob, stride_b, stride_t, batch, max_T, seq_lengths, beam, nbest,
                            vocab, blank, threshold, max_out_len, out_tokens, out_lengths,
                            out_scores, -1);
}
