/*
 * All-core CPU baseline: the data-parallel method run on host threads.
 *
 * NOT THE ORACLE, and test/benchmark infrastructure only: the benchmark's
 * CPU-baseline leg times it, and the test suite checks it bit-exact against
 * the sequential oracles (csv_oracle.c, lex_oracle.c). It shares no code,
 * header or table with the GPU path.
 *
 * CSV: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw Data",
 * Sec. 3, with one host thread per contiguous slice in place of a GPU thread
 * per chunk:
 *   1. every thread runs the DFA over its slice from every state at once (the
 *      multi-DFA of Fig. 2), giving the slice's state-transition vector;
 *   2. one thread composes the vectors in slice order: the state at each
 *      slice's start;
 *   3. every thread runs its slice again from that state (the tagging step)
 *      and lists its terminators (position and record bit) in its own array,
 *      counting its fields, records, column carry and first INVALID byte;
 *   4. one thread turns the counts into each slice's field index, record index,
 *      column and field start at its first byte (exclusive prefixes, the
 *      offsets of Fig. 4), and resolves the fields-per-record range as the passage "Inferring or validating number of columns"
 *      ("Inferring or validating number of columns") describes: a slice counts
 *      the field delimiters before its first record delimiter (relative: the
 *      record began in an earlier slice) and the fewest and most fields of the
 *      records after it; the carried column turns the relative count absolute;
 *   5. every thread writes its fields from its list at its field index.
 * Steps 3-5 give each field the record, column, offset and length the
 * sequential loop gives it, started from the slice's carried values.
 *
 * Lexer: "Lexing on the GPU: the scan is the easy part", section "A lexer is a
 * prefix scan": the restart lexer's only state across a slice boundary is its
 * DFA state (and the start of the token in progress, a carried position), so
 * the same steps apply with the lexer DFA's state-transition vector; step 3
 * lists where tokens end and their kinds.
 *
 * Step 1 steps only the distinct states still live: runs that reach the same
 * state stay together from then on, so start states whose runs have met share
 * one run (checked every 64 bytes; the CSV DFA keeps two runs, inside and
 * outside quotes; a lexer's runs usually meet within a token).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { TAG_VALUE = 0, TAG_FIELD = 1, TAG_RECORD = 2, TAG_INVALID = 3 };
enum { MAX_STATES = 1024, MAX_THREADS = 256, MERGE_BLOCK = 64 };

/* ------------------------------------------------------------ distinct runs */

/* Merges the runs run[0..*live) that hold equal states (each keeps the first
 * slot that holds its state) and remaps slot_of[0..Q) accordingly. seen[] is
 * all UINT32_MAX on entry and on return. */
static void merge_runs(uint32_t* run, uint32_t* live, uint32_t* slot_of, uint32_t Q, uint32_t* seen, uint32_t* remap)
{
    uint32_t dup = 0;
    for (uint32_t j = 0; j < *live; ++j) {
        if (seen[run[j]] != UINT32_MAX) dup = 1;
        else seen[run[j]] = j;
    }
    if (dup) {
        uint32_t k = 0;
        for (uint32_t j = 0; j < *live; ++j) {
            const uint32_t first = seen[run[j]];
            if (first == j) {
                remap[j] = k;
                run[k++] = run[j];
            } else {
                remap[j] = remap[first];
            }
        }
        for (uint32_t s = 0; s < Q; ++s) slot_of[s] = remap[slot_of[s]];
        *live = k;
    }
    for (uint32_t j = 0; j < *live; ++j) seen[run[j]] = UINT32_MAX;
}

/* The state-transition vector of bytes [a, b): vec[s] = the state reached from
 * s, for every s < Q. STEP(q, byte) is the next state. */
#define SLICE_VECTOR(NAME, CTX_T, STEP)                                                                            \
    static void NAME(const CTX_T* d, const uint8_t* bytes, uint64_t a, uint64_t b, uint32_t Q, uint32_t* vec)      \
    {                                                                                                              \
        uint32_t run[MAX_STATES], slot_of[MAX_STATES], seen[MAX_STATES], remap[MAX_STATES];                       \
        uint32_t live = Q;                                                                                         \
        for (uint32_t s = 0; s < Q; ++s) {                                                                         \
            run[s] = s;                                                                                            \
            slot_of[s] = s;                                                                                        \
            seen[s] = UINT32_MAX;                                                                                  \
        }                                                                                                          \
        uint64_t i = a;                                                                                            \
        while (i < b) {                                                                                            \
            const uint64_t e = live > 1 && b - i > MERGE_BLOCK ? i + MERGE_BLOCK : b;                             \
            for (uint32_t j = 0; j < live; ++j) {                                                                  \
                uint32_t q = run[j];                                                                               \
                for (uint64_t k = i; k < e; ++k) q = STEP(d, q, bytes[k]);                                         \
                run[j] = q;                                                                                        \
            }                                                                                                      \
            i = e;                                                                                                 \
            if (live > 1) merge_runs(run, &live, slot_of, Q, seen, remap);                                         \
        }                                                                                                          \
        for (uint32_t s = 0; s < Q; ++s) vec[s] = run[slot_of[s]];                                                 \
    }

/* Runs body(t) for t in [0, T) on T threads (thread 0: the caller). */
typedef struct {
    void (*body)(void* ctx, uint32_t t);
    void* ctx;
    uint32_t t;
} task_t;

static void* task_main(void* p)
{
    task_t* k = (task_t*)p;
    k->body(k->ctx, k->t);
    return NULL;
}

static int run_threads(uint32_t T, void (*body)(void*, uint32_t), void* ctx)
{
    pthread_t th[MAX_THREADS];
    task_t tk[MAX_THREADS];
    uint32_t started = 0;
    int rc = 0;
    for (uint32_t t = 1; t < T; ++t) {
        tk[t] = (task_t){body, ctx, t};
        if (pthread_create(&th[t], NULL, task_main, &tk[t]) != 0) {
            rc = -1;
            break;
        }
        started = t;
    }
    if (rc == 0) body(ctx, 0);
    for (uint32_t t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    return rc;
}

static uint64_t slice_lo(uint64_t n, uint32_t T, uint32_t t) { return n * t / T; }

/* a growable per-thread list of 64-bit entries */
typedef struct {
    uint64_t* v;
    uint64_t size, cap;
    int failed;
} list_t;

static void list_push(list_t* l, uint64_t x)
{
    if (l->size == l->cap) {
        const uint64_t cap = l->cap ? 2 * l->cap : 1024;
        uint64_t* v = (uint64_t*)realloc(l->v, cap * sizeof(uint64_t));
        if (!v) {
            l->failed = 1;
            return;
        }
        l->v = v;
        l->cap = cap;
    }
    if (!l->failed) l->v[l->size++] = x;
}

/* -------------------------------------------------------------------- CSV */

typedef struct {
    const uint8_t *next, *tag, *class_map;
    uint32_t n_classes;
} csv_dfa_t;

#define CSV_STEP(d, q, byte) ((uint32_t)(d)->next[(q) * (d)->n_classes + (d)->class_map[(byte)]])
SLICE_VECTOR(csv_slice_vector, csv_dfa_t, CSV_STEP)

typedef struct {
    uint32_t s_in, s_out, last_tag;
    list_t terms;       /* per terminator: position << 1 | record bit, in order */
    uint64_t nr;        /* record delimiters */
    uint64_t col_tail;  /* field delimiters after the slice's last record delimiter (all of them if none) */
    int has_rec;
    uint64_t col_head;  /* field delimiters before the slice's first record delimiter */
    uint64_t cmin, cmax;  /* fewest / most fields of the records after the first record delimiter */
    int64_t err;        /* first INVALID byte (-1: none) */
    uint64_t f_in, r_in, c_in, start_in;  /* field index, record, column, field start at the first byte */
} csv_slice_t;

typedef struct {
    const uint8_t* bytes;
    uint64_t n;
    uint32_t T, Q;
    csv_dfa_t d;
    uint32_t* vec; /* [T][Q] */
    csv_slice_t* sl;
    uint32_t *rec_out, *col_out, *off_out, *len_out;
    uint64_t cap;
} csv_job_t;

static void csv_vectors(void* p, uint32_t t)
{
    csv_job_t* j = (csv_job_t*)p;
    csv_slice_vector(&j->d, j->bytes, slice_lo(j->n, j->T, t), slice_lo(j->n, j->T, t + 1), j->Q,
                     j->vec + (size_t)t * j->Q);
}

static void csv_tags(void* p, uint32_t t)
{
    csv_job_t* j = (csv_job_t*)p;
    csv_slice_t* c = &j->sl[t];
    const uint64_t a = slice_lo(j->n, j->T, t), b = slice_lo(j->n, j->T, t + 1);
    const uint32_t C = j->d.n_classes;
    uint32_t s = c->s_in, last_tag = TAG_VALUE;
    uint64_t nr = 0, col = 0, col_head = 0, cmin = UINT64_MAX, cmax = 0;
    int64_t err = -1;
    int has_rec = 0;
    for (uint64_t i = a; i < b; ++i) {
        const uint32_t cl = j->d.class_map[j->bytes[i]];
        const uint32_t tg = j->d.tag[s * C + cl];
        s = j->d.next[s * C + cl];
        if (tg == TAG_FIELD) {
            list_push(&c->terms, i << 1);
            col++;
        } else if (tg == TAG_RECORD) {
            list_push(&c->terms, (i << 1) | 1u);
            nr++;
            if (has_rec) {
                if (col + 1 < cmin) cmin = col + 1;
                if (col + 1 > cmax) cmax = col + 1;
            } else {
                col_head = col;
            }
            col = 0;
            has_rec = 1;
        } else if (tg == TAG_INVALID && err < 0) {
            err = (int64_t)i;
        }
        last_tag = tg;
    }
    c->nr = nr;
    c->col_tail = col;
    c->col_head = col_head;
    c->cmin = cmin;
    c->cmax = cmax;
    c->has_rec = has_rec;
    c->err = err;
    c->last_tag = last_tag;
    c->s_out = s;
}

static void csv_write(void* p, uint32_t t)
{
    csv_job_t* j = (csv_job_t*)p;
    const csv_slice_t* c = &j->sl[t];
    uint64_t f = c->f_in, rec = c->r_in, col = c->c_in, field_start = c->start_in;
    for (uint64_t k = 0; k < c->terms.size; ++k, ++f) {
        const uint64_t x = c->terms.v[k], i = x >> 1;
        if (f < j->cap) {
            j->rec_out[f] = (uint32_t)rec;
            j->col_out[f] = (uint32_t)col;
            j->off_out[f] = (uint32_t)field_start;
            j->len_out[f] = (uint32_t)(i - field_start);
        }
        field_start = i + 1;
        if (x & 1u) {
            rec++;
            col = 0;
        } else {
            col++;
        }
    }
}

/* Same arguments and results as oracle_csv_parse, plus the thread count;
 * -1 on an invalid table or thread count, or when memory runs out. */
int cpu_parallel_csv_parse(const uint8_t* bytes, uint64_t n, uint32_t n_states, uint32_t n_classes,
                           uint32_t start_state, uint32_t accept_mask, const uint8_t* next, const uint8_t* tag,
                           const uint8_t* class_map, uint32_t* rec_out, uint32_t* col_out, uint32_t* off_out,
                           uint32_t* len_out, uint64_t cap, uint32_t n_threads, uint64_t* n_fields,
                           uint64_t* n_records, int64_t* error_pos, uint32_t* end_state, uint32_t* min_columns,
                           uint32_t* max_columns)
{
    if (n_states == 0 || n_states > MAX_STATES || n_classes == 0 || start_state >= n_states || n_threads == 0)
        return -1;
    for (uint32_t x = 0; x < n_states * n_classes; ++x)
        if (next[x] >= n_states) return -1;
    for (uint32_t x = 0; x < 256; ++x)
        if (class_map[x] >= n_classes) return -1;
    uint32_t T = n_threads > MAX_THREADS ? MAX_THREADS : n_threads;
    if (n < T) T = n ? (uint32_t)n : 1u;
    csv_job_t j = {bytes, n, T, n_states, {next, tag, class_map, n_classes}, NULL, NULL,
                   rec_out, col_out, off_out, len_out, cap};
    j.vec = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)T * n_states);
    j.sl = (csv_slice_t*)calloc(T, sizeof(csv_slice_t));
    int rc = (j.vec && j.sl) ? 0 : -1;
    /* 1. vectors; 2. start states */
    if (rc == 0) rc = run_threads(T, csv_vectors, &j);
    if (rc == 0) {
        uint32_t s = start_state;
        for (uint32_t t = 0; t < T; ++t) {
            j.sl[t].s_in = s;
            s = j.vec[(size_t)t * n_states + s];
        }
        /* 3. tags */
        rc = run_threads(T, csv_tags, &j);
        for (uint32_t t = 0; t < T && rc == 0; ++t)
            if (j.sl[t].terms.failed) rc = -1;
    }
    if (rc == 0) {
        /* 4. prefixes */
        uint64_t f = 0, r = 0, c = 0, start = 0, cmin = UINT64_MAX, cmax = 0;
        for (uint32_t t = 0; t < T; ++t) {
            csv_slice_t* x = &j.sl[t];
            x->f_in = f;
            x->r_in = r;
            x->c_in = c;
            x->start_in = start;
            if (x->has_rec) {  /* the record its first record delimiter ends began at column c */
                const uint64_t head = c + x->col_head + 1;
                if (head < cmin) cmin = head;
                if (head > cmax) cmax = head;
                if (x->cmin < cmin) cmin = x->cmin;
                if (x->cmax > cmax) cmax = x->cmax;
            }
            f += x->terms.size;
            r += x->nr;
            c = x->has_rec ? x->col_tail : c + x->col_tail;
            if (x->terms.size) start = (x->terms.v[x->terms.size - 1] >> 1) + 1;
        }
        /* 5. fields */
        rc = run_threads(T, csv_write, &j);
        if (rc == 0) {
            const csv_slice_t* last = &j.sl[T - 1];
            const uint32_t s_end = last->s_out;
            int64_t err = -1;
            for (uint32_t t = 0; t < T && err < 0; ++t) err = j.sl[t].err;
            /* the unterminated final field, as the sequential loop ends */
            if (n > 0 && last->last_tag != TAG_RECORD) {
                if (f < cap) {
                    rec_out[f] = (uint32_t)r;
                    col_out[f] = (uint32_t)c;
                    off_out[f] = (uint32_t)start;
                    len_out[f] = (uint32_t)(n - start);
                }
                f++;
                r++;
                if (c + 1 < cmin) cmin = c + 1;
                if (c + 1 > cmax) cmax = c + 1;
            }
            if (err < 0 && !((accept_mask >> s_end) & 1u)) err = (int64_t)n;
            *min_columns = r ? (uint32_t)cmin : 0u;
            *max_columns = r ? (uint32_t)cmax : 0u;
            *n_fields = f;
            *n_records = r;
            *error_pos = err;
            *end_state = s_end;
            rc = f > cap ? -2 : 0;
        }
    }
    if (j.sl)
        for (uint32_t t = 0; t < T; ++t) free(j.sl[t].terms.v);
    free(j.vec);
    free(j.sl);
    return rc;
}

/* ------------------------------------------------------------------ lexer */

typedef struct {
    const int16_t* delta;
    uint32_t q0;
} lex_dfa_t;

/* one byte of the restart lexer: the DFA's move, or a restart from q0 */
static inline uint32_t lex_step(const lex_dfa_t* d, uint32_t q, uint32_t byte)
{
    const int32_t x = d->delta[(uint64_t)q * 256 + byte];
    return x >= 0 ? (uint32_t)x : (uint32_t)d->delta[(uint64_t)d->q0 * 256 + byte];
}
SLICE_VECTOR(lex_slice_vector, lex_dfa_t, lex_step)

typedef struct {
    uint32_t q_in, q_out;
    list_t ends;  /* per token ended in the slice: its end (the restart position) << 16 | its kind */
    uint64_t t_in, start_in;
} lex_slice_t;

typedef struct {
    const uint8_t* bytes;
    uint64_t n;
    uint32_t T, Q;
    lex_dfa_t d;
    const uint16_t* kind_of;
    uint32_t* vec;
    lex_slice_t* sl;
    uint32_t *kind, *start, *len;
    uint64_t cap;
} lex_job_t;

static void lex_vectors(void* p, uint32_t t)
{
    lex_job_t* j = (lex_job_t*)p;
    lex_slice_vector(&j->d, j->bytes, slice_lo(j->n, j->T, t), slice_lo(j->n, j->T, t + 1), j->Q,
                     j->vec + (size_t)t * j->Q);
}

static void lex_ends(void* p, uint32_t t)
{
    lex_job_t* j = (lex_job_t*)p;
    lex_slice_t* c = &j->sl[t];
    const uint64_t a = slice_lo(j->n, j->T, t), b = slice_lo(j->n, j->T, t + 1);
    uint32_t q = c->q_in;
    for (uint64_t i = a; i < b; ++i) {
        const uint32_t byte = j->bytes[i];
        const int32_t x = j->d.delta[(uint64_t)q * 256 + byte];
        if (x >= 0) {
            q = (uint32_t)x;
        } else {
            list_push(&c->ends, (i << 16) | j->kind_of[q]);
            q = (uint32_t)j->d.delta[(uint64_t)j->d.q0 * 256 + byte];
        }
    }
    c->q_out = q;
}

static void lex_write(void* p, uint32_t t)
{
    lex_job_t* j = (lex_job_t*)p;
    const lex_slice_t* c = &j->sl[t];
    uint64_t k = c->t_in, tok_start = c->start_in;
    for (uint64_t e = 0; e < c->ends.size; ++e, ++k) {
        const uint64_t x = c->ends.v[e], i = x >> 16;
        if (k < j->cap) {
            j->kind[k] = (uint32_t)(x & 0xffffu);
            j->start[k] = (uint32_t)tok_start;
            j->len[k] = (uint32_t)(i - tok_start);
        }
        tok_start = i;
    }
}

/* Same arguments and results as oracle_lex_restart, plus the DFA's state count
 * (rows of delta) and the thread count; -1 on an invalid table or thread
 * count, or when memory runs out. */
int cpu_parallel_lex_restart(const uint8_t* bytes, uint64_t n, uint32_t n_states, uint32_t q0, const int16_t* delta,
                             const uint16_t* kind_of, uint32_t* kind, uint32_t* start, uint32_t* len, uint64_t cap,
                             uint32_t n_threads, uint64_t* n_tokens)
{
    if (n_states == 0 || n_states > MAX_STATES || q0 >= n_states || n_threads == 0) return -1;
    for (uint64_t x = 0; x < (uint64_t)n_states * 256; ++x)  /* states in range; the start state's row total */
        if (delta[x] >= (int32_t)n_states || (x / 256 == q0 && delta[x] < 0)) return -1;
    uint32_t T = n_threads > MAX_THREADS ? MAX_THREADS : n_threads;
    if (n < T) T = n ? (uint32_t)n : 1u;
    lex_job_t j = {bytes, n, T, n_states, {delta, q0}, kind_of, NULL, NULL, kind, start, len, cap};
    j.vec = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)T * n_states);
    j.sl = (lex_slice_t*)calloc(T, sizeof(lex_slice_t));
    int rc = (j.vec && j.sl) ? 0 : -1;
    if (rc == 0) rc = run_threads(T, lex_vectors, &j);
    if (rc == 0) {
        uint32_t q = q0;
        for (uint32_t t = 0; t < T; ++t) {
            j.sl[t].q_in = q;
            q = j.vec[(size_t)t * n_states + q];
        }
        rc = run_threads(T, lex_ends, &j);
        for (uint32_t t = 0; t < T && rc == 0; ++t)
            if (j.sl[t].ends.failed) rc = -1;
    }
    if (rc == 0) {
        uint64_t k = 0, s = 0;
        for (uint32_t t = 0; t < T; ++t) {
            lex_slice_t* x = &j.sl[t];
            x->t_in = k;
            x->start_in = s;
            k += x->ends.size;
            if (x->ends.size) s = x->ends.v[x->ends.size - 1] >> 16;
        }
        rc = run_threads(T, lex_write, &j);
        if (rc == 0) {
            if (n > 0) {  /* the last token ends at n */
                if (k < cap) {
                    kind[k] = kind_of[j.sl[T - 1].q_out];
                    start[k] = (uint32_t)s;
                    len[k] = (uint32_t)(n - s);
                }
                k++;
            }
            *n_tokens = k;
            rc = k > cap ? -2 : 0;
        }
    }
    if (j.sl)
        for (uint32_t t = 0; t < T; ++t) free(j.sl[t].ends.v);
    free(j.vec);
    free(j.sl);
    return rc;
}
