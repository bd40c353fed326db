/*
 * Seeded synthetic inputs for the delimiter-separated and lexer workloads.
 *
 * This file writes bytes and, when asked, the spans it placed (ground truth). It
 * contains no parsing arithmetic: no DFA is run here, no delimiter is classified,
 * nothing is scanned. It is shared by the CPU oracle's tests and by the HIP path's
 * tests and benchmark, and by nothing else.
 *
 * Random numbers: xoshiro256** (Blackman & Vigna, "Scrambled linear pseudorandom
 * number generators", ACM TOMS 2021), its 256-bit state filled from the seed by
 * four draws of splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), as the xoshiro authors recommend.
 * Integers below m use the 128-bit multiply-high map; Bernoulli draws compare one
 * 64-bit draw with an integer threshold p * 2^64, so every stream is bit-reproducible.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint64_t s[4]; } rng_t;

static uint64_t splitmix64(uint64_t* x)
{
    uint64_t z = (*x += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static inline uint64_t rotl64(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static inline uint64_t rng_next(rng_t* r)
{
    uint64_t* s = r->s;
    const uint64_t result = rotl64(s[1] * 5, 7) * 9;
    const uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return result;
}

static void rng_seed(rng_t* r, uint64_t seed)
{
    uint64_t x = seed;
    for (int i = 0; i < 4; ++i) r->s[i] = splitmix64(&x);
}

/* uniform integer in [0, m) */
static inline uint64_t rng_below(rng_t* r, uint64_t m)
{
    return (uint64_t)(((unsigned __int128)rng_next(r) * (unsigned __int128)m) >> 64);
}

static inline int rng_bern(rng_t* r, uint64_t thr) { return rng_next(r) < thr; }

/* ---- exported PRNG probes (so tests can pin the generator to its published definition) ---- */

void wl_splitmix64_stream(uint64_t seed, uint64_t* out, uint64_t count)
{
    uint64_t x = seed;
    for (uint64_t i = 0; i < count; ++i) out[i] = splitmix64(&x);
}

void wl_xoshiro_stream(const uint64_t state[4], uint64_t* out, uint64_t count)
{
    rng_t r;
    memcpy(r.s, state, sizeof r.s);
    for (uint64_t i = 0; i < count; ++i) out[i] = rng_next(&r);
}

void wl_xoshiro_seeded_stream(uint64_t seed, uint64_t* out, uint64_t count)
{
    rng_t r;
    rng_seed(&r, seed);
    for (uint64_t i = 0; i < count; ++i) out[i] = rng_next(&r);
}

/* ---- delimiter-separated text ---- */

static const char ALNUM[] = "0123456789ABCDEFGHIJKLMNOPQRSTUVWXYZabcdefghijklmnopqrstuvwxyz";

typedef struct {
    uint64_t seed;
    uint64_t n;           /* exact number of bytes written */
    uint32_t n_cols;      /* fields per ordinary record */
    uint32_t len_kind;    /* 0: uniform [len_lo, len_hi]; 1: geometric, p = 1/geo_den on {0,1,..}, capped at len_hi;
                             2: decimal number text, length uniform [len_lo, len_hi] */
    uint32_t len_lo, len_hi, geo_den;
    uint32_t comment_max; /* comment body length uniform [0, comment_max] */
    uint8_t fdelim, rdelim, quote, comment; /* comment == 0: no comment lines */
    uint32_t pad;
    uint64_t thr_quoted;  /* P(field is quoted)              * 2^64 */
    uint64_t thr_emb_f;   /* P(one field delimiter inside)   * 2^64 (quoted fields only) */
    uint64_t thr_emb_r;   /* P(one record delimiter inside)  * 2^64 (quoted fields only) */
    uint64_t thr_escape;  /* P(one doubled quote inside)     * 2^64 (quoted fields only) */
    uint64_t thr_comment; /* P(record is a comment line)     * 2^64 */
} wl_csv_params;

typedef struct {
    uint32_t *rec, *col, *off, *len; /* may be NULL */
    uint64_t cap;
    uint64_t count;                  /* out: fields placed (may exceed cap) */
    uint64_t records;                /* out */
} wl_truth;

/* n symbols uniform over alphabet[0..m) (m <= 64): the base-m digits of one 64-bit
 * draw read as a fraction in [0,1), eight digits per draw */
static void fill_from(rng_t* r, uint8_t* buf, uint64_t n, const char* alphabet, uint32_t m)
{
    uint64_t i = 0;
    while (i < n) {
        uint64_t x = rng_next(r);
        for (int j = 0; j < 8 && i < n; ++j) {
            unsigned __int128 p = (unsigned __int128)x * m;
            buf[i++] = (uint8_t)alphabet[(uint32_t)(p >> 64)];
            x = (uint64_t)p;
        }
    }
}

static const char DIGITS[] = "0123456789";

/* geometric thresholds: thr[k] = floor(2^64 * P(X <= k)), X ~ Geom(p) on {0,1,...} */
static uint64_t* geo_table(uint32_t den, uint32_t cap)
{
    uint64_t* t = (uint64_t*)malloc(sizeof(uint64_t) * (cap + 1));
    if (!t) return NULL;
    double q = 1.0 - 1.0 / (double)den, tail = 1.0;
    for (uint32_t k = 0; k <= cap; ++k) {
        tail *= q; /* P(X > k) = q^(k+1) */
        double cdf = 1.0 - tail;
        t[k] = cdf >= 1.0 ? UINT64_MAX : (uint64_t)(cdf * 18446744073709551616.0);
    }
    return t;
}

static uint32_t draw_geo(rng_t* r, const uint64_t* t, uint32_t cap)
{
    uint64_t u = rng_next(r);
    uint32_t lo = 0, hi = cap; /* smallest k with u < t[k], else cap */
    if (u >= t[cap]) return cap;
    while (lo < hi) {
        uint32_t mid = (lo + hi) / 2;
        if (u < t[mid]) hi = mid; else lo = mid + 1;
    }
    return lo;
}

static uint32_t draw_len(rng_t* r, const wl_csv_params* p, const uint64_t* geo)
{
    if (p->len_kind == 1) return draw_geo(r, geo, p->len_hi);
    return p->len_lo + (uint32_t)rng_below(r, (uint64_t)(p->len_hi - p->len_lo) + 1);
}

/* write one field's raw bytes into buf, return its length */
static uint32_t make_field(rng_t* r, const wl_csv_params* p, const uint64_t* geo, uint8_t* buf, uint8_t* tmp)
{
    uint32_t L = draw_len(r, p, geo);
    if (p->len_kind == 2) { /* decimal number text */
        int as_float = (int)rng_below(r, 2) && L >= 3;
        if (as_float) {
            uint32_t ip = 1 + (uint32_t)rng_below(r, L - 2);
            fill_from(r, buf, L, DIGITS, 10);
            buf[ip] = '.';
        } else {
            fill_from(r, buf, L, DIGITS, 10);
            if (L >= 2 && rng_below(r, 2)) buf[0] = '-';
        }
        return L;
    }
    if (!(p->thr_quoted && rng_bern(r, p->thr_quoted))) {
        fill_from(r, buf, L, ALNUM, 62);
        return L;
    }
    /* quoted: content = L alnum bytes with up to three inserted specials */
    uint32_t cl = L;
    fill_from(r, tmp, L, ALNUM, 62);
    const uint8_t specials[3] = { p->fdelim, p->rdelim, p->quote };
    const uint64_t thr[3] = { p->thr_emb_f, p->thr_emb_r, p->thr_escape };
    for (int s = 0; s < 3; ++s) {
        if (thr[s] && rng_bern(r, thr[s])) {
            uint32_t at = (uint32_t)rng_below(r, (uint64_t)cl + 1);
            memmove(tmp + at + 1, tmp + at, cl - at);
            tmp[at] = specials[s];
            cl++;
        }
    }
    uint32_t o = 0;
    buf[o++] = p->quote;
    for (uint32_t i = 0; i < cl; ++i) {
        buf[o++] = tmp[i];
        if (tmp[i] == p->quote) buf[o++] = p->quote; /* RFC 4180 doubling */
    }
    buf[o++] = p->quote;
    return o;
}

static void truth_put(wl_truth* t, uint64_t rec, uint64_t col, uint64_t off, uint64_t len)
{
    if (!t) return;
    if (t->rec && t->count < t->cap) {
        t->rec[t->count] = (uint32_t)rec;
        t->col[t->count] = (uint32_t)col;
        t->off[t->count] = (uint32_t)off;
        t->len[t->count] = (uint32_t)len;
    }
    t->count++;
}

/*
 * Records are generated until the next one would not fit in n bytes; the rest of the
 * budget is filled with alphanumeric bytes, which form one unquoted field of one more,
 * unterminated record (nothing if the budget is used up exactly).
 * Returns 0, or -1 on allocation failure.
 */
int wl_gen_csv(const wl_csv_params* p, uint8_t* out, wl_truth* truth)
{
    rng_t r;
    rng_seed(&r, p->seed);
    uint32_t maxf = 2 * (p->len_hi + 3) + 8;
    uint64_t maxrec = (uint64_t)p->n_cols * (maxf + 1) + p->comment_max + 8;
    uint8_t* rbuf = (uint8_t*)malloc(maxrec);
    uint8_t* tmp = (uint8_t*)malloc(maxf);
    uint32_t* foff = (uint32_t*)malloc(sizeof(uint32_t) * (p->n_cols + 1));
    uint32_t* flen = (uint32_t*)malloc(sizeof(uint32_t) * (p->n_cols + 1));
    uint64_t* geo = p->len_kind == 1 ? geo_table(p->geo_den, p->len_hi) : NULL;
    if (!rbuf || !tmp || !foff || !flen || (p->len_kind == 1 && !geo)) {
        free(rbuf); free(tmp); free(foff); free(flen); free(geo);
        return -1;
    }
    if (truth) { truth->count = 0; truth->records = 0; }
    uint64_t pos = 0, rec = 0;
    for (;;) {
        uint64_t rl = 0;
        uint32_t nf = 0;
        if (p->comment && p->thr_comment && rng_bern(&r, p->thr_comment)) {
            uint32_t cl = (uint32_t)rng_below(&r, (uint64_t)p->comment_max + 1);
            rbuf[rl++] = p->comment;
            for (uint32_t i = 0; i < cl; ++i) {
                uint32_t v = (uint32_t)rng_below(&r, 96); /* 95 printable ASCII bytes and TAB */
                rbuf[rl++] = v == 95 ? (uint8_t)'\t' : (uint8_t)(0x20 + v);
            }
            foff[0] = 0; flen[0] = (uint32_t)rl; nf = 1;
        } else {
            for (uint32_t c = 0; c < p->n_cols; ++c) {
                if (c) rbuf[rl++] = p->fdelim;
                foff[c] = (uint32_t)rl;
                flen[c] = make_field(&r, p, geo, rbuf + rl, tmp);
                rl += flen[c];
            }
            nf = p->n_cols;
        }
        rbuf[rl++] = p->rdelim;
        if (pos + rl > p->n) break;
        memcpy(out + pos, rbuf, rl);
        for (uint32_t c = 0; c < nf; ++c) truth_put(truth, rec, c, pos + foff[c], flen[c]);
        pos += rl;
        rec++;
    }
    if (pos < p->n) {
        fill_from(&r, out + pos, p->n - pos, ALNUM, 62);
        truth_put(truth, rec, 0, pos, p->n - pos);
        rec++;
    }
    if (truth) truth->records = rec;
    free(rbuf); free(tmp); free(foff); free(flen); free(geo);
    return 0;
}

/* ---- token streams for the lexer workload ----
 * Each generator entry owns a literal spelling or a pattern, and names the token
 * kind it produces. The caller supplies, for every ordered pair of entries (a, b),
 * what may sit between them: pair[a*ne+b] == 0 writes b right after a, 1..254
 * writes entry (pair-1) first as a separator, 255 forbids the pair (b is drawn
 * again). The caller derives that table from the token grammar; nothing here
 * looks at the grammar. Ground truth is the token sequence written. */

typedef struct {
    uint32_t pattern;     /* 0 literal, 1 identifier, 2 integer, 3 float, 4 string, 5 whitespace, 6 line comment */
    uint32_t kind;        /* token kind reported in the ground truth */
    uint32_t lit_off;     /* literal: offset into lits */
    uint32_t lit_len;
    uint32_t weight;      /* relative frequency (0: only ever written as a separator) */
} wl_token_entry;

static uint32_t write_token(rng_t* r, const wl_token_entry* k, const uint8_t* lits, uint8_t* b)
{
    static const char ID0[] = "abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZ_";
    static const char ID1[] = "abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZ_0123456789";
    static const char STR[] = "abcdefghijklmnopqrstuvwxyz ABCDEFGHIJKLMNOPQRSTUVWXYZ0123456789.,;:!?+-*/=<>()[]{}#$%&|^~'@`_";
    static const char ESCS[] = "\"\\nt";
    static const char WS[] = "    \t\n\n\r";
    static const char CM[] = "abcdefghijklmnopqrstuvwxyz ABCDEFGHIJ0123456789.,;:!?+-*/=<>()[]{}\"'\\#\t";
    uint32_t o = 0;
    switch (k->pattern) {
    case 0:
        memcpy(b, lits + k->lit_off, k->lit_len);
        return k->lit_len;
    case 1: {
        uint32_t L = 1 + (uint32_t)rng_below(r, 12);
        b[o++] = (uint8_t)ID0[rng_below(r, sizeof ID0 - 1)];
        while (o < L) b[o++] = (uint8_t)ID1[rng_below(r, sizeof ID1 - 1)];
        return o;
    }
    case 2: { /* decimal (70%), 0x hex (20%), 0b binary (10%) */
        static const char HX[] = "0123456789abcdefABCDEF";
        uint32_t form = (uint32_t)rng_below(r, 10);
        if (form < 7) {
            uint32_t L = 1 + (uint32_t)rng_below(r, 8);
            while (o < L) b[o++] = (uint8_t)('0' + rng_below(r, 10));
        } else {
            b[o++] = '0';
            b[o++] = form < 9 ? (rng_below(r, 2) ? 'x' : 'X') : (rng_below(r, 2) ? 'b' : 'B');
            uint32_t L = 1 + (uint32_t)rng_below(r, 8);
            for (uint32_t i = 0; i < L; ++i)
                b[o++] = form < 9 ? (uint8_t)HX[rng_below(r, sizeof HX - 1)] : (uint8_t)('0' + rng_below(r, 2));
        }
        return o;
    }
    case 3: { /* digits '.' digits [exponent] (80%), digits exponent (20%) */
        uint32_t a = 1 + (uint32_t)rng_below(r, 5);
        while (o < a) b[o++] = (uint8_t)('0' + rng_below(r, 10));
        int dotted = rng_below(r, 5) != 0;
        if (dotted) {
            uint32_t f = 1 + (uint32_t)rng_below(r, 5);
            b[o++] = '.';
            for (uint32_t i = 0; i < f; ++i) b[o++] = (uint8_t)('0' + rng_below(r, 10));
        }
        if (!dotted || rng_below(r, 4) == 0) {
            b[o++] = rng_below(r, 2) ? 'e' : 'E';
            uint32_t s = (uint32_t)rng_below(r, 3);
            if (s == 1) b[o++] = '+';
            if (s == 2) b[o++] = '-';
            uint32_t e = 1 + (uint32_t)rng_below(r, 3);
            for (uint32_t i = 0; i < e; ++i) b[o++] = (uint8_t)('0' + rng_below(r, 10));
        }
        return o;
    }
    case 4: { /* string: printable content, 10% escapes (one in five of them \xHH) */
        static const char HX[] = "0123456789abcdefABCDEF";
        uint32_t L = (uint32_t)rng_below(r, 24);
        b[o++] = '"';
        for (uint32_t i = 0; i < L; ++i) {
            if (rng_below(r, 10) == 0) {
                b[o++] = '\\';
                uint32_t e = (uint32_t)rng_below(r, 5);
                if (e < 4) {
                    b[o++] = (uint8_t)ESCS[e];
                } else {
                    b[o++] = 'x';
                    b[o++] = (uint8_t)HX[rng_below(r, sizeof HX - 1)];
                    b[o++] = (uint8_t)HX[rng_below(r, sizeof HX - 1)];
                }
            } else {
                b[o++] = (uint8_t)STR[rng_below(r, sizeof STR - 1)];
            }
        }
        b[o++] = '"';
        return o;
    }
    case 5: {
        uint32_t L = 1 + (uint32_t)rng_below(r, 4);
        while (o < L) b[o++] = (uint8_t)WS[rng_below(r, sizeof WS - 1)];
        return o;
    }
    case 6: {
        uint32_t L = (uint32_t)rng_below(r, 40);
        b[o++] = '/';
        b[o++] = '/';
        for (uint32_t i = 0; i < L; ++i) b[o++] = (uint8_t)CM[rng_below(r, sizeof CM - 1)];
        return o;
    }
    }
    return 0;
}

/*
 * Fill exactly n bytes with a token stream. Entries are drawn by weight; the pair
 * table decides what goes between neighbours. When the next token (with its
 * separator) would not fit, the rest of the budget is filled with pad_byte: those
 * bytes lengthen the last token when absorbs_pad[last entry] is set (the caller
 * knows which spellings run on through that byte), and otherwise form one token of
 * kind pad_kind. Returns 0, or -1 on bad arguments.
 */
int wl_gen_tokens(uint64_t seed, uint64_t n, const wl_token_entry* ents, uint32_t ne, const uint8_t* lits,
                  const uint8_t* pair, const uint8_t* absorbs_pad, uint32_t pad_kind, uint8_t pad_byte,
                  uint8_t* out, wl_truth* truth)
{
    rng_t r;
    rng_seed(&r, seed);
    uint64_t wsum = 0;
    for (uint32_t i = 0; i < ne; ++i) wsum += ents[i].weight;
    if (!wsum) return -1;
    uint8_t buf[512];
    uint64_t pos = 0;
    int64_t prev = -1;
    if (truth) { truth->count = 0; truth->records = 0; }
    for (;;) {
        uint64_t u = rng_below(&r, wsum);
        uint32_t k = 0;
        while (u >= ents[k].weight) { u -= ents[k].weight; ++k; }
        uint32_t o = 0, sl = 0, sk = 0;
        if (prev >= 0) {
            uint8_t pv = pair[(uint64_t)prev * ne + k];
            if (pv == 255) continue;
            if (pv) {
                sk = pv - 1u;
                sl = write_token(&r, &ents[sk], lits, buf);
                o = sl;
            }
        }
        uint32_t tl = write_token(&r, &ents[k], lits, buf + o);
        o += tl;
        if (pos + o > n) break;
        memcpy(out + pos, buf, o);
        if (sl) truth_put(truth, ents[sk].kind, 0, pos, sl);
        truth_put(truth, ents[k].kind, 0, pos + sl, tl);
        pos += o;
        prev = k;
    }
    if (pos < n) {
        memset(out + pos, pad_byte, n - pos);
        if (prev >= 0 && absorbs_pad[prev]) {
            if (truth && truth->len && truth->count - 1 < truth->cap) truth->len[truth->count - 1] += (uint32_t)(n - pos);
        } else {
            truth_put(truth, pad_kind, 0, pos, n - pos);
        }
    }
    return 0;
}
