// Numeric type inference and conversion of fields.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", "Type inference" (each field's minimal numerical type, then a
// reduction over a column's fields), "Default values for empty strings", and
// Sec. 3 (a field's symbol string converted to its column's type, threads
// working alone on short fields and collaborating on long ones; the pages'
// example block is 64 threads, one wave here).
//
// A field's text is its raw span. Its type is one of EMPTY < INT8 < INT16 <
// INT32 < INT64 < FLOAT64 < TEXT, from a 10-state automaton for the number
// grammar (optional sign; digits with or without a point; optional exponent)
// run over its bytes while the digits are folded into:
//   mag    the integer's magnitude (flag beyond 2^63), for INT fields;
//   w, z   the significant digits without leading zeros, trailing zeros kept
//          pending in z (flag beyond 2^53), and the fraction digits and the
//          exponent, so that |value| = w * 10^e10 with e10 = exp - frac + z.
// Conversion gives int64 values, or doubles in the class where one IEEE
// multiplication or division of exact operands rounds correctly (w <= 2^53
// and |e10| <= 22, or e10 > 22 with w * 10^(e10 - 22) <= 2^53; Clinger's
// fast path); other floats are flagged inexact and hold NaN.
//
// Work split (per workgroup of 256 threads, 8 fields per thread): a thread
// runs the automaton over a field's first 32 bytes; a field that is still a
// number after them is queued in LDS, and a wave then classifies it by
// composing the automaton's state maps over 16-byte pieces, one per lane, in a
// wave scan (a text field thus costs the wave one pass over its bytes). A
// queued field that is a number (long digit strings: leading zeros, or more
// digits than 19) is folded by one lane. Column types reduce in LDS per
// workgroup, then by an atomic maximum.
#include <algorithm>

#include "ppr_host.h"
#include "ppr_scan.h"

namespace ppr {
namespace {

constexpr int kNumBlock = 256;
constexpr int kNumWaves = kNumBlock / kWave;
constexpr int kNumPer = 8;           // fields per thread
constexpr uint32_t kNumThread = 32;  // bytes a thread reads before it queues a field that is still a number
constexpr uint32_t kNumQueue = 256;  // queued fields per workgroup (more: the thread finishes them itself)
constexpr uint32_t kNumMaxColumns = 4096;

// automaton states; NX rejects
enum : uint32_t { NS0 = 0, NSIGN, NINT, NDOT, NPOINT, NFRAC, NE, NESIGN, NEXP, NX };
// byte classes: 0 digit, 1 sign, 2 point, 3 e or E, 4 other
__device__ __forceinline__ uint32_t num_class(uint32_t b)
{
    return b - '0' < 10u ? 0u : (b == '+' || b == '-') ? 1u : b == '.' ? 2u : (b == 'e' || b == 'E') ? 3u : 4u;
}
// next state of each state (4 bits each) for one class
constexpr uint64_t pack_next(const uint32_t (&t)[10])
{
    uint64_t r = 0;
    for (int s = 0; s < 10; ++s) r |= (uint64_t)t[s] << (4 * s);
    return r;
}
//                                       S0      SIGN    INT    DOT    POINT  FRAC   E       ESIGN  EXP   X
constexpr uint32_t kOnDigit[10] = {NINT, NINT, NINT, NFRAC, NFRAC, NFRAC, NEXP, NEXP, NEXP, NX};
constexpr uint32_t kOnSign[10] = {NSIGN, NX, NX, NX, NX, NX, NESIGN, NX, NX, NX};
constexpr uint32_t kOnPoint[10] = {NPOINT, NPOINT, NDOT, NX, NX, NX, NX, NX, NX, NX};
constexpr uint32_t kOnExp[10] = {NX, NX, NE, NE, NX, NE, NX, NX, NX, NX};
constexpr uint32_t kOnOther[10] = {NX, NX, NX, NX, NX, NX, NX, NX, NX, NX};
constexpr uint64_t kNextDigit = pack_next(kOnDigit), kNextSign = pack_next(kOnSign), kNextPoint = pack_next(kOnPoint),
                   kNextExp = pack_next(kOnExp), kNextOther = pack_next(kOnOther);

// the transitions of class c, from immediates (a per-lane index into a table
// in memory would be a vector load per byte)
__device__ __forceinline__ uint64_t num_next(uint32_t c)
{
    return c == 0u ? kNextDigit : c == 1u ? kNextSign : c == 2u ? kNextPoint : c == 3u ? kNextExp : kNextOther;
}
__device__ __forceinline__ uint32_t num_step(uint32_t s, uint32_t c) { return (uint32_t)(num_next(c) >> (4 * s)) & 15u; }

constexpr uint64_t kTwo53 = 1ull << 53;
constexpr uint64_t kTwo63 = 1ull << 63;
constexpr uint64_t kExpCap = 1ull << 40;  // exponent digits saturate here (e10 then cannot be small)

struct NumAcc {
    uint32_t s, neg, mag_ovf, big, eneg;
    uint32_t z;     // pending zeros after the last nonzero significant digit
    uint64_t mag;   // integer magnitude (integer-part digits), up to 2^63
    uint64_t w;     // significant digits, up to 2^53
    uint64_t frac;  // digits after the point
    uint64_t ev;    // exponent digits' value, saturating
};

__device__ __forceinline__ NumAcc num_init() { return NumAcc{NS0, 0u, 0u, 0u, 0u, 0u, 0ull, 0ull, 0ull, 0ull}; }

__device__ __forceinline__ void num_fold_sig_slow(NumAcc& a, uint32_t d)
{
    uint64_t w = a.w;
    for (uint32_t k = 0; k <= a.z; ++k) {  // w * 10^(z + 1), stopping beyond 2^53
        w *= 10u;
        if (w > kTwo53) {
            a.big = 1;
            return;
        }
    }
    w += d;
    if (w > kTwo53) {
        a.big = 1;
        return;
    }
    a.w = w;
    a.z = 0;
}

// a significant digit into (w, z): zeros stay pending, a nonzero digit
// multiplies them in; the common case (no pending zeros, w far below 2^53)
// is one multiply-add
__device__ __forceinline__ void num_fold_sig(NumAcc& a, uint32_t d)
{
    if (a.big) return;
    if (d == 0) {
        if (a.w) ++a.z;  // (a leading zero adds nothing)
    } else if (a.z == 0 && a.w < kTwo53 / 10u) {
        a.w = a.w * 10u + d;
    } else {
        num_fold_sig_slow(a, d);
    }
}

// One byte, without branches (selects) where the thread is active (act); the
// rare slow fold (pending zeros, or w near 2^53) is the only branch.
__device__ __forceinline__ void num_byte_p(NumAcc& a, uint32_t b, bool act)
{
    const uint32_t c = num_class(b), s = a.s, d = b - '0';
    const bool dig = act && c == 0u;
    const bool in_int = s <= NINT, in_frac = s >= NDOT && s <= NFRAC, in_exp = s >= NE && s <= NEXP;
    const bool minus = b == '-';
    a.neg = (act && c == 1u && s == NS0) ? minus : a.neg;
    a.eneg = (act && c == 1u && s == NE) ? minus : a.eneg;
    // integer magnitude, up to 2^63
    const bool upd = dig && in_int && !a.mag_ovf;
    const bool fits = a.mag < kTwo63 / 10u || (a.mag == kTwo63 / 10u && d <= 8u);
    const uint64_t m10 = a.mag * 10u + d;
    a.mag = upd && fits ? m10 : a.mag;
    a.mag_ovf |= (upd && !fits) ? 1u : 0u;
    // fraction digits and exponent
    a.frac += (dig && in_frac) ? 1u : 0u;
    const uint64_t e10 = min(a.ev * 10u + d, kExpCap);
    a.ev = (dig && in_exp) ? e10 : a.ev;
    // significant digits: zeros pending, one multiply-add in the common case
    const bool sig = dig && (in_int || in_frac) && !a.big;
    const bool zero = d == 0u;
    const bool fast = sig && !zero && a.z == 0u && a.w < kTwo53 / 10u;
    a.z += (sig && zero && a.w != 0u) ? 1u : 0u;
    a.w = fast ? a.w * 10u + d : a.w;
    if (sig && !zero && !fast) num_fold_sig_slow(a, d);
    a.s = act ? num_step(s, c) : s;
}

__device__ __forceinline__ void num_byte(NumAcc& a, uint32_t b)
{
    const uint32_t c = num_class(b), s = a.s;
    if (c == 1u) {
        if (s == NS0) a.neg = b == '-';
        if (s == NE) a.eneg = b == '-';
    } else if (c == 0u) {
        const uint32_t d = b - '0';
        if (s <= NINT) {  // integer part (S0, SIGN, INT)
            if (!a.mag_ovf) {  // up to 2^63: below 2^63 / 10 the next digit always fits
                if (a.mag < kTwo63 / 10u) a.mag = a.mag * 10u + d;
                else if (a.mag == kTwo63 / 10u && d <= 8u) a.mag = a.mag * 10u + d;
                else a.mag_ovf = 1;
            }
            num_fold_sig(a, d);
        } else if (s <= NFRAC) {  // fraction (DOT, POINT, FRAC)
            ++a.frac;
            num_fold_sig(a, d);
        } else if (s != NX) {  // exponent (E, ESIGN, EXP)
            a.ev = min(a.ev * 10u + d, kExpCap);
        }
    }
    a.s = num_step(s, c);
}

// the type of a field whose bytes have all been folded into a (len > 0)
__device__ __forceinline__ uint32_t num_type(const NumAcc& a)
{
    if (a.s == NINT) {
        if (a.mag_ovf || (!a.neg && a.mag == kTwo63)) return PPR_NUM_FLOAT64;
        const uint64_t m = a.mag;
        const uint64_t b8 = a.neg ? 128u : 127u, b16 = a.neg ? 32768u : 32767u, b32 = a.neg ? 2147483648u : 2147483647u;
        return m <= b8 ? PPR_NUM_INT8 : m <= b16 ? PPR_NUM_INT16 : m <= b32 ? PPR_NUM_INT32 : PPR_NUM_INT64;
    }
    return (a.s == NDOT || a.s == NFRAC || a.s == NEXP) ? PPR_NUM_FLOAT64 : PPR_NUM_TEXT;
}

__constant__ double kPow10[23] = {1e0,  1e1,  1e2,  1e3,  1e4,  1e5,  1e6,  1e7,  1e8,  1e9,  1e10, 1e11,
                                  1e12, 1e13, 1e14, 1e15, 1e16, 1e17, 1e18, 1e19, 1e20, 1e21, 1e22};
constexpr uint64_t kNaNBits = 0x7ff8000000000000ull;

// the double of a number (INT or FLOAT text) in the exact class; false outside it
__device__ __forceinline__ bool num_exact(const NumAcc& a, double& out)
{
    if (a.big) return false;
    if (a.w == 0) {
        out = a.neg ? -0.0 : 0.0;
        return true;
    }
    const int64_t e10 = (a.eneg ? -(int64_t)a.ev : (int64_t)a.ev) - (int64_t)a.frac + (int64_t)a.z;
    double r;
    if (e10 >= -22 && e10 <= 22) {
        r = e10 >= 0 ? (double)a.w * kPow10[e10] : (double)a.w / kPow10[-e10];
    } else if (e10 > 22 && e10 - 22 <= 15) {
        uint64_t w = a.w;
        for (int64_t k = 0; k < e10 - 22; ++k) {
            w *= 10u;
            if (w > kTwo53) return false;
        }
        r = (double)w * 1e22;
    } else {
        return false;
    }
    out = a.neg ? -r : r;
    return true;
}

struct NumParams {
    const uint8_t* bytes;
    uint64_t n_bytes;
    const uint32_t *off, *len, *col, *col_first;
    uint64_t n_fields;
    uint32_t n_columns;
    uint8_t* field_type;      // infer: optional output
    uint32_t* column_type;    // infer: maxima (device); convert: the column types (device)
    int64_t int_default;
    uint64_t float_default;   // bits
    uint64_t* values;         // convert
    uint8_t* status;          // convert
    unsigned long long* counts;  // convert: fields per status 1..4
};

// s_cf: the columns' first fields in LDS (when the fields are grouped by column)
__device__ __forceinline__ uint32_t column_of(const NumParams& p, uint64_t j, const uint32_t* s_cf)
{
    if (p.col) return p.col[j];
    if (!p.col_first) return 0u;
    uint32_t lo = 0;  // the last column whose first field is at or before j
    for (uint32_t step = 1u << 12; step; step >>= 1)
        if (lo + step < p.n_columns && s_cf[lo + step] <= j) lo += step;
    return lo;
}

// a field's result: its type (infer), or its value and status (convert)
// (convert: returns the status)
template <bool CONVERT>
__device__ __forceinline__ uint32_t num_finish(const NumParams& p, uint64_t j, uint32_t c, uint32_t len,
                                               const NumAcc& a, uint32_t* s_ct)
{
    const uint32_t t = len == 0 ? (uint32_t)PPR_NUM_EMPTY : num_type(a);
    if (!CONVERT) {
        if (p.field_type) p.field_type[j] = (uint8_t)t;
        if (c < p.n_columns && s_ct[c] < t) atomicMax(&s_ct[c], t);
        return 0u;
    }
    const uint32_t ct = c < p.n_columns ? s_ct[c] : (uint32_t)PPR_NUM_TEXT;
    const bool as_float = ct == PPR_NUM_FLOAT64;
    const uint64_t dflt = as_float ? p.float_default : (uint64_t)p.int_default;
    uint64_t v;
    uint32_t st;
    if (ct == PPR_NUM_TEXT) {
        v = 0;
        st = PPR_NUM_NOT_CONVERTED;
    } else if (t == PPR_NUM_EMPTY) {
        v = dflt;
        st = PPR_NUM_DEFAULTED;
    } else if (t > ct) {
        v = dflt;
        st = PPR_NUM_MISMATCH;
    } else if (!as_float) {
        v = a.neg ? (uint64_t)0 - a.mag : a.mag;
        st = PPR_NUM_OK;
    } else {
        double d;
        if (num_exact(a, d)) {
            v = (uint64_t)__double_as_longlong(d);
            st = PPR_NUM_OK;
        } else {
            v = kNaNBits;
            st = PPR_NUM_INEXACT;
        }
    }
    p.values[j] = v;
    p.status[j] = (uint8_t)st;
    return st;
}

// a field's bytes [from, to) folded into a, one by one (stops once rejected)
__device__ __forceinline__ void num_fold_range(const NumParams& p, uint64_t base, uint32_t from, uint32_t to, NumAcc& a)
{
    for (uint32_t i = from; i < to && a.s != NX; ++i) num_byte(a, p.bytes[base + i]);
}

// the automaton's state map over 16 bytes (4 bits per state), from x
__device__ __forceinline__ uint64_t piece_map(const uint4& x, uint32_t nb)
{
    uint64_t m = 0;
    for (uint32_t s = 0; s < 10; ++s) m |= (uint64_t)s << (4 * s);
    const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {
        const uint64_t nx = num_next(num_class((wd[i >> 2] >> (8 * (i & 3u))) & 0xffu));
        uint64_t r = 0;
#pragma unroll
        for (uint32_t s = 0; s < 10; ++s) r |= ((nx >> (4 * ((m >> (4 * s)) & 15u))) & 15u) << (4 * s);
        m = i < nb ? r : m;
    }
    return m;
}

struct MapComb {  // x earlier, y later: y after x
    __device__ uint64_t operator()(uint64_t x, uint64_t y) const
    {
        uint64_t r = 0;
#pragma unroll
        for (uint32_t s = 0; s < 10; ++s) r |= ((y >> (4 * ((x >> (4 * s)) & 15u))) & 15u) << (4 * s);
        return r;
    }
};

template <bool CONVERT>
__global__ void __launch_bounds__(kNumBlock) num_kernel(NumParams p)
{
    // dynamic LDS: the column types, then (fields grouped by column) the columns' first fields
    extern __shared__ __align__(16) uint32_t s_num_dyn[];
    uint32_t* s_ct = s_num_dyn;
    uint32_t* s_cf = s_num_dyn + p.n_columns;
    __shared__ uint32_t s_q[kNumQueue];
    __shared__ NumAcc s_qa[kNumQueue];
    __shared__ uint32_t s_qn, s_cnt[8];
    const uint32_t tid = threadIdx.x, lane = (uint32_t)lane_id(), w = tid / kWave;
    for (uint32_t c = tid; c < p.n_columns; c += kNumBlock) s_ct[c] = CONVERT ? p.column_type[c] : 0u;
    if (!p.col && p.col_first)
        for (uint32_t c = tid; c <= p.n_columns; c += kNumBlock) s_cf[c] = p.col_first[c];
    if (tid < 8) s_cnt[tid] = 0;
    if (tid == 0) s_qn = 0;
    __syncthreads();

    // statuses 1-4 of this thread's fields (16 bits each; convert only)
    uint32_t n12 = 0, n34 = 0;
    auto count = [&](uint32_t st) {
        n12 += st == 1u ? 1u : st == 2u ? 0x10000u : 0u;
        n34 += st == 3u ? 1u : st == 4u ? 0x10000u : 0u;
    };

    // (1) thread-exclusive: each thread's fields, up to 32 bytes of each. The
    // loads run ahead of the work: a field's offset, length and column two
    // fields ahead, its first 32 bytes one field ahead.
    const uint64_t j0 = (uint64_t)blockIdx.x * (kNumBlock * kNumPer);
    struct FieldAt {
        uint32_t o, L, c;
    };
    auto load_field = [&](uint32_t k) {
        FieldAt f{0u, 0u, 0u};
        const uint64_t j = j0 + (uint64_t)k * kNumBlock + tid;
        if (k < (uint32_t)kNumPer && j < p.n_fields) {
            f.o = p.off[j];
            f.L = p.len[j];
            f.c = column_of(p, j, s_cf);
        }
        return f;
    };
    auto load_head = [&](const FieldAt& f, uint4 (&x)[2]) {
        if ((uint64_t)f.o + kNumThread <= p.n_bytes) {
            __builtin_memcpy(&x[0], p.bytes + f.o, 16);
            __builtin_memcpy(&x[1], p.bytes + f.o + 16, 16);
        } else {
            x[0] = x[1] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    FieldAt f_next = load_field(0), f_after = load_field(1);
    uint4 x_next[2];
    load_head(f_next, x_next);
#pragma unroll 1
    for (uint32_t k = 0; k < (uint32_t)kNumPer; ++k) {
        const uint64_t j = j0 + (uint64_t)k * kNumBlock + tid;
        if (j >= p.n_fields) break;
        const FieldAt f = f_next;
        const uint4 x[2] = {x_next[0], x_next[1]};
        f_next = f_after;
        f_after = load_field(k + 2);
        load_head(f_next, x_next);
        const uint32_t o = f.o, L = f.L, c = f.c;
        NumAcc a = num_init();
        if ((uint64_t)o + L > p.n_bytes) a.s = NX;  // (a span past the text: never for a parse's own fields)
        const uint32_t head = min(L, kNumThread);
        if ((uint64_t)o + kNumThread <= p.n_bytes) {
            const uint32_t wd[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
#pragma unroll
            for (uint32_t i = 0; i < kNumThread; ++i) {
                const bool act = i < head && a.s != NX;
                if (__ballot(act))  // (uniform: the wave skips bytes no lane still needs)
                    num_byte_p(a, (wd[i >> 2] >> (8 * (i & 3u))) & 0xffu, act);
            }
        } else if (a.s != NX) {
            num_fold_range(p, o, 0, head, a);  // (the text's last 32 bytes)
        }
        if (L > kNumThread && a.s != NX) {
            const uint32_t qi = atomicAdd(&s_qn, 1u);
            if (qi < kNumQueue) {
                s_q[qi] = k * kNumBlock + tid;
                s_qa[qi] = a;
                continue;
            }
            num_fold_range(p, o, kNumThread, L, a);  // (queue full: the thread goes on alone)
        }
        count(num_finish<CONVERT>(p, j, c, L, a, s_ct));
    }
    __syncthreads();

    // (2) wave-level: the queued fields, one per wave at a time
    const uint32_t nq = min(s_qn, kNumQueue);
    for (uint32_t qi = w; qi < nq; qi += kNumWaves) {
        const uint64_t j = j0 + s_q[qi];
        const uint32_t o = p.off[j], L = p.len[j], c = column_of(p, j, s_cf);
        NumAcc a = s_qa[qi];
        uint32_t s = a.s;
        // the state after the bytes [32, L): pieces of 16 bytes, one per lane, composed by a wave scan
        for (uint32_t b0 = kNumThread; b0 < L && s != NX; b0 += 16u * kWave) {
            const uint32_t pb = b0 + 16u * lane;
            uint64_t m = 0;
            for (uint32_t t = 0; t < 10; ++t) m |= (uint64_t)t << (4 * t);
            if (pb < L) {
                const uint32_t nb = min(16u, L - pb);
                uint4 x = make_uint4(0u, 0u, 0u, 0u);
                if ((uint64_t)o + pb + 16u <= p.n_bytes) {
                    __builtin_memcpy(&x, p.bytes + o + pb, 16);
                } else {
                    uint32_t wd[4] = {0u, 0u, 0u, 0u};
                    for (uint32_t t = 0; t < nb; ++t) wd[t >> 2] |= (uint32_t)p.bytes[o + pb + t] << (8 * (t & 3u));
                    x = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
                m = piece_map(x, nb);
            }
            const uint64_t all = readlane_t(wave_scan(m, (uint64_t)0x9876543210ull, MapComb{}), kWave - 1);
            s = (uint32_t)(all >> (4 * s)) & 15u;
        }
        if (s != NX && lane == 0) num_fold_range(p, o, kNumThread, L, a);  // a long number: one lane folds the rest
        else a.s = NX;
        if (lane == 0) count(num_finish<CONVERT>(p, j, c, L, a, s_ct));
    }
    if (CONVERT) {  // the wave's counts, into the workgroup's
        n12 = readlane_t(wave_scan(n12, 0u, AddU32{}), kWave - 1);
        n34 = readlane_t(wave_scan(n34, 0u, AddU32{}), kWave - 1);
        if (lane == 0) {
            atomicAdd(&s_cnt[1], n12 & 0xffffu);
            atomicAdd(&s_cnt[2], n12 >> 16);
            atomicAdd(&s_cnt[3], n34 & 0xffffu);
            atomicAdd(&s_cnt[4], n34 >> 16);
        }
    }
    __syncthreads();

    // (3) the workgroup's column maxima (infer) or status counts (convert), into the call's
    if (!CONVERT) {
        for (uint32_t c = tid; c < p.n_columns; c += kNumBlock) {
            const uint32_t t = s_ct[c];
            if (t && __hip_atomic_load(&p.column_type[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < t)
                atomicMax(&p.column_type[c], t);
        }
    } else if (tid >= 1 && tid <= 4 && s_cnt[tid]) {
        atomicAdd(&p.counts[tid - 1], (unsigned long long)s_cnt[tid]);
    }
}

__global__ void num_reset_kernel(uint32_t* column_type, uint32_t n_columns, unsigned long long* counts)
{
    for (uint32_t c = threadIdx.x; c < n_columns; c += blockDim.x) column_type[c] = 0u;
    if (threadIdx.x < 4) counts[threadIdx.x] = 0ull;
}

struct NumLayout {
    uint64_t counts, types, total;
};
inline NumLayout num_layout(uint32_t n_columns)
{
    NumLayout L;
    L.counts = 0;
    L.types = 256;
    L.total = align_up(L.types + (uint64_t)std::max<uint32_t>(n_columns, 1) * 4, 256);
    return L;
}

int num_check(const ppr_fields_t* f, void* d_ws, size_t ws_bytes)
{
    if (!f || !d_ws || f->n_columns == 0 || f->n_columns > kNumMaxColumns) return PPR_EINVAL;
    if (f->n_fields && (!f->bytes || !f->off || !f->len)) return PPR_EINVAL;
    if (f->n_fields >= (1ull << 40)) return PPR_ETOOBIG;
    if ((uintptr_t)d_ws & 255u) return PPR_EWORKSPACE;
    if (ws_bytes < num_layout(f->n_columns).total) return PPR_EWORKSPACE;
    return PPR_OK;
}

NumParams num_params(const ppr_fields_t* f, uint8_t* ws)
{
    NumParams p;
    memset(&p, 0, sizeof p);
    p.bytes = f->bytes;
    p.n_bytes = f->n_bytes;
    p.off = f->off;
    p.len = f->len;
    p.col = f->col;
    p.col_first = f->col ? nullptr : f->col_first;
    p.n_fields = f->n_fields;
    p.n_columns = f->n_columns;
    const NumLayout L = num_layout(f->n_columns);
    p.counts = reinterpret_cast<unsigned long long*>(ws + L.counts);
    p.column_type = reinterpret_cast<uint32_t*>(ws + L.types);
    return p;
}

inline size_t num_lds(const NumParams& p)
{
    return (size_t)p.n_columns * 4u + (!p.col && p.col_first ? ((size_t)p.n_columns + 1u) * 4u : 0u);
}

inline uint32_t num_grid(uint64_t n_fields)
{
    return (uint32_t)std::max<uint64_t>((n_fields + kNumBlock * kNumPer - 1) / (kNumBlock * kNumPer), 1);
}

}  // namespace
}  // namespace ppr

using namespace ppr;

extern "C" PPR_API size_t ppr_numbers_workspace_bytes(uint32_t n_columns)
{
    if (n_columns == 0 || n_columns > kNumMaxColumns) return 0;
    return (size_t)num_layout(n_columns).total;
}

extern "C" PPR_API int ppr_infer_types(const ppr_fields_t* f, uint8_t* d_field_type, uint32_t* column_type,
                                       void* d_ws, size_t ws_bytes, void* stream)
{
    int rc = num_check(f, d_ws, ws_bytes);
    if (rc) return rc;
    if (!column_type) return PPR_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    NumParams p = num_params(f, (uint8_t*)d_ws);
    p.field_type = d_field_type;
    hipLaunchKernelGGL(num_reset_kernel, dim3(1), dim3(256), 0, s, p.column_type, p.n_columns, p.counts);
    if (f->n_fields)
        hipLaunchKernelGGL(num_kernel<false>, dim3(num_grid(f->n_fields)), dim3(kNumBlock), num_lds(p), s, p);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    if (hipMemcpyAsync(column_type, p.column_type, (size_t)f->n_columns * 4u, hipMemcpyDeviceToHost, s) != hipSuccess)
        return PPR_EHIP;
    return hipStreamSynchronize(s) == hipSuccess ? PPR_OK : PPR_EHIP;
}

extern "C" PPR_API int ppr_convert(const ppr_fields_t* f, const uint32_t* column_type, int64_t int_default,
                                   double float_default, uint64_t* d_values, uint8_t* d_status, uint64_t counts[4],
                                   void* d_ws, size_t ws_bytes, void* stream)
{
    int rc = num_check(f, d_ws, ws_bytes);
    if (rc) return rc;
    if (!column_type || (f->n_fields && (!d_values || !d_status))) return PPR_EINVAL;
    for (uint32_t c = 0; c < f->n_columns; ++c)
        if (column_type[c] > PPR_NUM_TEXT) return PPR_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    NumParams p = num_params(f, (uint8_t*)d_ws);
    p.int_default = int_default;
    uint64_t fb;
    memcpy(&fb, &float_default, 8);
    p.float_default = fb;
    p.values = d_values;
    p.status = d_status;
    hipLaunchKernelGGL(num_reset_kernel, dim3(1), dim3(256), 0, s, p.column_type, 0u, p.counts);
    if (hipMemcpyAsync(p.column_type, column_type, (size_t)f->n_columns * 4u, hipMemcpyHostToDevice, s) != hipSuccess)
        return PPR_EHIP;
    if (f->n_fields)
        hipLaunchKernelGGL(num_kernel<true>, dim3(num_grid(f->n_fields)), dim3(kNumBlock), num_lds(p), s, p);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    unsigned long long h[4];
    if (hipMemcpyAsync(h, p.counts, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    if (counts)
        for (int i = 0; i < 4; ++i) counts[i] = h[i];
    return PPR_OK;
}
