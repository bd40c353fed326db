// Single-pass data-parallel DFA parse of delimiter-separated bytes on gfx950.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", Sec. 3. Every thread owns a chunk of bytes and runs one DFA instance
// per state over it, producing its state-transition vector (Fig. 2). An
// exclusive scan of the vectors under composition, seeded with the identity,
// gives each chunk its true start state. Each thread then re-simulates its chunk
// from that state and tags every byte (record delimiter, field delimiter, value,
// invalid), keeping the two delimiter bitmaps. Record counts (POPCNT +
// exclusive sum) and relative/absolute column offsets (Fig. 4) are scanned the
// same way, and every field is written out with its record, column, offset and
// length.
//
// MI355X mapping (not the page's CUDA design):
//   * one workgroup is one tile (512 threads x 64 bytes on the fast path); the
//     device-wide scans are decoupled look-backs (ppr_scan.h) in which every wave
//     of the workgroup reads 64 predecessors per round; two look-backs run in
//     one kernel, the state vectors first (known right after the first pass),
//     then the field/record/column carries (known only after the
//     re-simulation); a tile's index is its workgroup index (workgroups start in
//     index order on each XCD, so every tile a workgroup waits on has started);
//   * a state-transition vector is one byte per state in one or two VGPRs, so a
//     composite is one or two v_perm_b32 byte selects (ParPaRaw keeps such small
//     arrays in registers with bit-field insert/extract, Fig. 8);
//   * fast path (csv_fast_kernel): 64-byte chunks read with 16-byte loads; the
//     symbol group of four bytes at once by a v_perm hash lookup and an exact
//     compare (ParPaRaw matches symbols with SWAR, Table 2); an absorbing state
//     (such as INV) is the byte 0xFF, which v_perm maps to itself, so it needs
//     no vector entry; both passes step G = 2 or 4 bytes per LDS table lookup:
//     the pass-1 table holds the composite vector of every G-symbol string, the
//     pass-2 table the end state and terminator bits from every state;
//   * generic path (csv_generic_kernel): any table, chunk size 1..64, one byte
//     at a time from LDS.
#include "ppr.h"
#include "ppr_device.h"
#include "ppr_host.h"
#include "ppr_scan.h"

namespace ppr {

constexpr int kBlock = 256;      // generic path
constexpr int kWaves = kBlock / kWave;
constexpr int kFastBlock = 512;  // fast path: 32 KiB tiles
constexpr int kFastWaves = kFastBlock / kWave;
constexpr int kMaxChunk = 64;
constexpr int kFastChunk = 64;
constexpr uint32_t kNone = 0xffffffffu;
constexpr uint32_t kAbs = 0xffu;  // state code of the absorbing state (fast path)

// Carries of a run of bytes [ParPaRaw Sec. 3, offsets, Fig. 4]:
//   nf terminators, nr record delimiters,
//   column offset handed to what follows: absolute (a record delimiter was seen:
//     field delimiters after the last one) or relative (field delimiters seen),
//   lt = 1 + position of the last terminator (0: none),
//   err = first INVALID byte (kNone: none).
struct Carry {
    uint32_t nf, nr, colv, colabs, lt, err;
};

__device__ __forceinline__ Carry carry_identity() { return {0u, 0u, 0u, 0u, 0u, kNone}; }

// x earlier, y later. The column rule: a resolved (absolute) later offset wins,
// a relative one adds to the earlier offset. lt and err are absolute positions,
// so "last defined" and "first defined" are max and min.
__device__ __forceinline__ Carry carry_op(const Carry& x, const Carry& y)
{
    Carry r;
    r.nf = x.nf + y.nf;
    r.nr = x.nr + y.nr;
    r.colv = y.colabs ? y.colv : x.colv + y.colv;
    r.colabs = y.colabs | x.colabs;
    r.lt = max(x.lt, y.lt);
    r.err = min(x.err, y.err);
    return r;
}

__device__ __forceinline__ Carry shfl_up_carry(const Carry& c, int d)
{
    return {shfl_up(c.nf, d), shfl_up(c.nr, d), shfl_up(c.colv, d), shfl_up(c.colabs, d), shfl_up(c.lt, d),
            shfl_up(c.err, d)};
}
__device__ __forceinline__ Carry shfl_down_carry(const Carry& c, int d)
{
    return {shfl_down(c.nf, d), shfl_down(c.nr, d), shfl_down(c.colv, d), shfl_down(c.colabs, d),
            shfl_down(c.lt, d), shfl_down(c.err, d)};
}
__device__ __forceinline__ Carry shfl_carry(const Carry& c, int src)
{
    return {shfl(c.nf, src), shfl(c.nr, src), shfl(c.colv, src), shfl(c.colabs, src), shfl(c.lt, src),
            shfl(c.err, src)};
}
__device__ __forceinline__ Vec shfl_up_vec(Vec v, int d) { return {shfl_up(v.lo, d), shfl_up(v.hi, d)}; }
__device__ __forceinline__ Vec shfl_down_vec(Vec v, int d) { return {shfl_down(v.lo, d), shfl_down(v.hi, d)}; }
__device__ __forceinline__ Vec shfl_vec(Vec v, int s) { return {shfl(v.lo, s), shfl(v.hi, s)}; }

// Composite of vectors; with V8 false only entries 0-3 are live (lo).
template <bool V8>
__device__ __forceinline__ Vec comp(Vec a, Vec b)
{
    if constexpr (V8) return compose(a, b);
    else return {perm(b.lo, b.lo, a.lo), a.hi};
}

// entry s of a vector; the absorbing code (and anything >= 8) stays absorbing
__device__ __forceinline__ uint32_t vat(Vec v, uint32_t s)
{
    if (s >= 8u) return kAbs;
    const uint32_t w = s < 4 ? v.lo : v.hi;
    return (w >> ((s & 3u) * 8u)) & 0xffu;
}

// 8 entries -> 8 nibbles (0xff <-> 0xf; live entries are < 8)
__device__ __forceinline__ uint32_t vpack(Vec v) { return vec_pack(v); }
__device__ __forceinline__ Vec vunpack(uint32_t p)
{
    Vec v = vec_unpack(p);
    // nibble 0xf (absorbing) back to 0xff: bytes with bits 0-3 all set
    const uint32_t flo = v.lo & (v.lo >> 1) & (v.lo >> 2) & (v.lo >> 3) & 0x01010101u;
    const uint32_t fhi = v.hi & (v.hi >> 1) & (v.hi >> 2) & (v.hi >> 3) & 0x01010101u;
    v.lo |= flo * 0xf0u;
    v.hi |= fhi * 0xf0u;
    return v;
}

struct LookCtx {
    WsHeader* hdr;
    uint64_t* statA;
    StatB* statB;
    uint32_t epoch;
};

struct OutArrays {
    uint32_t* rec;
    uint32_t* col;
    uint32_t* off;
    uint32_t* len;
    uint64_t cap;
};

template <bool V8>
struct VecComb {
    __device__ Vec operator()(const Vec& a, const Vec& b) const { return comp<V8>(a, b); }
};
struct CarryComb {
    __device__ Carry operator()(const Carry& a, const Carry& b) const { return carry_op(a, b); }
};

// Publish a tile's carry. The aggregate holds tile-local counts (a tile has at
// most 2^15 bytes): nf | nr << 16, colv | colabs << 31, lt. The inclusive prefix
// holds absolute values (its column offset is always absolute): nf, nr, colv, lt.
// The first INVALID byte does not travel through the scan (see err_min).
__device__ __forceinline__ void publish_agg(StatB& s, const Carry& c, uint32_t epoch)
{
    st_relaxed(&s.agg[0], ew(epoch, c.nf | (c.nr << 16)));
    st_relaxed(&s.agg[1], ew(epoch, c.colv | (c.colabs << 31)));
    st_relaxed(&s.agg[2], ew(epoch, c.lt));
}
__device__ __forceinline__ void publish_incl(StatB& s, const Carry& c, uint32_t epoch)
{
    st_relaxed(&s.incl[0], ew(epoch, c.nf));
    st_relaxed(&s.incl[1], ew(epoch, c.nr));
    st_relaxed(&s.incl[2], ew(epoch, c.colv));
    st_relaxed(&s.incl[3], ew(epoch, c.lt));
}

// one tile's carry status: kFlagIncl / kFlagAgg with the carry, or 0
struct CarryPoll {
    const StatB* statB;
    uint32_t epoch;
    __device__ uint32_t operator()(int64_t u, Carry& out) const
    {
        const StatB& s = statB[u];
        const uint64_t i0 = ld_relaxed(&s.incl[0]), i1 = ld_relaxed(&s.incl[1]), i2 = ld_relaxed(&s.incl[2]),
                       i3 = ld_relaxed(&s.incl[3]);
        if (ew_ok(i0, epoch) && ew_ok(i1, epoch) && ew_ok(i2, epoch) && ew_ok(i3, epoch)) {
            out = {(uint32_t)i0, (uint32_t)i1, (uint32_t)i2, 1u, (uint32_t)i3, kNone};
            return kFlagIncl;
        }
        const uint64_t a0 = ld_relaxed(&s.agg[0]), a1 = ld_relaxed(&s.agg[1]), a2 = ld_relaxed(&s.agg[2]);
        if (ew_ok(a0, epoch) && ew_ok(a1, epoch) && ew_ok(a2, epoch)) {
            const uint32_t x0 = (uint32_t)a0, x1 = (uint32_t)a1;
            out = {x0 & 0xffffu, x0 >> 16, x1 & 0x7fffffffu, x1 >> 31, (uint32_t)a2, kNone};
            return kFlagAgg;
        }
        return 0;
    }
};

// one tile's vector status: the aggregate is the tile's packed vector, the
// inclusive prefix its end state, read back as a constant vector
struct VecPoll {
    const uint64_t* statA;
    uint32_t epoch;
    __device__ uint32_t operator()(int64_t u, Vec& out) const
    {
        const uint64_t w = ld_relaxed(&statA[u]);
        const uint32_t f = status_flag(w, epoch);
        if (f == kFlagAgg) out = vunpack(status_payload(w));
        if (f == kFlagIncl) {
            const uint32_t k = status_payload(w) * 0x01010101u;
            out = {k, k};
        }
        return f;
    }
};

template <int NW>
struct TileShared {
    Vec wvec[NW];
    Carry wcar[NW];
    Vec pvec[NW];
    Carry pcar[NW];
    int first[NW];
    Carry prefix;
    uint32_t state;
    uint32_t last_rec;
};

// Tile start state from the block's vector scan: tile 0 starts in the DFA's
// start state; later tiles look back. Publishes the tile's statuses.
template <int NW, bool V8>
__device__ uint32_t tile_start_state(const LookCtx& c, uint32_t tile, uint32_t start_code, Vec tot, Vec ident,
                                     TileShared<NW>* sh)
{
    const int tid = threadIdx.x;
    if (tile == 0) {
        if (tid == 0) {
            sh->state = start_code;
            st_relaxed(&c.statA[0], status_word(c.epoch, kFlagIncl, vat(tot, start_code)));
        }
    } else {
        if (tid == 0) st_relaxed(&c.statA[tile], status_word(c.epoch, kFlagAgg, vpack(tot)));
        const Vec acc = lookback<NW>(tile, ident, VecPoll{c.statA, c.epoch}, VecComb<V8>{}, sh->pvec, sh->first,
                                     &c.hdr->fault);
        if (tid == 0) {
            const uint32_t s = vat(acc, 0);  // a constant vector: the state after all earlier tiles
            sh->state = s;
            st_relaxed(&c.statA[tile], status_word(c.epoch, kFlagIncl, vat(tot, s)));
        }
    }
    __syncthreads();
    return sh->state;
}

// Everything after the re-simulation: per-thread carries from the terminator
// bitmaps, block scan, count look-back, field emission, and (last tile) the
// unterminated final field and the scalar results.
template <int NW>
__device__ void finish_tile(const LookCtx& c, const OutArrays& o, uint32_t n, uint32_t tile, uint32_t num_tiles,
                            uint64_t T, uint64_t RD, uint32_t err, uint32_t chunk_abs, uint32_t end_state,
                            bool end_accepting, TileShared<NW>* sh)
{
    const int tid = threadIdx.x;
    Carry cr;
    cr.nf = (uint32_t)__popcll(T);
    cr.nr = (uint32_t)__popcll(RD);
    if (RD) {
        const int hi = 63 - __clzll((long long)RD);
        const uint64_t above = hi == 63 ? 0ull : (~0ull << (hi + 1));
        cr.colv = (uint32_t)__popcll((T & ~RD) & above);
        cr.colabs = 1;
    } else {
        cr.colv = (uint32_t)__popcll(T);
        cr.colabs = 0;
    }
    cr.lt = T ? chunk_abs + (uint32_t)(63 - __clzll((long long)T)) + 1u : 0u;
    cr.err = kNone;
    if (err != kNone) atomicMin(&c.hdr->err_min, err);  // rare: only chunks holding an INVALID byte
    Carry cex, ctot;
    block_scan<NW>(cr, carry_identity(), cex, ctot, sh->wcar, CarryComb{});

    if (tile == 0) {
        if (tid == 0) {
            Carry z = carry_identity();
            z.colabs = 1;  // the input starts at column 0 of record 0
            sh->prefix = z;
            publish_incl(c.statB[0], carry_op(z, ctot), c.epoch);
        }
    } else {
        if (tid == 0) publish_agg(c.statB[tile], ctot, c.epoch);
        const Carry pre = lookback<NW>(tile, carry_identity(), CarryPoll{c.statB, c.epoch}, CarryComb{}, sh->pcar,
                                       sh->first, &c.hdr->fault);
        if (tid == 0) {
            sh->prefix = pre;
            publish_incl(c.statB[tile], carry_op(pre, ctot), c.epoch);
        }
    }
    __syncthreads();
    const Carry P = sh->prefix;

    {
        const Carry base = carry_op(P, cex);
        uint64_t fi = base.nf;
        uint32_t rec = base.nr, col = base.colv, off = base.lt;
        uint64_t bits = T;
        while (bits) {
            const uint32_t j = (uint32_t)__ffsll((unsigned long long)bits) - 1u;
            const uint32_t pos = chunk_abs + j;
            if (fi < o.cap) {
                o.rec[fi] = rec;
                o.col[fi] = col;
                o.off[fi] = off;
                o.len[fi] = pos - off;
            }
            ++fi;
            off = pos + 1;
            if ((RD >> j) & 1u) {
                ++rec;
                col = 0;
            } else {
                ++col;
            }
            bits &= bits - 1;
        }
    }

    if (tile == num_tiles - 1 && tid == 0) {
        const Carry I = carry_op(P, ctot);
        const uint32_t final_field = sh->last_rec ? 0u : 1u;
        if (final_field && I.nf < o.cap) {
            o.rec[I.nf] = I.nr;
            o.col[I.nf] = I.colv;
            o.off[I.nf] = I.lt;
            o.len[I.nf] = n - I.lt;
        }
        c.hdr->n_fields = (uint64_t)I.nf + final_field;
        c.hdr->n_records = (uint64_t)I.nr + final_field;
        c.hdr->end_state = end_state;
        c.hdr->error_pos = end_accepting ? (int64_t)-1 : (int64_t)n;  // before err_min is applied
    }
}

__global__ void csv_reset_kernel(WsHeader* hdr, uint32_t n, uint32_t start_state, uint32_t accept_mask)
{
    if (threadIdx.x == 0) {
        hdr->tile_counter = 0;
        hdr->fault = 0;
        hdr->err_min = 0xffffffffu;
        if (n == 0) {  // nothing to parse: the results of an empty input
            hdr->n_fields = 0;
            hdr->n_records = 0;
            hdr->end_state = start_state;
            hdr->error_pos = ((accept_mask >> start_state) & 1u) ? -1 : 0;
        }
    }
}

// ================================================================ generic path

struct CsvParams {
    const uint8_t* in;
    uint32_t n, L, tile_bytes, num_tiles;
    uint32_t start_state, accept_mask, epoch, reserved;
    OutArrays out;
    LookCtx look;
    uint32_t row_lo[PPR_MAX_CLASSES], row_hi[PPR_MAX_CLASSES];  // next-state vector of each class
    uint8_t nt[PPR_MAX_STATES][PPR_MAX_CLASSES];                // next | tag << 4
    uint8_t cls[256];
};

__global__ void __launch_bounds__(kBlock) csv_generic_kernel(CsvParams p)
{
    __shared__ __align__(16) uint8_t s_bytes[kBlock * kMaxChunk];
    __shared__ uint8_t s_cls[256];
    __shared__ uint8_t s_nt[PPR_MAX_STATES * PPR_MAX_CLASSES];
    __shared__ uint32_t s_rlo[PPR_MAX_CLASSES], s_rhi[PPR_MAX_CLASSES];
    __shared__ uint32_t s_tile;
    __shared__ TileShared<kWaves> sh;

    const int tid = threadIdx.x;
    if (tid == 0) {
        s_tile = blockIdx.x;
        sh.last_rec = 0;
    }
    s_cls[tid] = p.cls[tid];
    if (tid < PPR_MAX_STATES * PPR_MAX_CLASSES) s_nt[tid] = (&p.nt[0][0])[tid];
    if (tid < PPR_MAX_CLASSES) {
        s_rlo[tid] = p.row_lo[tid];
        s_rhi[tid] = p.row_hi[tid];
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t tile_start = tile * p.tile_bytes;
    const uint32_t tile_len = min(p.tile_bytes, p.n - tile_start);

    // stage the tile into LDS
    const uint8_t* src = p.in + tile_start;
    if ((((uintptr_t)src) & 15u) == 0) {
        const uint32_t nvec = tile_len >> 4;
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(s_bytes);
        for (uint32_t i = tid; i < nvec; i += kBlock) d4[i] = s4[i];
        for (uint32_t i = (nvec << 4) + tid; i < tile_len; i += kBlock) s_bytes[i] = src[i];
    } else {
        for (uint32_t i = tid; i < tile_len; i += kBlock) s_bytes[i] = src[i];
    }
    __syncthreads();

    const uint32_t L = p.L;
    const uint32_t pos0 = tid * L;
    const uint32_t my_len = pos0 < tile_len ? min(L, tile_len - pos0) : 0u;
    const uint32_t chunk_abs = tile_start + pos0;

    // pass 1: all instances at once
    Vec v = vec_identity();
    for (uint32_t j = 0; j < my_len; ++j) {
        const uint32_t c = s_cls[s_bytes[pos0 + j]];
        const uint32_t rl = s_rlo[c], rh = s_rhi[c];
        v = {perm(rh, rl, v.lo), perm(rh, rl, v.hi)};
    }
    Vec excl, tot;
    block_scan<kWaves>(v, vec_identity(), excl, tot, sh.wvec, VecComb<true>{});
    const uint32_t tile_state = tile_start_state<kWaves, true>(p.look, tile, p.start_state, tot, vec_identity(), &sh);

    // pass 2: one instance from the known state, tagging every byte
    uint32_t s = vat(excl, tile_state);
    uint64_t FD = 0, RD = 0;
    uint32_t err = kNone;
    for (uint32_t j = 0; j < my_len; ++j) {
        const uint32_t c = s_cls[s_bytes[pos0 + j]];
        const uint32_t e = s_nt[s * PPR_MAX_CLASSES + c];
        const uint32_t t = e >> 4;
        s = e & 15u;
        FD |= (uint64_t)(t == PPR_TAG_FIELD) << j;
        RD |= (uint64_t)(t == PPR_TAG_RECORD) << j;
        if (t == PPR_TAG_INVALID && err == kNone) err = chunk_abs + j;
    }
    if (my_len && chunk_abs + my_len == p.n) sh.last_rec = (uint32_t)((RD >> (my_len - 1)) & 1u);
    const uint32_t end_state = vat(tot, tile_state);
    finish_tile<kWaves>(p.look, p.out, p.n, tile, p.num_tiles, FD | RD, RD, err, chunk_abs, end_state,
                        (p.accept_mask >> end_state) & 1u, &sh);
}

// ================================================================ fast path

// Symbol codes: the catch-all class has code 2^CB - 1; every other class a
// smaller code. States are coded 0..nt-1 (tracked) and kAbs (absorbing).
constexpr int kTabWords = 2 * 256 + 9 * 256;  // largest step tables (pass 1 + pass 2), 32-bit words

struct FastParams {
    const uint8_t* in;
    uint32_t n, tile_bytes, num_tiles;
    uint32_t start_code, accept_codes;  // bit i: tracked code i accepting; bit 8: absorbing state accepting
    uint32_t nt;                        // tracked states
    uint32_t sh1, m1, sh2, m2;          // slot = ((byte >> sh1) & m1) | ((byte >> sh2) & m2), 3 bits
    uint32_t exp_lo, exp_hi;            // the special byte owning each slot (or a byte of another slot)
    uint32_t cls_lo, cls_hi;            // the code of each slot's special byte
    const uint32_t* tabs;               // step tables built for this call (workspace)
    OutArrays out;
    LookCtx look;
    uint8_t state_of[16];               // DFA state of each code (index 8: absorbing)
    uint8_t nxt[9][16];                 // [state code, row nt = absorbing][symbol code] -> next code
    uint8_t tag[9][16];
};

// symbol codes of four bytes: a 3-bit slot from two bit fields of each byte, the
// slot's special byte and code by v_perm, and an exact compare (SWAR zero-byte
// test); bytes that are not special get the catch-all code
template <int CB>
__device__ __forceinline__ uint32_t classify4(uint32_t w, const FastParams& p)
{
    const uint32_t h = ((w >> p.sh1) & p.m1) | ((w >> p.sh2) & p.m2);
    const uint32_t e = perm(p.exp_hi, p.exp_lo, h);
    const uint32_t c = perm(p.cls_hi, p.cls_lo, h);
    const uint32_t d = w ^ e;
    const uint32_t t = (((d & 0x7f7f7f7fu) + 0x7f7f7f7fu) | d) & 0x80808080u;  // 0x80: not a special byte
    const uint32_t x = t >> 7;
    return c | ((x << CB) - x);
}

// Pass-1 table: entry e (the codes of G bytes) -> composite vector from every
// tracked state. Pass-2 table: row r (state code, row nt = absorbing), entry e ->
// terminator bits (8..), record bits (16..), first INVALID byte (24..26, flag 31)
// and end state (0..7). Built once per call by a small kernel.
template <int CB, bool V8>
__global__ void csv_fast_tables_kernel(FastParams p, uint32_t* tabs)
{
    constexpr int G = CB == 2 ? 4 : 2;
    constexpr int E = 1 << (CB * G);
    constexpr uint32_t CM = (1u << CB) - 1u;
    const uint32_t nt = p.nt;
    for (uint32_t e = threadIdx.x; e < (uint32_t)E; e += blockDim.x) {
        uint32_t cg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) cg[g] = (e >> (CB * g)) & CM;
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < (V8 ? 8 : 4); ++i) {
            uint32_t s = (uint32_t)i < nt ? (uint32_t)i : kAbs;
            for (int g = 0; g < G; ++g)
                if (s != kAbs) s = p.nxt[s][cg[g]];
            if (i < 4) lo |= s << (8 * i);
            else hi |= s << (8 * (i - 4));
        }
        tabs[e] = lo;
        if (V8) tabs[E + e] = hi;
        uint32_t* t2 = tabs + (V8 ? 2 : 1) * E;
        for (uint32_t r = 0; r <= nt; ++r) {
            uint32_t s = r, ent = 0;
            for (int g = 0; g < G; ++g) {
                const uint32_t t = p.tag[s][cg[g]];
                const uint32_t ns = p.nxt[s][cg[g]];
                if (t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) ent |= 1u << (8 + g);
                if (t == PPR_TAG_RECORD) ent |= 1u << (16 + g);
                if (t == PPR_TAG_INVALID && !(ent >> 31)) ent |= (1u << 31) | ((uint32_t)g << 24);
                s = ns == kAbs ? nt : ns;
            }
            t2[r * E + e] = ent | (s == nt ? kAbs : s);
        }
    }
}

template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock) csv_fast_kernel(FastParams p)
{
    constexpr int G = CB == 2 ? 4 : 2;        // bytes per table lookup
    constexpr int E = 1 << (CB * G);          // table entries per state
    constexpr uint32_t CM = (1u << CB) - 1u;
    constexpr int NW = kFastChunk / 4;        // dwords per chunk
    constexpr int NI = kFastChunk / G;        // lookups per chunk
    constexpr uint32_t GM = (1u << G) - 1u;
    constexpr int T1W = V8 ? 2 * E : E;
    __shared__ uint32_t s_tab[T1W + 9 * E];
    __shared__ uint8_t s_nxt[9 * 16], s_tag[9 * 16];
    __shared__ TileShared<kFastWaves> sh;
    const uint32_t* s_t1 = s_tab;
    const uint32_t* s_t2 = s_tab + T1W;

    const int tid = threadIdx.x;
    const uint32_t tile = blockIdx.x;
    const uint32_t tile_start = tile * p.tile_bytes;
    const uint32_t tile_len = min(p.tile_bytes, p.n - tile_start);
    const uint32_t pos0 = tid * kFastChunk;
    const uint32_t my_len = pos0 < tile_len ? min((uint32_t)kFastChunk, tile_len - pos0) : 0u;
    const uint32_t chunk_abs = tile_start + pos0;
    const bool full = my_len == (uint32_t)kFastChunk;

    // the chunk's bytes first, so the loads overlap the table copy
    uint32_t w[NW];
    if (full) {
        const uint4* src = reinterpret_cast<const uint4*>(p.in + chunk_abs);
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
            const uint4 x = src[q];
            w[4 * q] = x.x;
            w[4 * q + 1] = x.y;
            w[4 * q + 2] = x.z;
            w[4 * q + 3] = x.w;
        }
    }
    const uint32_t nt = p.nt;
    const int tab_words = T1W + (int)(nt + 1) * E;
    for (int i = tid; i < tab_words; i += kFastBlock) s_tab[i] = p.tabs[i];
    if (tid < 9 * 16) {
        s_nxt[tid] = (&p.nxt[0][0])[tid];
        s_tag[tid] = (&p.tag[0][0])[tid];
    }
    if (tid == 0) sh.last_rec = 0;
    __syncthreads();

    Vec ident;
    {
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < 8; ++i) {
            const uint32_t s = (uint32_t)i < nt ? (uint32_t)i : kAbs;
            if (i < 4) lo |= s << (8 * i);
            else hi |= s << (8 * (i - 4));
        }
        ident = {lo, V8 ? hi : 0xffffffffu};
    }

    // pass 1: symbol codes, G bytes per lookup, and the chunk's vector as a tree
    // of composites over independent table reads
    uint32_t idx[NI];
    Vec v = ident;
    if (full) {
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const uint32_t code = classify4<CB>(w[k], p);
            if constexpr (G == 4) {
                idx[k] = __builtin_amdgcn_udot4(code, 0x40100401u, 0u, false);
            } else {
                constexpr uint32_t W = 1u << CB;
                idx[2 * k] = __builtin_amdgcn_udot4(code, 0x00000001u | (W << 8), 0u, false);
                idx[2 * k + 1] = __builtin_amdgcn_udot4(code, 0x00010000u | (W << 24), 0u, false);
            }
        }
        uint32_t tl[NI], th[NI];
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            tl[k] = s_t1[idx[k]];
            if (V8) th[k] = s_t1[E + idx[k]];
        }
#pragma unroll
        for (int width = NI; width > 1; width >>= 1) {
#pragma unroll
            for (int i = 0; i < width / 2; ++i) {
                // composite of group 2i then group 2i+1
                if constexpr (V8) {
                    const uint32_t l = perm(th[2 * i + 1], tl[2 * i + 1], tl[2 * i]);
                    const uint32_t h = perm(th[2 * i + 1], tl[2 * i + 1], th[2 * i]);
                    tl[i] = l;
                    th[i] = h;
                } else {
                    tl[i] = perm(tl[2 * i + 1], tl[2 * i + 1], tl[2 * i]);
                }
            }
        }
        v = {tl[0], V8 ? th[0] : 0xffffffffu};
    } else if (my_len) {
        // the input's ragged last chunk: one byte at a time
        for (uint32_t j = 0; j < my_len; ++j) {
            const uint32_t b = p.in[chunk_abs + j];
            const uint32_t code = classify4<CB>(b * 0x01010101u, p) & CM;
            uint32_t lo = 0, hi = 0;
            for (int i = 0; i < 8; ++i) {
                uint32_t s = vat(v, (uint32_t)i);
                if (s != kAbs) s = s_nxt[s * 16 + code];
                if (i < 4) lo |= s << (8 * i);
                else hi |= s << (8 * (i - 4));
            }
            v = {lo, V8 ? hi : 0xffffffffu};
        }
    }
    Vec excl, tot;
    block_scan<kFastWaves>(v, ident, excl, tot, sh.wvec, VecComb<V8>{});
    const uint32_t tile_state = tile_start_state<kFastWaves, V8>(p.look, tile, p.start_code, tot, ident, &sh);

    // pass 2: the state before each group follows from the pass-1 table (one
    // v_perm per group), then the tag lookups are independent
    uint32_t s = vat(excl, tile_state);
    uint64_t T = 0, RD = 0;
    uint32_t err = kNone;
    if (full) {
        uint32_t st[NI];
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            st[k] = s;
            const uint32_t tl = s_t1[idx[k]];
            const uint32_t th = V8 ? s_t1[E + idx[k]] : tl;
            s = perm(th, tl, s) & 0xffu;
        }
        uint32_t any = 0;
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const uint32_t e = s_t2[min(st[k], nt) * E + idx[k]];
            T |= (uint64_t)((e >> 8) & GM) << (G * k);
            RD |= (uint64_t)((e >> 16) & GM) << (G * k);
            any |= e;
        }
        if (any >> 31) {  // some byte is INVALID: find the first one
            for (int k = 0; k < NI; ++k) {
                const uint32_t e = s_t2[min(st[k], nt) * E + idx[k]];
                if (e >> 31) {
                    err = chunk_abs + (uint32_t)(G * k) + ((e >> 24) & 7u);
                    break;
                }
            }
        }
    } else if (my_len) {
        for (uint32_t j = 0; j < my_len; ++j) {
            const uint32_t b = p.in[chunk_abs + j];
            const uint32_t code = classify4<CB>(b * 0x01010101u, p) & CM;
            const uint32_t row = min(s, nt);
            const uint32_t t = s_tag[row * 16 + code];
            s = s_nxt[row * 16 + code];
            T |= (uint64_t)(t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) << j;
            RD |= (uint64_t)(t == PPR_TAG_RECORD) << j;
            if (t == PPR_TAG_INVALID && err == kNone) err = chunk_abs + j;
        }
    }
    if (my_len && chunk_abs + my_len == p.n) sh.last_rec = (uint32_t)((RD >> (my_len - 1)) & 1u);
    const uint32_t end_code = vat(tot, tile_state);
    const uint32_t end_state = p.state_of[min(end_code, 8u)];
    const bool end_ok = (p.accept_codes >> min(end_code, 8u)) & 1u;
    finish_tile<kFastWaves>(p.look, p.out, p.n, tile, p.num_tiles, T, RD, err, chunk_abs, end_state, end_ok, &sh);
}

// ---------------------------------------------------------------- host side

static int validate_dfa(const ppr_dfa_t* d, const uint8_t* cm)
{
    if (!d || !cm) return PPR_EINVAL;
    if (d->n_states < 1 || d->n_states > PPR_MAX_STATES) return PPR_EINVAL;
    if (d->n_classes < 1 || d->n_classes > PPR_MAX_CLASSES) return PPR_EINVAL;
    if (d->start_state >= d->n_states) return PPR_EINVAL;
    for (uint32_t s = 0; s < d->n_states; ++s)
        for (uint32_t c = 0; c < d->n_classes; ++c)
            if (d->next[s][c] >= d->n_states || d->tag[s][c] > PPR_TAG_INVALID) return PPR_EINVAL;
    for (int b = 0; b < 256; ++b)
        if (cm[b] >= d->n_classes) return PPR_EINVAL;
    return PPR_OK;
}

static uint32_t chunk_of(const ppr_parse_opts_t* o)
{
    uint32_t L = o ? o->chunk_bytes : 0u;
    if (L == 0) L = kFastChunk;
    return L <= (uint32_t)kMaxChunk ? L : 0u;
}

// header (256 B), step tables of the fast path, then the two status arrays
static WsLayout csv_layout(uint64_t n, uint32_t L)
{
    const uint64_t tile = (uint64_t)kBlock * L;
    const uint64_t tiles = (n + tile - 1) / tile;
    WsLayout w;
    w.tiles = tiles;
    w.off_a = 256 + kTabWords * 4;
    w.off_b = align_up(w.off_a + tiles * sizeof(uint64_t), 256);
    w.total = align_up(w.off_b + tiles * sizeof(StatB), 256);
    return w;
}

// Fast-path eligibility and its tables: a catch-all class, at most 8 other
// bytes separable by a 3-bit slot (byte >> shift) & 7, at most 8 tracked states.
static bool prepare_fast(const ppr_dfa_t* d, const uint8_t* cm, FastParams& f, int& cb, bool& v8)
{
    uint32_t count[PPR_MAX_CLASSES] = {0};
    for (int b = 0; b < 256; ++b) count[cm[b]]++;
    uint32_t K = 0;
    for (uint32_t c = 1; c < d->n_classes; ++c)
        if (count[c] > count[K]) K = c;
    uint8_t specials[256];
    int ns = 0;
    for (int b = 0; b < 256; ++b)
        if (cm[b] != K) specials[ns++] = (uint8_t)b;
    if (ns > 8) return false;
    // slot = ((b >> sh1) & m1) | ((b >> sh2) & m2): two bit fields, 3 bits in all
    int best_sh1 = -1, best_sh2 = 0;
    uint32_t best_m1 = 0;
    for (int m1 = 7; m1 >= 1 && best_sh1 < 0; --m1) {
        const uint32_t m2 = 7u & ~(uint32_t)m1;
        for (int sh1 = 0; sh1 <= 5 && best_sh1 < 0; ++sh1) {
            for (int sh2 = 0; sh2 <= 7 && best_sh1 < 0; ++sh2) {
                if (m2 == 0 && sh2 != 0) continue;
                if ((m2 & 4u) && sh2 > 5) continue;
                if ((m2 & 2u) && sh2 > 6) continue;
                uint32_t used = 0;
                bool ok = true;
                for (int i = 0; i < ns && ok; ++i) {
                    const uint32_t slot = ((specials[i] >> sh1) & m1) | ((specials[i] >> sh2) & m2);
                    if (used & (1u << slot)) ok = false;
                    used |= 1u << slot;
                }
                if (ok) {
                    best_sh1 = sh1;
                    best_sh2 = sh2;
                    best_m1 = (uint32_t)m1;
                }
            }
        }
    }
    if (best_sh1 < 0) return false;
    const uint32_t best_m2 = 7u & ~best_m1;
    auto slot_of = [&](uint32_t b) { return ((b >> best_sh1) & best_m1) | ((b >> best_sh2) & best_m2); };
    cb = d->n_classes <= 4 ? 2 : d->n_classes <= 8 ? 3 : 4;
    const uint32_t catch_code = (1u << cb) - 1u;
    uint8_t code_of[PPR_MAX_CLASSES];
    uint32_t next_code = 0;
    for (uint32_t c = 0; c < d->n_classes; ++c) code_of[c] = c == K ? (uint8_t)catch_code : (uint8_t)next_code++;
    // slot tables
    uint8_t exp[8], cls[8];
    for (int sl = 0; sl < 8; ++sl) {
        // a byte that hashes to another slot never matches this one
        int other = -1;
        for (int b = 0; b < 256 && other < 0; ++b)
            if (slot_of((uint32_t)b) != (uint32_t)sl) other = b;
        exp[sl] = (uint8_t)other;
        cls[sl] = (uint8_t)catch_code;
    }
    for (int i = 0; i < ns; ++i) {
        const uint32_t slot = slot_of(specials[i]);
        exp[slot] = specials[i];
        cls[slot] = code_of[cm[specials[i]]];
    }
    f.sh1 = (uint32_t)best_sh1;
    f.sh2 = (uint32_t)best_sh2;
    f.m1 = best_m1 * 0x01010101u;
    f.m2 = best_m2 * 0x01010101u;
    f.exp_lo = exp[0] | exp[1] << 8 | exp[2] << 16 | (uint32_t)exp[3] << 24;
    f.exp_hi = exp[4] | exp[5] << 8 | exp[6] << 16 | (uint32_t)exp[7] << 24;
    f.cls_lo = cls[0] | cls[1] << 8 | cls[2] << 16 | (uint32_t)cls[3] << 24;
    f.cls_hi = cls[4] | cls[5] << 8 | cls[6] << 16 | (uint32_t)cls[7] << 24;
    // states: one absorbing state (if any) becomes kAbs, the rest are tracked
    int abs_state = -1;
    for (uint32_t s = 0; s < d->n_states && abs_state < 0; ++s) {
        bool a = true;
        for (uint32_t c = 0; c < d->n_classes; ++c) a = a && d->next[s][c] == s;
        if (a) abs_state = (int)s;
    }
    uint8_t code_of_state[PPR_MAX_STATES];
    uint32_t nt = 0;
    memset(f.state_of, 0, sizeof f.state_of);
    for (uint32_t s = 0; s < d->n_states; ++s) {
        if ((int)s == abs_state) {
            code_of_state[s] = (uint8_t)kAbs;
            f.state_of[8] = (uint8_t)s;
        } else {
            code_of_state[s] = (uint8_t)nt;
            f.state_of[nt] = (uint8_t)s;
            ++nt;
        }
    }
    v8 = nt > 4;
    f.nt = nt;
    f.start_code = code_of_state[d->start_state];
    f.accept_codes = 0;
    for (uint32_t s = 0; s < d->n_states; ++s)
        if ((d->accept_mask >> s) & 1u) f.accept_codes |= 1u << (code_of_state[s] == kAbs ? 8u : code_of_state[s]);
    memset(f.nxt, kAbs, sizeof f.nxt);
    memset(f.tag, PPR_TAG_INVALID, sizeof f.tag);
    for (uint32_t s = 0; s < d->n_states; ++s) {
        const uint32_t row = code_of_state[s] == kAbs ? nt : code_of_state[s];
        for (uint32_t c = 0; c < d->n_classes; ++c) {
            f.nxt[row][code_of[c]] = code_of_state[d->next[s][c]];
            f.tag[row][code_of[c]] = d->tag[s][c];
        }
    }
    return true;
}

template <int CB, bool V8>
static void launch_fast(const FastParams& f, hipStream_t s)
{
    hipLaunchKernelGGL((csv_fast_tables_kernel<CB, V8>), dim3(1), dim3(256), 0, s, f, const_cast<uint32_t*>(f.tabs));
    hipLaunchKernelGGL((csv_fast_kernel<CB, V8>), dim3(f.num_tiles), dim3(kFastBlock), 0, s, f);
}

}  // namespace ppr

using namespace ppr;

extern "C" size_t ppr_parse_workspace_bytes(uint64_t n, const ppr_parse_opts_t* opts)
{
    const uint32_t L = chunk_of(opts);
    if (!L || n >= 0xffffffffull) return 0;
    return (size_t)csv_layout(n, L).total;
}

extern "C" int ppr_parse_async(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                               const ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts,
                               void* stream)
{
    int rc = validate_dfa(dfa, class_map);
    if (rc) return rc;
    if (!out || !d_ws || (n && !d_bytes)) return PPR_EINVAL;
    if (n >= 0xffffffffull) return PPR_ETOOBIG;
    const uint32_t L = chunk_of(opts);
    if (!L) return PPR_EINVAL;
    if (out->cap_fields && (!out->record_idx || !out->column_ids || !out->field_offsets || !out->field_lengths))
        return PPR_EINVAL;
    const WsLayout lay = csv_layout(n, L);
    if (ws_bytes < lay.total || ((uintptr_t)d_ws & 255u)) return PPR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    WsHeader* hdr = (WsHeader*)ws;
    const uint32_t accept = dfa->accept_mask & ((1u << dfa->n_states) - 1u);

    hipLaunchKernelGGL(csv_reset_kernel, dim3(1), dim3(64), 0, s, hdr, (uint32_t)n, dfa->start_state, accept);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    if (n == 0) return PPR_OK;

    OutArrays oa{out->record_idx, out->column_ids, out->field_offsets, out->field_lengths, out->cap_fields};
    LookCtx lc{hdr, (uint64_t*)(ws + lay.off_a), (StatB*)(ws + lay.off_b), next_epoch()};

    // fast path: 64-byte chunks, 16-byte aligned input, a table it can encode
    if (L == (uint32_t)kFastChunk && ((uintptr_t)d_bytes & 15u) == 0) {
        FastParams f;
        memset(&f, 0, sizeof f);
        int cb = 0;
        bool v8 = false;
        if (prepare_fast(dfa, class_map, f, cb, v8)) {
            f.in = d_bytes;
            f.n = (uint32_t)n;
            f.tile_bytes = kFastBlock * kFastChunk;
            f.num_tiles = (uint32_t)((n + f.tile_bytes - 1) / f.tile_bytes);
            f.out = oa;
            f.look = lc;
            f.tabs = (const uint32_t*)(ws + 256);
            if (cb == 2) v8 ? launch_fast<2, true>(f, s) : launch_fast<2, false>(f, s);
            else if (cb == 3) v8 ? launch_fast<3, true>(f, s) : launch_fast<3, false>(f, s);
            else v8 ? launch_fast<4, true>(f, s) : launch_fast<4, false>(f, s);
            return hipGetLastError() == hipSuccess ? PPR_OK : PPR_EHIP;
        }
    }

    CsvParams p;
    memset(&p, 0, sizeof p);
    p.in = d_bytes;
    p.n = (uint32_t)n;
    p.L = L;
    p.tile_bytes = kBlock * L;
    p.num_tiles = (uint32_t)lay.tiles;
    p.start_state = dfa->start_state;
    p.accept_mask = accept;
    p.out = oa;
    p.look = lc;
    for (uint32_t c = 0; c < PPR_MAX_CLASSES; ++c) {
        uint32_t lo = 0, hi = 0;
        for (uint32_t st = 0; st < PPR_MAX_STATES; ++st) {
            const uint32_t nx = (st < dfa->n_states && c < dfa->n_classes) ? dfa->next[st][c] : st;
            if (st < 4) lo |= nx << (8 * st); else hi |= nx << (8 * (st - 4));
        }
        p.row_lo[c] = lo;
        p.row_hi[c] = hi;
    }
    for (uint32_t st = 0; st < PPR_MAX_STATES; ++st)
        for (uint32_t c = 0; c < PPR_MAX_CLASSES; ++c)
            p.nt[st][c] = (st < dfa->n_states && c < dfa->n_classes)
                              ? (uint8_t)(dfa->next[st][c] | (dfa->tag[st][c] << 4))
                              : (uint8_t)st;
    memcpy(p.cls, class_map, 256);
    hipLaunchKernelGGL(csv_generic_kernel, dim3(p.num_tiles), dim3(kBlock), 0, s, p);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    return PPR_OK;
}

extern "C" int ppr_parse_results(const void* d_ws, uint64_t n, ppr_parse_out_t* out, void* stream)
{
    (void)n;
    if (!d_ws || !out) return PPR_EINVAL;
    WsHeader h;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(&h, d_ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    out->n_fields = h.n_fields;
    out->n_records = h.n_records;
    // the first INVALID byte wins over a non-accepting end state
    out->error_pos = h.err_min != 0xffffffffu ? (int64_t)h.err_min : h.error_pos;
    out->end_state = h.end_state;
    if (h.fault) return PPR_EHIP;
    return out->n_fields > out->cap_fields ? PPR_ECAPACITY : PPR_OK;
}

extern "C" int ppr_parse(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                         ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream)
{
    int rc = ppr_parse_async(d_bytes, n, dfa, class_map, out, d_ws, ws_bytes, opts, stream);
    if (rc) return rc;
    return ppr_parse_results(d_ws, n, out, stream);
}
