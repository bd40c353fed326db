// Multi-kernel streaming DFA parse of delimiter-separated bytes on gfx950.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", Sec. 3 (the same steps as the single-pass generic kernel): per-chunk
// state-transition vectors from a multi-DFA simulation (Fig. 2), an exclusive
// scan of their composites for the chunk start states, re-simulation and
// tagging, record counts and relative/absolute column offsets (Fig. 4), field
// emission.
//
// MI355X mapping. The device-wide scans run over tile aggregates in one-
// workgroup kernels between streaming kernels, so no workgroup ever waits on
// another (a decoupled look-back serialises tiles behind the slowest recent
// predecessor's loads):
//   codes   load each 64-byte chunk once (16-byte loads), give every byte its
//           symbol code (SWAR hash + exact compare, as ParPaRaw matches symbols
//           with SWAR, Table 2), store one table index per group of G bytes
//           (1/4 or 1/2 byte per input byte), and reduce the tile's chunk
//           vectors (G bytes per LDS table lookup, a tree of v_perm composites);
//   states  one workgroup: exclusive scan of the tile vectors -> tile start states;
//   carries re-derive each chunk's start state from the stored indices, tag its
//           bytes (pass-2 table: terminator/record bits of G bytes per lookup),
//           store the chunk's start state, reduce the tile's count carry;
//   prefix  one workgroup: exclusive scan of the tile carries, the unterminated
//           final field, the result counts;
//   emit    re-tag from the chunk start state and write every field's record,
//           column, offset and length.
// An absorbing state (such as INV) is the byte 0xFF in a vector, which v_perm
// maps to itself, so it needs no vector entry.
#include <algorithm>

#include "ppr_csv_common.h"
#include "ppr_scan.h"

namespace ppr {

template <int CB>
struct Geo {
    static constexpr int G = CB == 2 ? 4 : 2;       // bytes per table lookup
    static constexpr int E = 1 << (CB * G);         // table entries per state
    static constexpr uint32_t CM = (1u << CB) - 1u;
    static constexpr int ND = kFastChunk / 4;       // dwords per chunk
    static constexpr int NI = kFastChunk / G;       // groups per chunk (index bytes)
    static constexpr int NP = NI / 4;               // index words per chunk
    static constexpr uint32_t GM = (1u << G) - 1u;
};


// Count carries [ParPaRaw Sec. 3, offsets, Fig. 4] in the fast path's
// encodings. Inside a tile (at most 2^15 bytes): nfr = terminators |
// record delimiters << 16, col = column offset handed on (bit 31: absolute, a
// record delimiter was seen), lt = 1 + position of the last terminator (0:
// none). Across tiles the two counts get a word each.
struct TCarry {
    uint32_t nfr, col, lt;
};
struct GCarry {
    uint32_t nf, nr, col, lt;
};

// x earlier, y later: an absolute later column offset wins, a relative one adds
// (the earlier offset's absolute flag stays in bit 31)
__device__ __forceinline__ uint32_t col_op(uint32_t x, uint32_t y) { return (int32_t)y < 0 ? y : x + y; }

struct TCarryComb {
    __device__ TCarry operator()(const TCarry& x, const TCarry& y) const
    {
        return {x.nfr + y.nfr, col_op(x.col, y.col), max(x.lt, y.lt)};
    }
};
struct GCarryComb {
    __device__ GCarry operator()(const GCarry& x, const GCarry& y) const
    {
        return {x.nf + y.nf, x.nr + y.nr, col_op(x.col, y.col), max(x.lt, y.lt)};
    }
};

// the carry of one chunk from its terminator and record-delimiter bitmaps
__device__ __forceinline__ TCarry chunk_carry(uint64_t T, uint64_t RD, uint32_t chunk_abs)
{
    TCarry c;
    c.nfr = (uint32_t)__popcll(T) | ((uint32_t)__popcll(RD) << 16);
    if (RD) {
        const int hi = 63 - __clzll((long long)RD);
        const uint64_t above = hi == 63 ? 0ull : (~0ull << (hi + 1));
        c.col = (uint32_t)__popcll(T & above) | 0x80000000u;
    } else {
        c.col = (uint32_t)__popcll(T);
    }
    c.lt = T ? chunk_abs + (uint32_t)(63 - __clzll((long long)T)) + 1u : 0u;
    return c;
}

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

// identity vector over the tracked state codes; the rest is absorbing
template <bool V8>
__device__ __forceinline__ Vec fast_ident(uint32_t nt)
{
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t s = (uint32_t)i < nt ? (uint32_t)i : kAbs;
        if (i < 4) lo |= s << (8 * i);
        else hi |= s << (8 * (i - 4));
    }
    return {lo, V8 ? hi : 0xffffffffu};
}

// chunk geometry inside a tile
struct ChunkPos {
    uint32_t tile, tile_start, tile_len, chunk_abs, my_len;
    bool full;
};

__device__ __forceinline__ ChunkPos chunk_pos(uint32_t n, uint32_t tile)
{
    ChunkPos c;
    c.tile = tile;
    c.tile_start = c.tile * (uint32_t)kFastTile;
    c.tile_len = min((uint32_t)kFastTile, n - c.tile_start);
    const uint32_t pos0 = threadIdx.x * (uint32_t)kFastChunk;
    c.my_len = pos0 < c.tile_len ? min((uint32_t)kFastChunk, c.tile_len - pos0) : 0u;
    c.chunk_abs = c.tile_start + pos0;
    c.full = c.my_len == (uint32_t)kFastChunk;
    return c;
}

// the chunk's vector from its group indices: independent table reads, then a
// tree of composites (group 2i before group 2i+1)
template <int CB, bool V8>
__device__ __forceinline__ Vec tree_vector(const uint32_t (&idx)[Geo<CB>::NI], const uint32_t* s_t1)
{
    constexpr int E = Geo<CB>::E, NI = Geo<CB>::NI;
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
    return {tl[0], V8 ? th[0] : 0xffffffffu};
}

// the input's ragged last chunk, one byte at a time: its vector
template <int CB, bool V8>
__device__ Vec ragged_vector(const FastParams& p, const ChunkPos& c, Vec v, const uint8_t* s_nxt)
{
    for (uint32_t j = 0; j < c.my_len; ++j) {
        const uint32_t code = classify4<CB>(p.in[c.chunk_abs + j] * 0x01010101u, p) & Geo<CB>::CM;
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < 8; ++i) {
            uint32_t s = vat(v, (uint32_t)i);
            if (s != kAbs) s = s_nxt[s * 16 + code];
            if (i < 4) lo |= s << (8 * i);
            else hi |= s << (8 * (i - 4));
        }
        v = {lo, V8 ? hi : 0xffffffffu};
    }
    return v;
}

// Pass-2 table entry: bits 0-15 the byte offset of the next state's row,
// 16..16+G-1 terminator bits, 20..20+G-1 record-delimiter bits, 24-26 the
// first INVALID byte of the group, 31 some byte is INVALID.
constexpr uint32_t kRowMask = 0xffffu;

// the 64 bits of each kind from the gathered tag bytes of 8 groups of 4 bytes
// (byte g of w0/w1 = terminator nibble | record nibble << 4 of group g / 4 + g)
__device__ __forceinline__ void nibbles_to_bits(uint32_t w0, uint32_t w1, uint32_t& t32, uint32_t& r32)
{
    const uint32_t m = 0x0f0f0f0fu;
    const uint32_t t0 = (w0 & m) | ((w0 >> 4) & ~m), t1 = (w1 & m) | ((w1 >> 4) & ~m);
    const uint32_t r0 = ((w0 >> 4) & m) | ((w0 >> 8) & ~m), r1 = ((w1 >> 4) & m) | ((w1 >> 8) & ~m);
    t32 = perm(t1, t0, 0x06040200u);
    r32 = perm(r1, r0, 0x06040200u);
}

// Pass 2 over a full chunk from state code s: a chain of pass-2 lookups, one per
// group, each addressed by the previous entry's row offset. Returns the OR of
// the entries (bit 31: some byte is INVALID).
template <int CB>
__device__ __forceinline__ uint32_t pass2_full(const uint32_t (&idx)[Geo<CB>::NI], uint32_t s, uint32_t nt,
                                               const uint32_t* s_t2, uint64_t& T, uint64_t& RD)
{
    constexpr int E = Geo<CB>::E, NI = Geo<CB>::NI, G = Geo<CB>::G;
    constexpr uint32_t GM = Geo<CB>::GM;
    const char* base = reinterpret_cast<const char*>(s_t2);
    uint32_t row = min(s, nt) * (uint32_t)(E * 4);
    uint32_t e[NI], any = 0;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        e[k] = *reinterpret_cast<const uint32_t*>(base + row + idx[k] * 4u);
        row = e[k] & kRowMask;
        any |= e[k];
    }
    if constexpr (G == 4) {
        uint32_t w[NI / 4];
#pragma unroll
        for (int q = 0; q < NI / 4; ++q)
            w[q] = perm(e[4 * q + 1], e[4 * q], 0x0c0c0602u) | perm(e[4 * q + 3], e[4 * q + 2], 0x06020c0cu);
        uint32_t tl, th, rl, rh;
        nibbles_to_bits(w[0], w[1], tl, rl);
        nibbles_to_bits(w[2], w[3], th, rh);
        T = (uint64_t)tl | ((uint64_t)th << 32);
        RD = (uint64_t)rl | ((uint64_t)rh << 32);
    } else {
        uint32_t tw[2] = {0u, 0u}, rw[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            tw[(G * k) / 32] |= ((e[k] >> 16) & GM) << ((G * k) % 32);
            rw[(G * k) / 32] |= ((e[k] >> 20) & GM) << ((G * k) % 32);
        }
        T = (uint64_t)tw[0] | ((uint64_t)tw[1] << 32);
        RD = (uint64_t)rw[0] | ((uint64_t)rw[1] << 32);
    }
    return any;
}

// position of the first INVALID byte of a full chunk known to hold one
template <int CB>
__device__ uint32_t first_invalid(const uint32_t (&idx)[Geo<CB>::NI], uint32_t s, uint32_t nt, const uint32_t* s_t2,
                                  uint32_t chunk_abs)
{
    constexpr int E = Geo<CB>::E, NI = Geo<CB>::NI, G = Geo<CB>::G;
    const char* base = reinterpret_cast<const char*>(s_t2);
    uint32_t row = min(s, nt) * (uint32_t)(E * 4);
    for (int k = 0; k < NI; ++k) {
        const uint32_t e = *reinterpret_cast<const uint32_t*>(base + row + idx[k] * 4u);
        if (e >> 31) return chunk_abs + (uint32_t)(G * k) + ((e >> 24) & 7u);
        row = e & kRowMask;
    }
    return kNone;
}

// pass 2 over the ragged last chunk, one byte at a time
template <int CB>
__device__ void pass2_ragged(const FastParams& p, const ChunkPos& c, uint32_t s, uint32_t nt, const uint8_t* s_nxt,
                             const uint8_t* s_tag, uint64_t& T, uint64_t& RD, uint32_t& err)
{
    T = 0;
    RD = 0;
    for (uint32_t j = 0; j < c.my_len; ++j) {
        const uint32_t code = classify4<CB>(p.in[c.chunk_abs + j] * 0x01010101u, p) & Geo<CB>::CM;
        const uint32_t row = min(s, nt);
        const uint32_t t = s_tag[row * 16 + code];
        s = s_nxt[row * 16 + code];
        T |= (uint64_t)(t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) << j;
        RD |= (uint64_t)(t == PPR_TAG_RECORD) << j;
        if (t == PPR_TAG_INVALID && err == kNone) err = c.chunk_abs + j;
    }
}

// What the carries and emit kernels read per chunk: its group indices (NI
// bytes, 16-byte loads) and its vector of the tile's earlier bytes. Loaded one
// tile ahead of use.
template <int CB, bool V8>
struct IdxIn {
    uint32_t pw[Geo<CB>::NP];
    uint32_t cvlo, cvhi;
};

template <int CB, bool V8>
__device__ __forceinline__ IdxIn<CB, V8> load_in(const FastParams& p, const ChunkPos& c)
{
    constexpr int NI = Geo<CB>::NI, NP = Geo<CB>::NP;
    IdxIn<CB, V8> in;
    const size_t ci = (size_t)c.tile * kFastBlock + threadIdx.x;
    if (c.full) {
        const uint4* src = reinterpret_cast<const uint4*>(p.idx + ci * NI);
#pragma unroll
        for (int q = 0; q < NP / 4; ++q) {
            const uint4 x = src[q];
            in.pw[4 * q] = x.x;
            in.pw[4 * q + 1] = x.y;
            in.pw[4 * q + 2] = x.z;
            in.pw[4 * q + 3] = x.w;
        }
    }
    in.cvlo = p.cvec_lo[ci];
    in.cvhi = V8 ? p.cvec_hi[ci] : 0xffffffffu;
    return in;
}

template <int CB, bool V8>
__device__ __forceinline__ void unpack_idx(const IdxIn<CB, V8>& in, uint32_t (&idx)[Geo<CB>::NI])
{
#pragma unroll
    for (int k = 0; k < Geo<CB>::NI; ++k) idx[k] = (in.pw[k / 4] >> (8 * (k % 4))) & 0xffu;
}

// Pass-1 table: entry e (the codes of G bytes) -> composite vector from every
// tracked state. Pass-2 table: row r (state code, row nt = absorbing), entry e ->
// the next state's row offset, the group's tag bits (see pass2_full). One
// workgroup builds them for the call and resets the workspace header.
template <int CB, bool V8>
__global__ void csv_fast_tables_kernel(FastParams p)
{
    constexpr int G = Geo<CB>::G, E = Geo<CB>::E;
    constexpr uint32_t CM = Geo<CB>::CM;
    __shared__ uint8_t s_nxt[9 * 16], s_tag[9 * 16];
    if (threadIdx.x < 9 * 16) {
        s_nxt[threadIdx.x] = (&p.nxt[0][0])[threadIdx.x];
        s_tag[threadIdx.x] = (&p.tag[0][0])[threadIdx.x];
    }
    if (threadIdx.x == 0) {
        p.hdr->tile_counter = 0;
        p.hdr->fault = 0;
        p.hdr->err_min = kNone;
        p.hdr->last_rec = 0;
        p.hdr->path = PPR_PATH_STREAMING;
    }
    __syncthreads();
    uint32_t* tabs = p.tabs;
    const uint32_t nt = p.nt;
    for (uint32_t e = threadIdx.x; e < (uint32_t)E; e += blockDim.x) {
        uint32_t cg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) cg[g] = (e >> (CB * g)) & CM;
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < (V8 ? 8 : 4); ++i) {
            uint32_t s = (uint32_t)i < nt ? (uint32_t)i : kAbs;
            for (int g = 0; g < G; ++g)
                if (s != kAbs) s = s_nxt[s * 16 + cg[g]];
            if (i < 4) lo |= s << (8 * i);
            else hi |= s << (8 * (i - 4));
        }
        tabs[e] = lo;
        if (V8) tabs[E + e] = hi;
        uint32_t* t2 = tabs + (V8 ? 2 : 1) * E;
        for (uint32_t r = 0; r <= nt; ++r) {
            uint32_t s = r, ent = 0;
            for (int g = 0; g < G; ++g) {
                const uint32_t t = s_tag[s * 16 + cg[g]];
                const uint32_t ns = s_nxt[s * 16 + cg[g]];
                if (t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) ent |= 1u << (16 + g);
                if (t == PPR_TAG_RECORD) ent |= 1u << (20 + g);
                if (t == PPR_TAG_INVALID && !(ent >> 31)) ent |= (1u << 31) | ((uint32_t)g << 24);
                s = ns == kAbs ? nt : ns;
            }
            t2[r * E + e] = ent | (s * (uint32_t)E * 4u);
        }
    }
}

// The streaming kernels run num_ranges workgroups; workgroup b owns the
// contiguous tiles [t0, t1) below and walks them in order, loading the next
// tile's inputs while it works on the current one. Along its range it carries
// the state (carries, emit) and the count carry (emit) from tile to tile, so
// the device-wide scans only run over the num_ranges range aggregates, in each
// workgroup's prologue.
__device__ __forceinline__ void range_of(const FastParams& p, uint32_t b, uint32_t& t0, uint32_t& t1)
{
    t0 = (uint32_t)((uint64_t)b * p.num_tiles / p.num_ranges);
    t1 = (uint32_t)((uint64_t)(b + 1) * p.num_tiles / p.num_ranges);
}

__device__ __forceinline__ Vec unpack_vec(uint64_t x) { return Vec{(uint32_t)x, (uint32_t)(x >> 32)}; }

// composite of the range vectors of ranges 0..b-1 (thread i takes ranges 2i, 2i+1)
template <bool V8>
__device__ Vec ranges_before(const FastParams& p, uint32_t b, const Vec& ident, Vec* s_wave)
{
    // (loads from clamped indices, then word-wise selects)
    const uint32_t i0 = 2 * threadIdx.x, i1 = i0 + 1;
    const Vec a = unpack_vec(p.range_vec[min(i0, kMaxRanges - 1)]);
    const Vec c = unpack_vec(p.range_vec[min(i1, kMaxRanges - 1)]);
    const Vec v = select_t(i0 < b, a, ident);
    return block_reduce<kFastWaves>(select_t(i1 < b, comp<V8>(v, c), v), ident, s_wave, VecComb<V8>{});
}

// count carry of ranges 0..b-1
__device__ GCarry carries_before(const FastParams& p, uint32_t b, GCarry* s_wave)
{
    const uint32_t i0 = 2 * threadIdx.x, i1 = i0 + 1;
    const GCarryComb comb;
    const GCarry zero{0, 0, 0, 0};
    const uint4 x = p.range_carry[min(i0, kMaxRanges - 1)], y = p.range_carry[min(i1, kMaxRanges - 1)];
    const GCarry a = select_t(i0 < b, GCarry{x.x, x.y, x.z, x.w}, zero);
    const GCarry c = select_t(i1 < b, comb(a, GCarry{y.x, y.y, y.z, y.w}), a);
    return block_reduce<kFastWaves>(c, zero, s_wave, comb);
}

// codes: symbol codes -> group indices (stored); each chunk's vector of the
// tile's bytes before it, the tile vectors and the range vector (stored)
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock) csv_codes_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    constexpr int NI = Gm::NI, ND = Gm::ND, NP = Gm::NP;
    constexpr int T1W = V8 ? 2 * Gm::E : Gm::E;
    __shared__ uint32_t s_t1[T1W];
    __shared__ uint8_t s_nxt[9 * 16];
    __shared__ Vec s_wave[2][kFastWaves];

    const int tid = threadIdx.x;
    uint32_t t0, t1;
    range_of(p, blockIdx.x, t0, t1);
    auto load_raw = [&](const ChunkPos& c, uint32_t (&w)[ND]) {
        if (c.full) {
            const uint4* src = reinterpret_cast<const uint4*>(p.in + c.chunk_abs);
#pragma unroll
            for (int q = 0; q < ND / 4; ++q) {
                const uint4 x = src[q];
                w[4 * q] = x.x;
                w[4 * q + 1] = x.y;
                w[4 * q + 2] = x.z;
                w[4 * q + 3] = x.w;
            }
        }
    };
    uint32_t tile = t0;
    ChunkPos c = chunk_pos(p.n, tile);
    uint32_t w[ND];
    load_raw(c, w);
    for (int i = tid; i < T1W; i += kFastBlock) s_t1[i] = p.tabs[i];
    if (tid < 9 * 16) s_nxt[tid] = (&p.nxt[0][0])[tid];
    __syncthreads();
    const Vec ident = fast_ident<V8>(p.nt);
    Vec rv = ident;

    for (uint32_t it = 0;; ++it) {
        const uint32_t next = tile + 1;
        const ChunkPos cn = chunk_pos(p.n, next < t1 ? next : tile);
        uint32_t wn[ND];
        if (next < t1) load_raw(cn, wn);

        Vec v = ident;
        if (c.full) {
            uint32_t idx[NI];
#pragma unroll
            for (int k = 0; k < ND; ++k) {
                const uint32_t code = classify4<CB>(w[k], p);
                if constexpr (Gm::G == 4) {
                    idx[k] = __builtin_amdgcn_udot4(code, 0x40100401u, 0u, false);
                } else {
                    constexpr uint32_t W = 1u << CB;
                    idx[2 * k] = __builtin_amdgcn_udot4(code, 0x00000001u | (W << 8), 0u, false);
                    idx[2 * k + 1] = __builtin_amdgcn_udot4(code, 0x00010000u | (W << 24), 0u, false);
                }
            }
            uint32_t pw[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q)
                pw[q] = idx[4 * q] | (idx[4 * q + 1] << 8) | (idx[4 * q + 2] << 16) | (idx[4 * q + 3] << 24);
            uint4* dst = reinterpret_cast<uint4*>(p.idx + ((size_t)tile * kFastBlock + tid) * NI);
#pragma unroll
            for (int q = 0; q < NP / 4; ++q)
                dst[q] = make_uint4(pw[4 * q], pw[4 * q + 1], pw[4 * q + 2], pw[4 * q + 3]);
            v = tree_vector<CB, V8>(idx, s_t1);
        } else if (c.my_len) {
            v = ragged_vector<CB, V8>(p, c, v, s_nxt);
        }
        Vec excl, tot;
        block_scan<kFastWaves>(v, ident, excl, tot, s_wave[it & 1], VecComb<V8>{});
        const size_t ci = (size_t)tile * kFastBlock + tid;
        p.cvec_lo[ci] = excl.lo;
        if (V8) p.cvec_hi[ci] = excl.hi;
        if (tid == 0) p.tile_vec[tile] = (uint64_t)tot.lo | ((uint64_t)tot.hi << 32);
        rv = comp<V8>(rv, tot);

        if (next >= t1) break;
        tile = next;
        c = cn;
#pragma unroll
        for (int k = 0; k < ND; ++k) w[k] = wn[k];
    }
    if (tid == 0) p.range_vec[blockIdx.x] = (uint64_t)rv.lo | ((uint64_t)rv.hi << 32);
}

// pass-2 table rows (tracked states + the absorbing row) and the byte tables
template <bool V8, int E>
struct Pass2Shared {
    uint32_t t2[(V8 ? 9 : 5) * E];
    uint8_t nxt[9 * 16], tag[9 * 16];
};

template <int CB, bool V8>
__device__ __forceinline__ void load_pass2(const FastParams& p, Pass2Shared<V8, Geo<CB>::E>& sh)
{
    constexpr int E = Geo<CB>::E;
    const uint32_t* t2g = p.tabs + (V8 ? 2 : 1) * E;
    const int words = (int)(p.nt + 1) * E;
    for (int i = threadIdx.x; i < words; i += kFastBlock) sh.t2[i] = t2g[i];
    if (threadIdx.x < 9 * 16) {
        sh.nxt[threadIdx.x] = (&p.nxt[0][0])[threadIdx.x];
        sh.tag[threadIdx.x] = (&p.tag[0][0])[threadIdx.x];
    }
}

// carries: the range's start state (stored), tags from each chunk's start
// state, the range's count carry (stored); the last range stores the end state
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock) csv_carries_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    constexpr int NI = Gm::NI;
    __shared__ Pass2Shared<V8, Gm::E> sh;
    __shared__ TCarry s_wc[2][kFastWaves];
    __shared__ Vec s_wv[kFastWaves];

    const uint32_t b = blockIdx.x;
    uint32_t t0, t1;
    range_of(p, b, t0, t1);
    uint32_t tile = t0;
    ChunkPos c = chunk_pos(p.n, tile);
    IdxIn<CB, V8> in = load_in<CB, V8>(p, c);
    uint64_t tv = p.tile_vec[tile];
    const uint32_t nt = p.nt;
    load_pass2<CB, V8>(p, sh);
    const Vec ident = fast_ident<V8>(nt);
    uint32_t run = vat(ranges_before<V8>(p, b, ident, s_wv), p.start_code);  // (its barrier publishes sh)
    if (threadIdx.x == 0) p.range_state[b] = run;
    const GCarryComb gcomb;
    GCarry rc{0, 0, 0, 0};

    for (uint32_t it = 0;; ++it) {
        const uint32_t next = tile + 1;
        const ChunkPos cn = chunk_pos(p.n, next < t1 ? next : tile);
        IdxIn<CB, V8> inn;
        uint64_t tvn = 0;
        if (next < t1) {
            inn = load_in<CB, V8>(p, cn);
            tvn = p.tile_vec[next];
        }

        const uint32_t s = vat(Vec{in.cvlo, in.cvhi}, run);
        uint64_t T = 0, RD = 0;
        uint32_t err = kNone;
        if (c.full) {
            uint32_t idx[NI];
            unpack_idx<CB, V8>(in, idx);
            if (pass2_full<CB>(idx, s, nt, sh.t2, T, RD) >> 31)
                err = first_invalid<CB>(idx, s, nt, sh.t2, c.chunk_abs);
        } else if (c.my_len) {
            pass2_ragged<CB>(p, c, s, nt, sh.nxt, sh.tag, T, RD, err);
        }
        if (err != kNone) atomicMin(&p.hdr->err_min, err);
        if (c.my_len && c.chunk_abs + c.my_len == p.n) p.hdr->last_rec = (uint32_t)((RD >> (c.my_len - 1)) & 1u);
        const TCarry ct =
            block_reduce<kFastWaves>(chunk_carry(T, RD, c.chunk_abs), TCarry{0, 0, 0}, s_wc[it & 1], TCarryComb{});
        rc = gcomb(rc, GCarry{ct.nfr & 0xffffu, ct.nfr >> 16, ct.col, ct.lt});
        run = vat(unpack_vec(tv), run);

        if (next >= t1) break;
        tile = next;
        c = cn;
        in = inn;
        tv = tvn;
    }
    if (threadIdx.x == 0) {
        p.range_carry[b] = make_uint4(rc.nf, rc.nr, rc.col, rc.lt);
        if (b == p.num_ranges - 1) {
            const uint32_t e = min(run, 8u);
            p.hdr->end_state = p.state_of[e];
            p.hdr->error_pos = ((p.accept_codes >> e) & 1u) ? (int64_t)-1 : (int64_t)p.n;  // before err_min
        }
    }
}

// fields staged in LDS per round, so that the four output arrays are written
// with consecutive addresses across the lanes
constexpr int kStage = 2048;

// emit: tags from each chunk's start state; every field's record, column,
// offset and length; the last range writes the unterminated final field and
// the result counts
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock) csv_emit_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    constexpr int NI = Gm::NI;
    __shared__ Pass2Shared<V8, Gm::E> sh;
    __shared__ TCarry s_wc[2][kFastWaves];
    __shared__ GCarry s_wg[kFastWaves];
    __shared__ uint32_t s_stage[4][kStage];

    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    uint32_t t0, t1;
    range_of(p, b, t0, t1);
    uint32_t tile = t0;
    ChunkPos c = chunk_pos(p.n, tile);
    IdxIn<CB, V8> in = load_in<CB, V8>(p, c);
    uint64_t tv = p.tile_vec[tile];
    uint32_t run = p.range_state[b];
    const uint32_t nt = p.nt;
    const OutArrays& o = p.out;
    load_pass2<CB, V8>(p, sh);
    const GCarryComb gcomb;
    // the input starts at column 0 of record 0: an absolute zero column offset
    GCarry P = gcomb(GCarry{0u, 0u, 0x80000000u, 0u}, carries_before(p, b, s_wg));  // (its barrier publishes sh)

    for (uint32_t it = 0;; ++it) {
        const uint32_t next = tile + 1;
        const ChunkPos cn = chunk_pos(p.n, next < t1 ? next : tile);
        IdxIn<CB, V8> inn;
        uint64_t tvn = 0;
        if (next < t1) {
            inn = load_in<CB, V8>(p, cn);
            tvn = p.tile_vec[next];
        }

        const uint32_t s = vat(Vec{in.cvlo, in.cvhi}, run);
        uint64_t T = 0, RD = 0;
        if (c.full) {
            uint32_t idx[NI];
            unpack_idx<CB, V8>(in, idx);
            pass2_full<CB>(idx, s, nt, sh.t2, T, RD);
        } else if (c.my_len) {
            uint32_t err = kNone;
            pass2_ragged<CB>(p, c, s, nt, sh.nxt, sh.tag, T, RD, err);
        }
        TCarry cex, ctot;
        block_scan<kFastWaves>(chunk_carry(T, RD, c.chunk_abs), TCarry{0, 0, 0}, cex, ctot, s_wc[it & 1],
                               TCarryComb{});

        const uint32_t first = cex.nfr & 0xffffu, mine = (uint32_t)__popcll(T), tile_nf = ctot.nfr & 0xffffu;
        for (uint32_t r0 = 0; r0 < tile_nf; r0 += kStage) {
            const uint32_t r1 = min(r0 + (uint32_t)kStage, tile_nf);
            if (mine && first < r1 && first + mine > r0) {
                uint32_t li = first, rec = P.nr + (cex.nfr >> 16);
                uint32_t col = col_op(P.col, cex.col) & 0x7fffffffu;
                uint32_t off = max(P.lt, cex.lt);
                uint64_t bits = T;
                while (bits && li < r1) {
                    const uint32_t j = (uint32_t)__ffsll((unsigned long long)bits) - 1u;
                    const uint32_t pos = c.chunk_abs + j;
                    if (li >= r0) {
                        s_stage[0][li - r0] = rec;
                        s_stage[1][li - r0] = col;
                        s_stage[2][li - r0] = off;
                        s_stage[3][li - r0] = pos - off;
                    }
                    ++li;
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
            __syncthreads();
            const uint64_t g0 = (uint64_t)P.nf + r0;
            for (uint32_t i = tid; i < r1 - r0; i += kFastBlock) {
                const uint64_t gi = g0 + i;
                if (gi < o.cap) {
                    o.rec[gi] = s_stage[0][i];
                    o.col[gi] = s_stage[1][i];
                    o.off[gi] = s_stage[2][i];
                    o.len[gi] = s_stage[3][i];
                }
            }
            __syncthreads();
        }
        P = gcomb(P, GCarry{ctot.nfr & 0xffffu, ctot.nfr >> 16, ctot.col, ctot.lt});
        run = vat(unpack_vec(tv), run);

        if (next >= t1) break;
        tile = next;
        c = cn;
        in = inn;
        tv = tvn;
    }
    if (tid == 0 && b == p.num_ranges - 1) {
        const uint32_t final_field = p.hdr->last_rec ? 0u : 1u;
        if (final_field && P.nf < o.cap) {
            o.rec[P.nf] = P.nr;
            o.col[P.nf] = P.col & 0x7fffffffu;
            o.off[P.nf] = P.lt;
            o.len[P.nf] = p.n - P.lt;
        }
        p.hdr->n_fields = (uint64_t)P.nf + final_field;
        p.hdr->n_records = (uint64_t)P.nr + final_field;
    }
}

template <int CB, bool V8>
static void launch(const FastParams& f, const ppr_parse_opts_t* o, hipStream_t s)
{
    const dim3 grid(f.num_ranges), block(kFastBlock);
    stage_event(o, 0, s);
    hipLaunchKernelGGL((csv_fast_tables_kernel<CB, V8>), dim3(1), dim3(256), 0, s, f);
    stage_event(o, 1, s);
    hipLaunchKernelGGL((csv_codes_kernel<CB, V8>), grid, block, 0, s, f);
    stage_event(o, 2, s);
    hipLaunchKernelGGL((csv_carries_kernel<CB, V8>), grid, block, 0, s, f);
    stage_event(o, 3, s);
    hipLaunchKernelGGL((csv_emit_kernel<CB, V8>), grid, block, 0, s, f);
    stage_event(o, 4, s);
}

int launch_csv_fast(const FastParams& f, int cb, bool v8, const ppr_parse_opts_t* o, hipStream_t s)
{
    if (cb == 2) v8 ? launch<2, true>(f, o, s) : launch<2, false>(f, o, s);
    else if (cb == 3) v8 ? launch<3, true>(f, o, s) : launch<3, false>(f, o, s);
    else v8 ? launch<4, true>(f, o, s) : launch<4, false>(f, o, s);
    return hipGetLastError() == hipSuccess ? PPR_OK : PPR_EHIP;
}

}  // namespace ppr
