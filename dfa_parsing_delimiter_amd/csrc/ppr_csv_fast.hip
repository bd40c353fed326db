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
#include <type_traits>

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
    static constexpr int PAR = G == 4 ? 2 : 1;      // pass-2 tables used in turn (one per group parity)
};


// Count carries [ParPaRaw Sec. 3, offsets, Fig. 4] of a run of bytes: nf
// terminators, nr record delimiters, col the column offset handed on, lt = 1 +
// position of the last terminator (0: none). The column offset is absolute
// (field delimiters after the run's last record delimiter) exactly when the
// run holds a record delimiter, nr > 0, and relative (all its field
// delimiters) otherwise, so the relative/absolute flag needs no bit of its
// own and a column offset may take all 32 bits. The input's start is column 0
// of record 0, so a prefix that starts there is absolute either way.
struct GCarry {
    uint32_t nf, nr, col, lt;
};

// column offset after x then y (y later, holding ynr record delimiters): an
// absolute later offset wins, a relative one adds to the earlier offset
__device__ __forceinline__ uint32_t col_after(uint32_t xcol, uint32_t ycol, uint32_t ynr)
{
    return ynr ? ycol : xcol + ycol;
}

struct GCarryComb {
    __device__ GCarry operator()(const GCarry& x, const GCarry& y) const
    {
        return {x.nf + y.nf, x.nr + y.nr, col_after(x.col, y.col, y.nr), max(x.lt, y.lt)};
    }
};

struct AddComb {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MaxComb {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};

// Count carries of a workgroup's spans without a 4-word scan: each lane's
// terminator and record counts (packed, a span holds at most 128 of each), the
// 1 + position of its last terminator, and the 1-based index among its
// terminators of its last record delimiter. Per wave, a sum scan of the packed
// counts gives each lane's exclusive counts; the wave's last terminator and
// last record field are those of its last lane holding one (a ballot and a
// readlane: positions grow with the lane); its column carry is the terminators
// after its last record delimiter. Wave 0 then scans the waves' carries and
// hands each wave its exclusive carry and the total through LDS.
struct SpanCarry {
    uint32_t excl_nf;  // terminators in the wave's earlier lanes
    uint32_t mine;     // this lane's terminators
    GCarry wave_excl;  // carry of the tile's earlier waves
    GCarry total;      // carry of the whole tile
};

constexpr int kSpanScratch = 2 * kFastWaves + 1;  // GCarry entries of span_carry's LDS scratch

// The count carry of a wave's spans (every lane gets it), from each lane's
// bitmaps; excl_nf: the terminators of the wave's earlier lanes, nf: the lane's.
struct WaveCarry {
    GCarry wc;
    uint32_t excl_nf, nf;
};

template <int NCH>
__device__ __forceinline__ WaveCarry wave_carry(const uint64_t (&T)[NCH], const uint64_t (&RD)[NCH], uint32_t abs)
{
    uint32_t nr = 0, lt = 0, rdl = 0, before = 0;
#pragma unroll
    for (int h = 0; h < NCH; ++h) {
        const uint32_t nh = (uint32_t)__popcll(T[h]);
        nr += (uint32_t)__popcll(RD[h]);
        if (T[h]) lt = abs + (uint32_t)(kFastChunk * h) + (uint32_t)(63 - __clzll((long long)T[h])) + 1u;
        if (RD[h]) {
            const int hb = 63 - __clzll((long long)RD[h]);
            rdl = before + (uint32_t)__popcll(T[h] & (hb == 63 ? ~0ull : ((2ull << hb) - 1ull)));
        }
        before += nh;
    }
    const uint32_t nf = before;
    const uint32_t inc = wave_scan(nf | (nr << 16), 0u, AddComb{});
    const uint32_t excl = wave_shr1(0u, inc);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane(inc, kWave - 1);
    const uint64_t has_t = __ballot(nf != 0), has_r = __ballot(rdl != 0);
    const uint32_t max_lt = has_t ? (uint32_t)__builtin_amdgcn_readlane(lt, 63 - __clzll((long long)has_t)) : 0u;
    // 1-based wave-local index of the wave's last record field
    const uint32_t max_rd =
        has_r ? (uint32_t)__builtin_amdgcn_readlane((excl & 0xffffu) + rdl, 63 - __clzll((long long)has_r)) : 0u;
    const uint32_t wnf = tot & 0xffffu;
    return WaveCarry{GCarry{wnf, tot >> 16, max_rd ? wnf - max_rd : wnf, max_lt}, excl & 0xffffu, nf};
}

template <int NCH>
__device__ __forceinline__ SpanCarry span_carry(const uint64_t (&T)[NCH], const uint64_t (&RD)[NCH], uint32_t abs,
                                                GCarry* s_wave)
{
    const WaveCarry wcr = wave_carry<NCH>(T, RD, abs);
    const GCarry wc = wcr.wc;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const GCarry zero{0, 0, 0, 0};
    if (lane_id() == 0) s_wave[w] = wc;
    __syncthreads();
    if (w == 0) {  // s_wave[NW + i]: carry of the waves before wave i; s_wave[2 NW]: the total
        const GCarry ws = row_scan<kFastWaves>(lane_value<kFastWaves>(s_wave, zero), zero, GCarryComb{});
        const GCarry ex = wave_shr1(zero, ws);
        if (lane_id() < kFastWaves) s_wave[kFastWaves + lane_id()] = ex;
        if (lane_id() == kFastWaves - 1) s_wave[2 * kFastWaves] = ws;
    }
    __syncthreads();
    SpanCarry r;
    r.excl_nf = wcr.excl_nf;
    r.mine = wcr.nf;
    r.wave_excl = s_wave[kFastWaves + w];
    r.total = s_wave[2 * kFastWaves];
    return r;
}

// v_perm_b32, for the classification shared with the host check (ppr_slots.h)
struct PermOp {
    __device__ uint32_t operator()(uint32_t hi, uint32_t lo, uint32_t sel) const { return perm(hi, lo, sel); }
};

// Symbol codes (times 4) of four bytes (ppr_slots.h): the slot's special byte
// and code by v_perm, and an exact match test by one more v_perm of the
// difference; bytes that are not special get the catch-all code.
template <int CB>
__device__ __forceinline__ uint32_t classify4(uint32_t w, const FastParams& p)
{
    return slot_codes4(w, p.slots, Geo<CB>::CM * 0x04040404u, PermOp{});
}

// symbol code of one byte (the ragged paths)
template <int CB>
__device__ __forceinline__ uint32_t classify1(uint32_t b, const FastParams& p)
{
    return (classify4<CB>(b * 0x01010101u, p) >> 2) & Geo<CB>::CM;
}

// The table addresses (4 x the group index: c0 + 4 c1 + 16 c2 + 64 c3, or
// c0 + 2^CB c1) of a full chunk's groups, and the group indices packed four
// per word (one byte per group).
template <int CB>
__device__ __forceinline__ void chunk_codes(const uint32_t (&w)[Geo<CB>::ND], const FastParams& p,
                                            uint32_t (&ia)[Geo<CB>::NI], uint32_t (&pw)[Geo<CB>::NP])
{
    using Gm = Geo<CB>;
#pragma unroll
    for (int k = 0; k < Gm::ND; ++k) {
        const uint32_t code4 = classify4<CB>(w[k], p);
        if constexpr (Gm::G == 4) {
            ia[k] = __builtin_amdgcn_udot4(code4, 0x40100401u, 0u, false);
        } else {
            constexpr uint32_t W = 1u << CB;
            ia[2 * k] = __builtin_amdgcn_udot4(code4, 0x00000001u | (W << 8), 0u, false);
            ia[2 * k + 1] = __builtin_amdgcn_udot4(code4, 0x00010000u | (W << 24), 0u, false);
        }
    }
#pragma unroll
    for (int q = 0; q < Gm::NP; ++q)
        pw[q] = (ia[4 * q] >> 2) | (ia[4 * q + 1] << 6) | (ia[4 * q + 2] << 14) | (ia[4 * q + 3] << 22);
}

// the value of the even lane of this lane's pair (DPP quad_perm [0,0,2,2])
__device__ __forceinline__ uint32_t even_lane(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xa0, 0xf, 0xf, false);
}

// Whether every live hypothesis of a prefix vector has reached one state: each
// entry is either that state x or absorbing (kAbs). x = kAbs when every entry
// is. Once a prefix agrees, every longer one does (the live hypotheses then
// move together), so the agreed chunks of a tile are a suffix of it.
template <bool V8>
__device__ __forceinline__ bool vec_agreed(const Vec& v, uint32_t& x)
{
    uint32_t m = kAbs;
#pragma unroll
    for (int i = 0; i < (V8 ? 8 : 4); ++i) m = min(m, ((i < 4 ? v.lo : v.hi) >> (8 * (i & 3))) & 0xffu);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < (V8 ? 8 : 4); ++i) {
        const uint32_t e = ((i < 4 ? v.lo : v.hi) >> (8 * (i & 3))) & 0xffu;
        ok = ok && (e == m || e == kAbs);
    }
    x = m;
    return ok;
}

// Speculation (not a step of the pages' method, but built on its
// state-transition vectors, ParPaRaw Sec. 3, parsing context; the outputs are
// the plain method's): a chunk whose tile-exclusive vector agrees starts in the
// agreed state whatever state the tile starts in,
// unless the true path has died (reached the absorbing state) before it. The
// codes kernel counts the fields of a tile's agreed chunks when the tile's own
// vector agrees on a tracked state and it is not the input's last tile; the
// carries kernel uses that count when the tile's true start state reaches
// that same state at the tile's end (the true path is then alive at every
// agreed chunk, so their starts are the agreed states), and otherwise runs
// pass 2 over the whole tile.
template <bool V8>
__device__ __forceinline__ bool tile_speculates(const FastParams& p, uint32_t tile, const Vec& tv, uint32_t& x)
{
    return tile + 1u < p.num_tiles && vec_agreed<V8>(tv, x) && x != kAbs;
}

// What a span's index slot holds (speculating configurations). The codes
// kernel stores the tag bitmaps of an agreed chunk (terminators, then record
// delimiters, 8 bytes each: the 16 bytes its indices take) in place of its
// indices, when its tile speculates and the absorbing state tags no byte as a
// terminator. Readers take them when the tile's speculation holds (mode 1),
// nothing when it does not (mode 2: the true path has died, so those chunks are
// in the absorbing state and end no field), and run pass 2 on the indices of
// every other span (mode 0).
template <bool V8>
__device__ __forceinline__ bool tile_bits(const FastParams& p, uint32_t tile, const Vec& tv, uint32_t& x)
{
    return p.quiet_abs && tile < p.num_tiles && tile_speculates<V8>(p, tile, tv, x);
}

template <int CB, bool V8>
__device__ __forceinline__ int span_mode(bool bits, bool holds, uint32_t cvlo, uint32_t cvhi);

// words of a tile's speculative carry (p.spec, 8 per tile)
// (nf, nr, col, lt; then the first INVALID byte of the agreed chunks)
constexpr uint32_t kSpWords = 8;

// Speculation runs for 4-byte groups and at most 4 tracked states (one VGPR
// per vector); the other geometries need more registers in the codes kernel
// than it can spare.
template <int CB, bool V8>
constexpr bool kSpeculates = CB == 2 && !V8;

template <int CB, bool V8>
__device__ __forceinline__ int span_mode(bool bits, bool holds, uint32_t cvlo, uint32_t cvhi)
{
    if constexpr (!kSpeculates<CB, V8>) {
        return 0;
    } else {
        uint32_t x;
        if (!bits || !vec_agreed<V8>(Vec{cvlo, cvhi}, x)) return 0;
        return holds ? 1 : 2;
    }
}

// A span vector that no prefix has (its entries are neither tracked states
// nor absorbing): the carries kernel puts it in place of the vector of a span
// whose slot it has filled with the span's tag bitmaps. It agrees (every entry
// the same), so the emit kernel reads that slot as bitmaps (mode 1).
constexpr uint32_t kBitsMark = 0xfefefefeu;

// the tag bitmaps of a span's two chunks from its slot (mode 1)
__device__ __forceinline__ void slot_bits(const uint32_t* pw, uint64_t (&T)[2], uint64_t (&RD)[2])
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        T[h] = (uint64_t)pw[4 * h] | ((uint64_t)pw[4 * h + 1] << 32);
        RD[h] = (uint64_t)pw[4 * h + 2] | ((uint64_t)pw[4 * h + 3] << 32);
    }
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

// the chunk's vector from its table addresses: independent table reads, then
// a tree of composites (group 2i before group 2i+1)
template <int CB, bool V8>
__device__ __forceinline__ Vec tree_vector(const uint32_t (&ia)[Geo<CB>::NI], const uint32_t* s_t1)
{
    constexpr int E = Geo<CB>::E, NI = Geo<CB>::NI;
    uint32_t tl[NI], th[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
        tl[k] = lds_at(s_t1, ia[k]);
        if (V8) th[k] = lds_at(s_t1 + E, ia[k]);
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
        const uint32_t code = classify1<CB>(p.in[c.chunk_abs + j], p);
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

// Pass-2 table: one row of kRowStride entries per state code (row nt: the
// absorbing state), entry e = the table index of a group of G symbols. Entry
// bits 0-2 hold the first INVALID byte of the group, bit 7 is set if some byte
// is INVALID, bits 8-15 hold the row of the next lookup. With the row in byte
// 1, the next lookup's word index (row << 8 | index byte) is one v_perm of the
// previous entry and the packed index word.
//
// G = 2: one table; bits 16..17 are the terminator bits, 20..21 the
// record-delimiter bits (bit g: byte g of the group).
//
// G = 4: two tables, used by the even and the odd groups of a chunk in turn
// (an even group's entry names a row of the odd table, rows nt+1 .. 2nt+1, and
// the reverse). The even table holds the terminator nibble in bits 16-19 and
// the record-delimiter nibble in 24-27, the odd table in bits 20-23 and 28-31,
// so the OR of a pair's two entries holds the pair's 8 terminator bits in byte
// 2 and its 8 record-delimiter bits in byte 3: one v_perm of two pairs then
// gives the bitmaps of 16 bytes.
constexpr int kRowStride = 256;
constexpr uint32_t kP2Invalid = 0x80u;

// word index of the lookup for index byte i of idxw after entry prev
__device__ __forceinline__ uint32_t p2_index(uint32_t prev, uint32_t idxw, int i)
{
    return perm(prev, idxw, 0x0c0c0500u | (uint32_t)i);
}

// Pass 2 over NCH consecutive full chunks of a thread (NCH NI groups, packed
// four index bytes per word in pw) from state code s: a chain of pass-2
// lookups, one per group, each addressed by the previous entry (p2_index).
// T[h] / RD[h]: terminator / record bitmaps of chunk h (bit j = byte j).
// Returns the OR of the entries (kP2Invalid: some byte is INVALID). (Cutting the
// chain into independent runs, with start states from the pass-1 table, costs
// more instructions than the shorter LDS wait saves: these kernels are bound by
// instruction issue.)
template <int CB, int NCH>
__device__ __forceinline__ uint32_t pass2_run(const uint32_t (&pw)[NCH * Geo<CB>::NP], uint32_t s, uint32_t nt,
                                              const uint32_t* s_t2, uint64_t (&T)[NCH], uint64_t (&RD)[NCH])
{
    constexpr int NG = NCH * Geo<CB>::NI, G = Geo<CB>::G;
    constexpr uint32_t GM = Geo<CB>::GM;
    uint32_t prev = min(s, nt) << 8;
    uint32_t any = 0;
    if constexpr (G == 4) {
        // per index word (16 bytes): terminator bits in 0-15, record-delimiter bits in 16-31
        uint32_t w[NG / 4];
#pragma unroll
        for (int q = 0; q < NG / 4; ++q) {
            const uint32_t e0 = s_t2[p2_index(prev, pw[q], 0)];
            const uint32_t e1 = s_t2[p2_index(e0, pw[q], 1)];
            const uint32_t e2 = s_t2[p2_index(e1, pw[q], 2)];
            const uint32_t e3 = s_t2[p2_index(e2, pw[q], 3)];
            prev = e3;
            const uint32_t a = e0 | e1, b = e2 | e3;
            any |= a | b;
            w[q] = perm(b, a, 0x07030602u);
        }
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
            T[h] = (uint64_t)perm(w[4 * h + 1], w[4 * h], 0x05040100u) |
                   ((uint64_t)perm(w[4 * h + 3], w[4 * h + 2], 0x05040100u) << 32);
            RD[h] = (uint64_t)perm(w[4 * h + 1], w[4 * h], 0x07060302u) |
                    ((uint64_t)perm(w[4 * h + 3], w[4 * h + 2], 0x07060302u) << 32);
        }
    } else {
        uint32_t tw[2 * NCH], rw[2 * NCH];
#pragma unroll
        for (int i = 0; i < 2 * NCH; ++i) tw[i] = rw[i] = 0u;
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            const uint32_t e = s_t2[p2_index(prev, pw[k / 4], k % 4)];
            prev = e;
            any |= e;
            tw[(G * k) / 32] |= ((e >> 16) & GM) << ((G * k) % 32);
            rw[(G * k) / 32] |= ((e >> 20) & GM) << ((G * k) % 32);
        }
#pragma unroll
        for (int h = 0; h < NCH; ++h) {
            T[h] = (uint64_t)tw[2 * h] | ((uint64_t)tw[2 * h + 1] << 32);
            RD[h] = (uint64_t)rw[2 * h] | ((uint64_t)rw[2 * h + 1] << 32);
        }
    }
    return any;
}

template <int CB>
__device__ __forceinline__ uint32_t pass2_pair(const uint32_t (&pw)[2 * Geo<CB>::NP], uint32_t s, uint32_t nt,
                                               const uint32_t* s_t2, uint64_t (&T)[2], uint64_t (&RD)[2])
{
    return pass2_run<CB, 2>(pw, s, nt, s_t2, T, RD);
}

// position of the first INVALID byte of NCH full chunks known to hold one
template <int CB, int NCH>
__device__ uint32_t first_invalid(const uint32_t (&pw)[NCH * Geo<CB>::NP], uint32_t s, uint32_t nt,
                                  const uint32_t* s_t2, uint32_t abs)
{
    constexpr int NG = NCH * Geo<CB>::NI, G = Geo<CB>::G;
    // z is 0 (nt <= 8) but not known to the compiler, so these lookups are made
    // again rather than shared with the common path's chain, whose entries
    // would otherwise stay in registers for this rare case
    const uint32_t z = nt >> 16;
    uint32_t prev = min(s, nt) << 8, first = kNone;
#pragma unroll
    for (int k = 0; k < NG; ++k) {  // (no early exit: indices into pw stay compile-time constants)
        const uint32_t e = s_t2[p2_index(prev, pw[k / 4], k % 4) | z];
        if ((e & kP2Invalid) && first == kNone) first = abs + (uint32_t)(G * k) + (e & 7u);
        prev = e;
    }
    return first;
}

// where a thread of the carries and emit kernels works: super-tile st (two
// tiles of the codes kernel, 64 KiB), bytes [abs, abs + my_len) of at most 128,
// which are the codes kernel's chunks 2 (tid mod 256) and 2 (tid mod 256) + 1 of
// its tile 2 st + tid / 256
struct PairPos {
    uint32_t st, tile, abs, my_len;
    size_t pair;  // global pair index: tile * 256 + tid mod 256
    bool valid, full;
};

__device__ __forceinline__ PairPos pair_pos(const FastParams& p, uint32_t st)
{
    PairPos c;
    c.st = st;
    c.tile = 2 * st + threadIdx.x / (kFastBlock / 2);
    c.valid = c.tile < p.num_tiles;
    c.abs = st * (uint32_t)(2 * kFastTile) + threadIdx.x * (uint32_t)(2 * kFastChunk);
    c.my_len = c.abs < p.n ? min((uint32_t)(2 * kFastChunk), p.n - c.abs) : 0u;
    c.full = c.my_len == (uint32_t)(2 * kFastChunk);
    c.pair = (size_t)c.tile * (kFastBlock / 2) + threadIdx.x % (kFastBlock / 2);
    return c;
}

// pass 2 over a ragged span (the input's last bytes), one byte at a time
template <int CB>
__device__ void pass2_ragged(const FastParams& p, const PairPos& c, uint32_t s, uint32_t nt, const uint8_t* s_nxt,
                             const uint8_t* s_tag, uint64_t (&T)[2], uint64_t (&RD)[2], uint32_t& err)
{
    T[0] = T[1] = RD[0] = RD[1] = 0;
    for (uint32_t j = 0; j < c.my_len; ++j) {
        const uint32_t code = classify1<CB>(p.in[c.abs + j], p);
        const uint32_t row = min(s, nt);
        const uint32_t t = s_tag[row * 16 + code];
        s = s_nxt[row * 16 + code];
        T[j >> 6] |= (uint64_t)(t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) << (j & 63);
        RD[j >> 6] |= (uint64_t)(t == PPR_TAG_RECORD) << (j & 63);
        if (t == PPR_TAG_INVALID && err == kNone) err = c.abs + j;
    }
}

// What the carries and emit kernels read per thread: the group indices of its
// two chunks (2 NI bytes, 16-byte loads) and the first chunk's vector of its
// tile's earlier bytes. Loaded one super-tile ahead of use.
template <int CB, bool V8>
struct IdxIn {
    uint32_t pw[2 * Geo<CB>::NP];
    uint32_t cvlo, cvhi;
    uint64_t tvl;  // lane l: tile vector 2 st + (l & 1) (kept per lane until used, see span_state)
};

// FULL: the span is known to be full (no branch around the loads)
template <int CB, bool V8, bool FULL>
__device__ __forceinline__ IdxIn<CB, V8> load_in(const FastParams& p, const PairPos& c)
{
    constexpr int NI = Geo<CB>::NI, NP = Geo<CB>::NP;
    IdxIn<CB, V8> in;
    if (FULL || c.full) {
        const uint4* src = reinterpret_cast<const uint4*>(p.idx + c.pair * (2 * NI));
#pragma unroll
        for (int q = 0; q < NP / 2; ++q) {
            const uint4 x = src[q];
            in.pw[4 * q] = x.x;
            in.pw[4 * q + 1] = x.y;
            in.pw[4 * q + 2] = x.z;
            in.pw[4 * q + 3] = x.w;
        }
    }
    const size_t ci = c.valid ? c.pair : 0;  // the span's first (even) chunk
    in.cvlo = p.cvec_lo[ci];
    in.cvhi = V8 ? p.cvec_hi[ci] : 0xffffffffu;
    in.tvl = p.tile_vec[min(2 * c.st + (threadIdx.x & 1u), p.num_tiles - 1)];
    return in;
}

// The workspace header's per-call fields (the first kernel of a call resets them).
__device__ __forceinline__ void reset_header(const FastParams& p)
{
    p.hdr->tile_counter = 0;
    p.hdr->fault = 0;
    p.hdr->err_min = kNone;
    p.hdr->last_rec = 0;
    p.hdr->path = p.path;
    p.hdr->cols_min = kNone;
    p.hdr->cols_max = 0;
    p.hdr->bad_records = 0;
    p.hdr->first_bad = kNone;
}

// Pass-1 table: entry e (the codes of G bytes) -> composite vector from every
// tracked state (words [0, E): entries 0-3, words [E, 2E): entries 4-7). The
// threads of a workgroup build it together from the byte step table s_nxt.
template <int CB, bool V8>
__device__ void build_pass1(uint32_t* t1, const uint8_t* s_nxt, uint32_t nt)
{
    constexpr int G = Geo<CB>::G, E = Geo<CB>::E;
    constexpr uint32_t CM = Geo<CB>::CM;
    for (uint32_t e = threadIdx.x; e < (uint32_t)E; e += blockDim.x) {
        uint32_t lo = 0, hi = 0;
        for (int i = 0; i < (V8 ? 8 : 4); ++i) {
            uint32_t s = (uint32_t)i < nt ? (uint32_t)i : kAbs;
            for (int g = 0; g < G; ++g)
                if (s != kAbs) s = s_nxt[s * 16 + ((e >> (CB * g)) & CM)];
            if (i < 4) lo |= s << (8 * i);
            else hi |= s << (8 * (i - 4));
        }
        t1[e] = lo;
        if (V8) t1[E + e] = hi;
    }
}

// Pass-2 tables (layout above: rows of kRowStride entries, one set of nt + 1
// rows per table), built by the threads of a workgroup from the byte tables.
template <int CB>
__device__ void build_pass2(uint32_t* t2, const uint8_t* s_nxt, const uint8_t* s_tag, uint32_t nt)
{
    constexpr int G = Geo<CB>::G, E = Geo<CB>::E;
    constexpr uint32_t CM = Geo<CB>::CM;
    const uint32_t cells = (nt + 1) * (uint32_t)E;
    for (uint32_t i = threadIdx.x; i < cells; i += blockDim.x) {
        const uint32_t r = i / (uint32_t)E, e = i % (uint32_t)E;
        uint32_t s = r, tb = 0, rb = 0, inv = 0;
        for (int g = 0; g < G; ++g) {
            const uint32_t c = (e >> (CB * g)) & CM;
            const uint32_t t = s_tag[s * 16 + c];
            const uint32_t ns = s_nxt[s * 16 + c];
            if (t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) tb |= 1u << g;
            if (t == PPR_TAG_RECORD) rb |= 1u << g;
            if (t == PPR_TAG_INVALID && !inv) inv = kP2Invalid | (uint32_t)g;
            s = ns == kAbs ? nt : ns;
        }
        if constexpr (G == 4) {
            t2[r * kRowStride + e] = inv | ((nt + 1 + s) << 8) | (tb << 16) | (rb << 24);
            t2[(nt + 1 + r) * kRowStride + e] = inv | (s << 8) | (tb << 20) | (rb << 28);
        } else {
            t2[r * kRowStride + e] = inv | (s << 8) | (tb << 16) | (rb << 20);
        }
    }
}

// The fused path's tables (in the workspace, read by every workgroup), built
// by workgroup 0, which also resets the workspace header; every workgroup
// clears a share of the two look-back status arrays.
template <int CB, bool V8>
__global__ void csv_fast_tables_kernel(FastParams p)
{
    __shared__ uint8_t s_nxt[9 * 16], s_tag[9 * 16];
    clear_status(reinterpret_cast<uint4*>(p.stat_vec), ((uint64_t)p.num_tiles + 1) / 2);
    clear_status(reinterpret_cast<uint4*>(p.stat_carry), (uint64_t)p.num_tiles * (sizeof(StatB) / 16));
    if (blockIdx.x != 0) return;
    if (threadIdx.x < 9 * 16) {
        s_nxt[threadIdx.x] = (&p.nxt[0][0])[threadIdx.x];
        s_tag[threadIdx.x] = (&p.tag[0][0])[threadIdx.x];
    }
    if (threadIdx.x == 0) reset_header(p);
    __syncthreads();
    build_pass1<CB, V8>(p.tabs, s_nxt, p.nt);
    build_pass2<CB>(p.tabs + (V8 ? 2 : 1) * Geo<CB>::E, s_nxt, s_tag, p.nt);
}

// The streaming kernels run num_ranges workgroups; workgroup b owns the
// contiguous super-tiles [s0, s1) below (a super-tile is two tiles of the codes
// kernel, 64 KiB) and walks them in order, loading the next one's inputs while
// it works on the current one. Along its range it carries the state (carries,
// emit) and the count carry (emit) from super-tile to super-tile, so the
// device-wide scans only run over the num_ranges range aggregates, in each
// workgroup's prologue.
__device__ __forceinline__ void range_of(const FastParams& p, uint32_t b, uint32_t& s0, uint32_t& s1)
{
    s0 = (uint32_t)((uint64_t)b * p.num_super / p.num_ranges);
    s1 = (uint32_t)((uint64_t)(b + 1) * p.num_super / p.num_ranges);
}

__device__ __forceinline__ Vec unpack_vec(uint64_t x) { return Vec{(uint32_t)x, (uint32_t)(x >> 32)}; }

// composite of the range vectors of ranges 0..b-1 (thread i takes ranges 2i, 2i+1;
// loads from clamped indices, then word-wise selects)
template <bool V8>
__device__ Vec ranges_before(const FastParams& p, uint32_t b, const Vec& ident, Vec* s_wave)
{
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

// pass-2 table rows (tracked states + the absorbing row, per table) and the byte tables
template <bool V8, int PAR>
struct Pass2Shared {
    uint32_t t2[PAR * (V8 ? 9 : 5) * kRowStride];
    uint8_t nxt[9 * 16], tag[9 * 16];
};

// The byte tables and the pass-2 tables in LDS, built by the workgroup (the
// caller's next barrier publishes the pass-2 tables).
template <int CB, bool V8>
__device__ __forceinline__ void load_pass2(const FastParams& p, Pass2Shared<V8, Geo<CB>::PAR>& sh)
{
    if (threadIdx.x < 9 * 16) {
        sh.nxt[threadIdx.x] = (&p.nxt[0][0])[threadIdx.x];
        sh.tag[threadIdx.x] = (&p.tag[0][0])[threadIdx.x];
    }
    __syncthreads();
    build_pass2<CB>(sh.t2, sh.nxt, sh.tag, p.nt);
}

// codes: symbol codes -> group indices (stored); the vector of the tile's bytes
// before each even chunk, the tile vectors and the range vector (stored).
//
// The loop runs over the range's entirely full tiles with no per-chunk
// branch, so that the next tile's loads stay in flight while the current one is
// worked on; the input's ragged last tile, if the range holds it, is done after
// the loop by the same body with the per-chunk checks.
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock) csv_codes_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    constexpr int NI = Gm::NI, ND = Gm::ND, NP = Gm::NP;
    constexpr int T1W = V8 ? 2 * Gm::E : Gm::E;
    __shared__ uint32_t s_t1[T1W];
    __shared__ uint8_t s_nxt[9 * 16];
    __shared__ Vec s_wave[2][kFastWaves];
    __shared__ Pass2Shared<V8, Gm::PAR> s_p2;
    __shared__ uint4 s_sx[2][kFastWaves][2];  // per wave: its speculative carry, its first INVALID byte

    const int tid = threadIdx.x;
    // workgroup b takes tiles b, b + G, b + 2G, ... (G = the grid): the workgroups
    // in flight read one contiguous window of the input
    const uint32_t stride = gridDim.x;
    const uint32_t tfull_all = p.n / (uint32_t)kFastTile;  // tiles [0, tfull_all) are entirely full
    auto load_full = [&](uint32_t tile, uint32_t (&w)[ND]) {
        const uint4* src = reinterpret_cast<const uint4*>(p.in + (size_t)tile * kFastTile + tid * kFastChunk);
#pragma unroll
        for (int q = 0; q < ND / 4; ++q) {
            const uint4 x = src[q];
            w[4 * q] = x.x;
            w[4 * q + 1] = x.y;
            w[4 * q + 2] = x.z;
            w[4 * q + 3] = x.w;
        }
    };
    uint32_t w[ND];
    const uint32_t t0 = blockIdx.x;
    if (t0 < tfull_all) load_full(t0, w);
    if (tid < 9 * 16) s_nxt[tid] = (&p.nxt[0][0])[tid];
    if (blockIdx.x == 0 && tid == 0) reset_header(p);  // (no kernel of the call has read it yet)
    __syncthreads();
    build_pass1<CB, V8>(s_t1, s_nxt, p.nt);
    load_pass2<CB, V8>(p, s_p2);
    __syncthreads();
    const Vec ident = fast_ident<V8>(p.nt);

    // classify, store the indices, the chunk's vector
    auto store_slot = [&](uint32_t tile, const uint32_t (&pw)[NP]) {
        uint4* dst = reinterpret_cast<uint4*>(p.idx + ((size_t)tile * kFastBlock + tid) * NI);
#pragma unroll
        for (int q = 0; q < NP / 4; ++q)
            dst[q] = make_uint4(pw[4 * q], pw[4 * q + 1], pw[4 * q + 2], pw[4 * q + 3]);
    };
    // (speculating configurations store the slot after the block scan: indices
    // or tag bitmaps)
    auto full_chunk = [&](uint32_t tile, const uint32_t (&wc)[ND], uint32_t (&pw)[NP]) {
        uint32_t ia[NI];
        chunk_codes<CB>(wc, p, ia, pw);
        if constexpr (!kSpeculates<CB, V8>) store_slot(tile, pw);
        return tree_vector<CB, V8>(ia, s_t1);
    };
    // The speculative carry of a full tile (see tile_speculates): pass 2 over
    // each chunk of an agreed span from its agreed state; each wave's count
    // carry and first INVALID byte go to LDS, and thread 0 combines them and
    // stores the tile's after the next barrier (the next tile's block scan, or
    // the one at the end), so that this costs no barrier of its own.
    int64_t spec_tile = -1;  // the tile whose wave carries wait in s_sx[spec_buf]
    uint32_t spec_buf = 0;
    auto speculate = [&](uint32_t tile, const Vec& excl, const uint32_t (&pw)[NP], uint32_t it, uint64_t (&T)[1],
                         uint64_t (&RD)[1]) {
        const Vec ev{even_lane(excl.lo), V8 ? even_lane(excl.hi) : 0xffffffffu};
        uint32_t xs, x;
        const bool mine = vec_agreed<V8>(ev, xs);  // the span's first chunk agrees
        vec_agreed<V8>(excl, x);                   // this chunk's start (it agrees if that one does)
        T[0] = RD[0] = 0ull;
        uint32_t err = kNone;
        const uint32_t abs = tile * (uint32_t)kFastTile + (uint32_t)tid * (uint32_t)kFastChunk;
        if (mine) {
            const uint32_t any = pass2_run<CB, 1>(pw, x, p.nt, s_p2.t2, T, RD);
            if (any & kP2Invalid) err = first_invalid<CB, 1>(pw, x, p.nt, s_p2.t2, abs);
        }
        const GCarry wc = wave_carry<1>(T, RD, abs).wc;
        const uint32_t werr = wave_min_defined(err);
        if (lane_id() == 0) {
            s_sx[it & 1][tid / kWave][0] = make_uint4(wc.nf, wc.nr, wc.col, wc.lt);
            s_sx[it & 1][tid / kWave][1] = make_uint4(werr, 0u, 0u, 0u);
        }
        spec_tile = tile;
        spec_buf = it & 1;
        return mine;
    };
    // after a barrier: the pending tile's speculative carry
    auto flush_spec = [&]() {
        if (spec_tile >= 0 && tid == 0) {
            const GCarryComb gc;
            GCarry r{0u, 0u, 0u, 0u};
            uint32_t e = kNone;
#pragma unroll
            for (int i = 0; i < kFastWaves; ++i) {
                const uint4 q = s_sx[spec_buf][i][0];
                r = gc(r, GCarry{q.x, q.y, q.z, q.w});
                e = min(e, s_sx[spec_buf][i][1].x);
            }
            uint4* dst = reinterpret_cast<uint4*>(p.spec + (size_t)spec_tile * kSpWords);
            dst[0] = make_uint4(r.nf, r.nr, r.col, r.lt);
            dst[1] = make_uint4(e, 0u, 0u, 0u);
        }
        spec_tile = -1;
    };
    // scan the tile's chunk vectors, store those of the even chunks (where the
    // carries and emit kernels' two-chunk spans start) and the tile vector
    //
    // Every lane issues the same stores (an odd lane writes its even
    // neighbour's vector to the same word, every wave the tile vector): with
    // no store skipped by a branch, the compiler knows how many memory
    // operations follow each prefetch and waits for the prefetch alone, not for
    // the previous tile's stores as well.
    auto finish = [&](uint32_t tile, const Vec& v, uint32_t it, Vec& excl, Vec& tot) {
        block_scan<kFastWaves>(v, ident, excl, tot, s_wave[it & 1], VecComb<V8>{});
        flush_spec();  // (the block scan's barrier publishes the previous tile's wave carries)
        const size_t ci = (size_t)tile * (kFastBlock / 2) + (uint32_t)tid / 2;
        p.cvec_lo[ci] = even_lane(excl.lo);
        if (V8) p.cvec_hi[ci] = even_lane(excl.hi);
        p.tile_vec[tile] = (uint64_t)tot.lo | ((uint64_t)tot.hi << 32);
    };
    // a full tile: codes, indices, vectors, and the speculative carry where the
    // tile vector (the block scan's total, the same in every thread) agrees
    auto full_tile = [&](uint32_t tile, const uint32_t (&wc)[ND], uint32_t it) {
        uint32_t pw[NP];
        Vec excl, tot;
        finish(tile, full_chunk(tile, wc, pw), it, excl, tot);
        if constexpr (kSpeculates<CB, V8>) {
            uint32_t xt;
            if (tile_speculates<V8>(p, tile, tot, xt)) {
                uint64_t T[1], RD[1];
                if (speculate(tile, excl, pw, it, T, RD) && p.quiet_abs) {
                    pw[0] = (uint32_t)T[0];
                    pw[1] = (uint32_t)(T[0] >> 32);
                    pw[2] = (uint32_t)RD[0];
                    pw[3] = (uint32_t)(RD[0] >> 32);
                }
            }
            store_slot(tile, pw);
        }
    };

    // Two register buffers used in turn, and an unconditional prefetch (the
    // last full tile is read again at the end): no copy of a register still
    // being loaded and no branch around a load, either of which would make the
    // compiler wait for the prefetch before the current tile's work. The first
    // tile is peeled off the loop, so that every entry to the loop body, like
    // every other tile, follows a tile's stores: the wait for a prefetch then
    // leaves those stores in flight.
    uint32_t w2[ND];
    uint32_t tile = t0;
    // the last full tile this workgroup takes
    const uint32_t tlast = tfull_all > t0 ? t0 + (tfull_all - 1 - t0) / stride * stride : t0;
    uint32_t it = 0;
    if (tile < tfull_all) {
        load_full(min(tile + stride, tlast), w2);
        full_tile(tile, w, it++);
        tile += stride;
        while (tile < tfull_all) {
            load_full(min(tile + stride, tlast), w);
            full_tile(tile, w2, it++);
            tile += stride;
            if (tile >= tfull_all) break;
            load_full(min(tile + stride, tlast), w2);
            full_tile(tile, w, it++);
            tile += stride;
        }
    }
    if (tile < p.num_tiles) {  // the input's ragged last tile (it never speculates)
        const ChunkPos c = chunk_pos(p.n, tile);
        Vec v = ident;
        if (c.full) {
            load_full(tile, w);
            uint32_t pw[NP];
            v = full_chunk(tile, w, pw);
            if constexpr (kSpeculates<CB, V8>) store_slot(tile, pw);
        } else if (c.my_len) {
            v = ragged_vector<CB, V8>(p, c, v, s_nxt);
        }
        Vec excl, tot;
        finish(tile, v, it, excl, tot);
    }
    if (spec_tile >= 0) {  // (uniform)
        __syncthreads();
        flush_spec();
    }
}

// range vectors: one wave per range composes the range's tile vectors, 64 at a
// time (coalesced loads, a DPP wave scan)
template <bool V8>
__global__ void __launch_bounds__(kWave) csv_range_vec_kernel(FastParams p)
{
    uint32_t s0, s1;
    range_of(p, blockIdx.x, s0, s1);
    const uint32_t t0 = 2 * s0, t1 = min(2 * s1, p.num_tiles);
    const Vec ident = fast_ident<V8>(p.nt);
    Vec rv = ident;
    for (uint32_t t = t0; t < t1; t += kWave) {
        const uint32_t i = t + threadIdx.x;
        const Vec x = i < t1 ? unpack_vec(p.tile_vec[i]) : ident;
        rv = comp<V8>(rv, readlane_t(wave_scan(x, ident, VecComb<V8>{}), kWave - 1));
    }
    if (threadIdx.x == 0) p.range_vec[blockIdx.x] = (uint64_t)rv.lo | ((uint64_t)rv.hi << 32);
}

// The tile vectors of super-tile st from the lane-wise prefetch (the second is
// the identity if the super-tile has one tile). Broadcast only here, at their
// use: moving a loaded value to a scalar register at the prefetch would make
// the compiler wait for every load in flight.
template <bool V8>
__device__ __forceinline__ void super_vecs(const FastParams& p, uint32_t st, uint64_t tvl, const Vec& ident, Vec& v0,
                                           Vec& v1)
{
    const uint32_t lo = (uint32_t)tvl, hi = (uint32_t)(tvl >> 32);
    v0 = Vec{(uint32_t)__builtin_amdgcn_readlane(lo, 0), (uint32_t)__builtin_amdgcn_readlane(hi, 0)};
    v1 = Vec{(uint32_t)__builtin_amdgcn_readlane(lo, 1), (uint32_t)__builtin_amdgcn_readlane(hi, 1)};
    if (2 * st + 1 >= p.num_tiles) v1 = ident;
}

// Pass 2 for this thread's span: tags as bitmaps, the first INVALID byte (if
// wanted: err given and look true). ts0 / ts1: the state before the
// super-tile's first / second tile.
template <int CB, bool V8, bool FULL>
__device__ __forceinline__ void span_tags(const FastParams& p, const PairPos& c, const IdxIn<CB, V8>& in,
                                          uint32_t ts0, uint32_t ts1, const Pass2Shared<V8, Geo<CB>::PAR>& sh,
                                          uint64_t (&T)[2], uint64_t (&RD)[2], uint32_t* err, bool look = true,
                                          int mode = 0)
{
    const uint32_t nt = p.nt;
    const uint32_t s = vat(Vec{in.cvlo, in.cvhi}, threadIdx.x < kFastBlock / 2 ? ts0 : ts1);
    T[0] = T[1] = RD[0] = RD[1] = 0;
    if (mode == 2) return;
    if (mode == 1) {
        slot_bits(in.pw, T, RD);
        return;
    }
    if (FULL || c.full) {
        const uint32_t any = pass2_pair<CB>(in.pw, s, nt, sh.t2, T, RD);
        if (err && look && (any & kP2Invalid)) *err = first_invalid<CB, 2>(in.pw, s, nt, sh.t2, c.abs);
    } else if (c.my_len) {
        uint32_t e = kNone;
        pass2_ragged<CB>(p, c, s, nt, sh.nxt, sh.tag, T, RD, e);
        if (err) *err = e;
    }
}

// Runs body(st, in, it) over the range's super-tiles [s0, s1) in order: the
// entirely full ones [s0, sfull) with two register buffers used in turn and an
// unconditional prefetch (the last full super-tile is read again at the end),
// then the input's ragged last super-tile, if the range holds it. it = (st -
// s0) mod 2 alternates from call to call, for LDS scratch used in turn.
template <int CB, bool V8, typename FullBody, typename TailBody>
__device__ __forceinline__ void walk_supers(const FastParams& p, uint32_t s0, uint32_t s1, const FullBody& full,
                                            const TailBody& tail)
{
    const uint32_t sfull = min(s1, p.n / (uint32_t)(2 * kFastTile));
    uint32_t st = s0;
    IdxIn<CB, V8> a, b;
    if (st < sfull) a = load_in<CB, V8, true>(p, pair_pos(p, st));
    while (st < sfull) {
        b = load_in<CB, V8, true>(p, pair_pos(p, min(st + 1, sfull - 1)));
        full(st, a, 0u);
        if (++st >= sfull) break;
        a = load_in<CB, V8, true>(p, pair_pos(p, min(st + 1, sfull - 1)));
        full(st, b, 1u);
        ++st;
    }
    if (st < s1) tail(st, load_in<CB, V8, false>(p, pair_pos(p, st)), (st - s0) & 1u);  // (buffers keep alternating)
}

// Terminators of a 128-byte span (bitmaps T, bit j = byte j) at span
// positions k and later, 0 <= k < 128.
__device__ __forceinline__ uint32_t count_from(const uint64_t (&T)[2], uint32_t k)
{
    const uint64_t m0 = k < 64 ? ~0ull << k : 0ull;
    const uint64_t m1 = k < 64 ? ~0ull : ~0ull << (k - 64);
    return (uint32_t)(__popcll(T[0] & m0) + __popcll(T[1] & m1));
}

// A range's count carry from the codes kernel's speculative carries. A tile
// qualifies when its speculative carry holds (see tile_speculates) and it
// agrees from its span kSpecSpans - 1 on: then only the spans before its
// agreed ones need pass 2, at most kSpecSpans - 1, and those of 32 qualifying
// tiles run at once (16 threads per tile) instead of in the tiles' order. The
// other tiles of the range run pass 2 over all their spans, two tiles at a
// time (the input's last tile among them: it never qualifies). Ranges without a
// qualifying tile take the walk over their super-tiles instead.
constexpr uint32_t kSpecSpans = 16;
constexpr uint32_t kRangeTilesMax = 128;  // tiles of a range for n < 2^32 (1024 ranges of whole super-tiles)

struct FastRangeShared {
    uint32_t ts[kRangeTilesMax];  // each tile's start state
    uint4 tc[kRangeTilesMax];     // each tile's count carry
    uint32_t te[kRangeTilesMax];  // each tile's first INVALID byte
    uint8_t fastl[kRangeTilesMax], slowl[kRangeTilesMax];  // the qualifying tiles and the others, in order
    uint8_t bits[kRangeTilesMax];  // 0: indices only; 1: bitmaps that hold; 2: bitmaps of a dead path (span_mode)
    uint32_t nfast, nslow;
    uint32_t end;              // the state after the range
    uint4 red[2][kFastWaves];  // wave partials of the other tiles
};

// v combined over the 16 lanes of its row (a butterfly: every lane gets it)
template <typename Op>
__device__ __forceinline__ uint32_t row16_all(uint32_t v, const Op& op)
{
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) v = op(v, (uint32_t)__shfl_xor((int)v, m));
    return v;
}

struct MinComb {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};

// 1 + position of the last set bit of two consecutive 64-bit bitmaps of a span at abs (0: none)
__device__ __forceinline__ uint32_t last_pos1(const uint64_t (&B)[2], uint32_t abs)
{
    if (B[1]) return abs + (uint32_t)kFastChunk + (uint32_t)(64 - __clzll((long long)B[1]));
    if (B[0]) return abs + (uint32_t)(64 - __clzll((long long)B[0]));
    return 0u;
}

// terminators of a span at abs after position L - 1 (all when L is 0 or before the span)
__device__ __forceinline__ uint32_t terms_after(const uint64_t (&T)[2], uint32_t abs, uint32_t L)
{
    const uint32_t nf = (uint32_t)(__popcll(T[0]) + __popcll(T[1]));
    return L == 0 || abs >= L ? nf : (abs + 2u * kFastChunk > L ? count_from(T, L - abs) : 0u);
}

// Pass 2 over span pair of a full tile from the tile's start state ts.
template <int CB>
__device__ __forceinline__ void span_pass2(const FastParams& p, size_t pair, uint32_t cv, uint32_t ts, uint32_t abs,
                                           const Pass2Shared<false, Geo<CB>::PAR>& sh, uint64_t (&T)[2],
                                           uint64_t (&RD)[2], uint32_t& err)
{
    constexpr int NP = Geo<CB>::NP, NI = Geo<CB>::NI;
    uint32_t pw[2 * NP];
    const uint4* src = reinterpret_cast<const uint4*>(p.idx + pair * (2 * NI));
#pragma unroll
    for (int q = 0; q < NP / 2; ++q) {
        const uint4 v = src[q];
        pw[4 * q] = v.x;
        pw[4 * q + 1] = v.y;
        pw[4 * q + 2] = v.z;
        pw[4 * q + 3] = v.w;
    }
    const uint32_t st = vat(Vec{cv, 0xffffffffu}, ts);
    const uint32_t any = pass2_pair<CB>(pw, st, p.nt, sh.t2, T, RD);
    err = (any & kP2Invalid) ? first_invalid<CB, 2>(pw, st, p.nt, sh.t2, abs) : kNone;
}

// Every thread calls it; returns whether it stored the range's carry and first
// INVALID byte (false: the range needs the walk over its super-tiles).
template <int CB>
__device__ bool carries_fast_range(const FastParams& p, uint32_t b, uint32_t s0, uint32_t s1, uint32_t run,
                                   const Pass2Shared<false, Geo<CB>::PAR>& sh, FastRangeShared& fr)
{
    const uint32_t ta = 2 * s0, tb = min(2 * s1, p.num_tiles), nr_t = tb - ta;
    if (nr_t > kRangeTilesMax) return false;
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t w = threadIdx.x / kWave;
    const Vec ident = fast_ident<false>(p.nt);
    if (w == 0) {  // the tiles' start states, and which qualify
        uint32_t s = run, nf = 0, ns = 0;
        for (uint32_t base = 0; base < nr_t; base += kWave) {
            const uint32_t i = base + lane;
            const bool valid = i < nr_t;
            const Vec tv = unpack_vec(p.tile_vec[ta + (valid ? i : 0u)]);
            const Vec inc = wave_scan(select_t(valid, tv, ident), ident, VecComb<false>{});
            const uint32_t ts = vat(wave_shr1(ident, inc), s);
            uint32_t x, x2;
            const bool sp = valid && tile_speculates<false>(p, ta + i, tv, x);
            bool f = sp && vat(tv, ts) == x;
            if (valid) fr.bits[i] = (uint8_t)(sp && p.quiet_abs ? (vat(tv, ts) == x ? 1 : 2) : 0);
            if (f) f = vec_agreed<false>(Vec{p.cvec_lo[(size_t)(ta + i) * (kFastBlock / 2) + (kSpecSpans - 1)],
                                             0xffffffffu},
                                         x2);
            const uint64_t below = (1ull << lane) - 1ull;
            const uint64_t mf = __ballot(f), ms = __ballot(valid && !f);
            if (valid) {
                fr.ts[i] = ts;
                if (f) fr.fastl[nf + (uint32_t)__popcll(mf & below)] = (uint8_t)i;
                else fr.slowl[ns + (uint32_t)__popcll(ms & below)] = (uint8_t)i;
            }
            nf += (uint32_t)__popcll(mf);
            ns += (uint32_t)__popcll(ms);
            s = vat(readlane_t(inc, kWave - 1), s);
        }
        if (lane == 0) {
            fr.nfast = nf;
            fr.nslow = ns;
            fr.end = s;
        }
    }
    __syncthreads();
    const uint32_t nfast = fr.nfast, nslow = fr.nslow;
    if (nfast == 0) return false;
    const GCarryComb gc;
    // qualifying tiles: the spans before the agreed ones, 16 threads per tile
    for (uint32_t g = 0; g < nfast; g += kFastBlock / kSpecSpans) {
        const uint32_t li = g + threadIdx.x / kSpecSpans, j = threadIdx.x % kSpecSpans;
        const bool valid = li < nfast;
        const uint32_t i = fr.fastl[valid ? li : g], t = ta + i;
        const size_t pair = (size_t)t * (kFastBlock / 2) + j;
        const uint32_t cv = p.cvec_lo[pair];
        uint32_t xs;
        const bool todo = valid && !vec_agreed<false>(Vec{cv, 0xffffffffu}, xs);
        const uint32_t abs = t * (uint32_t)kFastTile + j * (uint32_t)(2 * kFastChunk);
        uint64_t T[2] = {0ull, 0ull}, RD[2] = {0ull, 0ull};
        uint32_t err = kNone;
        if (todo) {
            span_pass2<CB>(p, pair, cv, fr.ts[i], abs, sh, T, RD, err);
            if (p.quiet_abs) {  // the span's bitmaps for the emit kernel, which then runs no pass 2 on this tile
                uint4* dst = reinterpret_cast<uint4*>(p.idx + pair * (2 * Geo<CB>::NI));
                dst[0] = make_uint4((uint32_t)T[0], (uint32_t)(T[0] >> 32), (uint32_t)RD[0], (uint32_t)(RD[0] >> 32));
                dst[1] = make_uint4((uint32_t)T[1], (uint32_t)(T[1] >> 32), (uint32_t)RD[1], (uint32_t)(RD[1] >> 32));
                p.cvec_lo[pair] = kBitsMark;
            }
        }
        // their count carry: the last record delimiter L (a row maximum), the terminators after it
        const uint32_t L = row16_all(last_pos1(RD, abs), MaxComb{});
        const GCarry pre{row16_all((uint32_t)(__popcll(T[0]) + __popcll(T[1])), AddComb{}),
                         row16_all((uint32_t)(__popcll(RD[0]) + __popcll(RD[1])), AddComb{}),
                         row16_all(terms_after(T, abs, L), AddComb{}), row16_all(last_pos1(T, abs), MaxComb{})};
        const uint32_t perr = row16_all(err, MinComb{});
        if (valid && j == 0) {
            const uint4* sp = reinterpret_cast<const uint4*>(p.spec + (size_t)t * kSpWords);
            const uint4 a = sp[0], e = sp[1];
            const GCarry c = gc(pre, GCarry{a.x, a.y, a.z, a.w});
            fr.tc[i] = make_uint4(c.nf, c.nr, c.col, c.lt);
            fr.te[i] = min(perr, e.x);
        }
    }
    // the other tiles: every span, a tile per half of the workgroup
    for (uint32_t k = 0; k < nslow; k += 2) {
        const uint32_t h = threadIdx.x / (kFastBlock / 2), j = threadIdx.x % (kFastBlock / 2);
        const bool valid = k + h < nslow;
        const uint32_t i = fr.slowl[valid ? k + h : k], t = ta + i;
        const size_t pair = (size_t)t * (kFastBlock / 2) + j;
        const uint32_t abs = t * (uint32_t)kFastTile + j * (uint32_t)(2 * kFastChunk);
        const uint32_t my_len = abs < p.n ? min((uint32_t)(2 * kFastChunk), p.n - abs) : 0u;
        uint64_t T[2] = {0ull, 0ull}, RD[2] = {0ull, 0ull};
        uint32_t err = kNone;
        const uint32_t cv = p.cvec_lo[pair];
        const int mode = span_mode<CB, false>(fr.bits[i] != 0, fr.bits[i] == 1, cv, 0xffffffffu);
        if (mode == 1) {
            const uint4* src = reinterpret_cast<const uint4*>(p.idx + pair * (2 * Geo<CB>::NI));
            const uint4 a = src[0], c2 = src[1];
            const uint32_t pw[8] = {a.x, a.y, a.z, a.w, c2.x, c2.y, c2.z, c2.w};
            slot_bits(pw, T, RD);
        } else if (mode == 2) {
        } else if (my_len == 2u * kFastChunk) {
            span_pass2<CB>(p, pair, cv, fr.ts[i], abs, sh, T, RD, err);
        } else if (my_len) {  // the input's ragged last tile: from the bytes
            PairPos c;
            c.abs = abs;
            c.my_len = my_len;
            pass2_ragged<CB>(p, c, vat(Vec{cv, 0xffffffffu}, fr.ts[i]), p.nt, sh.nxt, sh.tag, T, RD, err);
        }
        if (valid && my_len && abs + my_len == p.n)  // the thread holding the input's last byte
            p.hdr->last_rec = (uint32_t)((RD[(my_len - 1) >> 6] >> ((my_len - 1) & 63)) & 1u);
        // positions grow with the lanes: a wave's last is its last lane's holding one
        const uint32_t rdp = last_pos1(RD, abs), ltp = last_pos1(T, abs);
        const uint64_t hr = __ballot(rdp != 0), ht = __ballot(ltp != 0);
        const uint32_t wrd = hr ? (uint32_t)__builtin_amdgcn_readlane(rdp, 63 - __clzll((long long)hr)) : 0u;
        if (lane == 0) fr.red[0][w] = make_uint4(wrd, 0u, 0u, 0u);
        __syncthreads();
        const uint32_t w0 = h * (kFastWaves / 2);
        uint32_t L = 0;
#pragma unroll
        for (int q = 0; q < kFastWaves / 2; ++q) L = max(L, fr.red[0][w0 + q].x);
        const uint32_t nf = (uint32_t)(__popcll(T[0]) + __popcll(T[1]));
        const uint32_t nr = (uint32_t)(__popcll(RD[0]) + __popcll(RD[1]));
        const uint32_t cnt = readlane_t(wave_scan(nf | (nr << 16), 0u, AddComb{}), kWave - 1);
        const uint32_t aft = readlane_t(wave_scan(terms_after(T, abs, L), 0u, AddComb{}), kWave - 1);
        const uint32_t wlt = ht ? (uint32_t)__builtin_amdgcn_readlane(ltp, 63 - __clzll((long long)ht)) : 0u;
        const uint32_t werr = wave_min_defined(err);
        if (lane == 0) fr.red[1][w] = make_uint4(cnt, aft, wlt, werr);
        __syncthreads();
        if (valid && j == 0) {
            uint32_t snf = 0, snr = 0, sc = 0, sl = 0, se = kNone;
#pragma unroll
            for (int q = 0; q < kFastWaves / 2; ++q) {
                const uint4 v = fr.red[1][w0 + q];
                snf += v.x & 0xffffu;
                snr += v.x >> 16;
                sc += v.y;
                sl = max(sl, v.z);
                se = min(se, v.w);
            }
            fr.tc[i] = make_uint4(snf, snr, sc, sl);
            fr.te[i] = fr.bits[i] == 1 ? min(se, p.spec[(size_t)t * kSpWords + 4]) : se;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        GCarry r{0u, 0u, 0u, 0u};
        uint32_t e = kNone;
        for (uint32_t i = 0; i < nr_t; ++i) {
            const uint4 q = fr.tc[i];
            r = gc(r, GCarry{q.x, q.y, q.z, q.w});
            e = min(e, fr.te[i]);
        }
        p.range_carry[b] = make_uint4(r.nf, r.nr, r.col, r.lt);
        p.range_err[b] = e;
        if (b == p.num_ranges - 1) {
            const uint32_t x = min(fr.end, 8u);
            p.hdr->end_state = p.state_of[x];
            p.hdr->error_pos = (p.partial || ((p.accept_codes >> x) & 1u)) ? (int64_t)-1 : (int64_t)p.n;  // before err_min
        }
    }
    return true;
}

// Register budgets of the carries and emit kernels (waves per SIMD; a
// workgroup is two per SIMD). With 4-byte groups both wait mostly on their
// pass-2 lookup chains and fit 64 VGPRs, four workgroups per CU (the emit
// kernel only with at most 4 tracked states: with more, its LDS holds three).
// With 2-byte groups they take up to 128 (the carries kernel would spill below
// that, and the emit kernel measured slower at 80 VGPRs and three workgroups
// per CU).
template <int CB>
constexpr int kCarriesWavesPerSimd = CB == 2 ? 8 : 4;
template <int CB, bool V8>
constexpr int kEmitWavesPerSimd = CB == 2 && !V8 ? 8 : 4;

// carries: the range's start state (stored), tags from each span's start state,
// the range's count carry (stored); the last range stores the end state.
//
// The count carry needs no scan: terminator and record counts add up and the
// last terminator is a maximum, in any order, so each thread accumulates its
// own; the column carry (terminators after the range's last record delimiter)
// follows from one block maximum per super-tile, the position of its last
// record delimiter: a super-tile that has one restarts every thread's count at
// its terminators after that position, one without adds all of them. The
// thread sums and maxima are reduced once, at the end of the range.
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock, kCarriesWavesPerSimd<CB>) csv_carries_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    __shared__ Pass2Shared<V8, Gm::PAR> sh;
    __shared__ uint32_t s_rd[2][kFastWaves];
    __shared__ Vec s_wv[kFastWaves];
    __shared__ uint4 s_red[kFastWaves];
    __shared__ uint32_t s_err[kFastWaves];

    const uint32_t b = blockIdx.x;
    const uint32_t lane = (uint32_t)lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    uint32_t s0, s1;
    range_of(p, b, s0, s1);
    const uint32_t nt = p.nt;
    const Vec ident = fast_ident<V8>(nt);
    load_pass2<CB, V8>(p, sh);
    uint32_t run = vat(ranges_before<V8>(p, b, ident, s_wv), p.start_code);  // (its barrier publishes sh)
    if (threadIdx.x == 0) p.range_state[b] = run;
    if constexpr (kSpeculates<CB, V8>) {
        __shared__ FastRangeShared s_fr;
        if (carries_fast_range<CB>(p, b, s0, s1, run, sh, s_fr)) return;
    }
    uint32_t acc_nf = 0, acc_nr = 0, acc_col = 0, acc_lt = 0;
    uint32_t sp_err = kNone;  // from the speculative carries of tiles read from bitmaps (uniform)
    // the first INVALID byte of the wave's spans (wave-uniform): once found, later
    // super-tiles (larger positions) are not searched; the range's (the waves'
    // minimum) is stored, and the emit kernel takes the minimum over the ranges
    // (atomics on one word from every wave would serialize)
    uint32_t wave_err = kNone;

    auto step = [&](auto full_tag, uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) {
        constexpr bool FULL = decltype(full_tag)::value;
        const PairPos c = pair_pos(p, st);
        Vec v0, v1;
        super_vecs<V8>(p, st, in.tvl, ident, v0, v1);
        const uint32_t ts1 = vat(v0, run);
        uint32_t xa = 0, xb = 0;
        const bool ba = kSpeculates<CB, V8> && tile_bits<V8>(p, 2 * st, v0, xa);
        const bool bb = kSpeculates<CB, V8> && tile_bits<V8>(p, 2 * st + 1, v1, xb);
        const bool ha = vat(v0, run) == xa, hb = vat(v1, ts1) == xb;
        const bool upper = threadIdx.x >= kFastBlock / 2;
        const int mode = span_mode<CB, V8>(upper ? bb : ba, upper ? hb : ha, in.cvlo, in.cvhi);
        uint64_t T[2], RD[2];
        uint32_t err = kNone;
        span_tags<CB, V8, FULL>(p, c, in, run, ts1, sh, T, RD, &err, wave_err == kNone, mode);
        // a tile read from bitmaps: its agreed chunks' first INVALID byte is in its speculative carry
        if (ba && ha) sp_err = min(sp_err, p.spec[(size_t)(2 * st) * kSpWords + 4]);
        if (bb && hb) sp_err = min(sp_err, p.spec[(size_t)(2 * st + 1) * kSpWords + 4]);
        if (wave_err == kNone) wave_err = wave_min_defined(err);
        if (c.my_len && c.abs + c.my_len == p.n)  // the thread holding the input's last byte
            p.hdr->last_rec = (uint32_t)((RD[(c.my_len - 1) >> 6] >> ((c.my_len - 1) & 63)) & 1u);
        const uint32_t nf = (uint32_t)(__popcll(T[0]) + __popcll(T[1]));
        acc_nf += nf;
        acc_nr += (uint32_t)(__popcll(RD[0]) + __popcll(RD[1]));
        if (T[1]) acc_lt = c.abs + (uint32_t)kFastChunk + (uint32_t)(63 - __clzll((long long)T[1])) + 1u;
        else if (T[0]) acc_lt = c.abs + (uint32_t)(63 - __clzll((long long)T[0])) + 1u;
        // 1 + position of the super-tile's last record delimiter (0: none)
        uint32_t rdp = 0;
        if (RD[1]) rdp = c.abs + (uint32_t)kFastChunk + (uint32_t)(63 - __clzll((long long)RD[1])) + 1u;
        else if (RD[0]) rdp = c.abs + (uint32_t)(63 - __clzll((long long)RD[0])) + 1u;
        const uint64_t has_r = __ballot(rdp != 0);
        if (lane == 0)
            s_rd[it & 1][w] = has_r ? (uint32_t)__builtin_amdgcn_readlane(rdp, 63 - __clzll((long long)has_r)) : 0u;
        __syncthreads();
        const uint4 x = reinterpret_cast<const uint4*>(s_rd[it & 1])[0];
        const uint4 y = reinterpret_cast<const uint4*>(s_rd[it & 1])[1];
        const uint32_t L = max(max(max(x.x, x.y), max(x.z, x.w)), max(max(y.x, y.y), max(y.z, y.w)));
        if (L == 0) acc_col += nf;
        else if (c.abs >= L) acc_col = nf;
        else acc_col = c.abs + 2u * kFastChunk > L ? count_from(T, L - c.abs) : 0u;
        run = vat(v1, ts1);
    };
    walk_supers<CB, V8>(
        p, s0, s1, [&](uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) { step(std::true_type{}, st, in, it); },
        [&](uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) { step(std::false_type{}, st, in, it); });

    // the range's carry: sums of nf, nr, col and the maximum of lt over the threads
    const uint32_t snf = wave_scan(acc_nf, 0u, AddComb{}), snr = wave_scan(acc_nr, 0u, AddComb{});
    const uint32_t scol = wave_scan(acc_col, 0u, AddComb{}), slt = wave_scan(acc_lt, 0u, MaxComb{});
    if (lane == kWave - 1) s_red[w] = make_uint4(snf, snr, scol, slt);
    if (lane == 0) s_err[w] = min(wave_err, sp_err);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint4 r = s_red[0];
        uint32_t e = s_err[0];
        for (int i = 1; i < kFastWaves; ++i) {
            const uint4 q = s_red[i];
            r = make_uint4(r.x + q.x, r.y + q.y, r.z + q.z, max(r.w, q.w));
            e = min(e, s_err[i]);
        }
        p.range_carry[b] = make_uint4(r.x, r.y, r.z, r.w);
        p.range_err[b] = e;
        if (b == p.num_ranges - 1) {
            const uint32_t e = min(run, 8u);
            p.hdr->end_state = p.state_of[e];
            p.hdr->error_pos = (p.partial || ((p.accept_codes >> e) & 1u)) ? (int64_t)-1 : (int64_t)p.n;  // before err_min
        }
    }
}


// Running values of a wave's field emission (wave-uniform): the record index,
// column and offset of its next field.
struct FieldRun {
    uint32_t rec, col, off;
};

// One round of at most 64 of a wave's fields: lane l writes field g0 + l (g0
// wave-uniform) from its list entry e (position - base << 1 | record bit). The
// record index is the running one plus the record bits of the earlier lanes
// (mbcnt), the column counts from the last record field before the lane, the
// offset follows the previous lane's terminator (DPP). The four arrays are
// written through wave-uniform base pointers, so every store is one scalar
// base plus the lane's offset. Only the window's first `slots` fields are
// written (those below the capacity); rel: the round's offset in the window.
// lt_mask: the lanes below this one. A lane whose field ends a record notes
// that record's fields (its column + 1) in its running record counts.
__device__ __forceinline__ void field_round(const OutArrays& o, uint32_t g0, uint32_t rel, uint32_t slots,
                                            uint32_t cnt, uint32_t e, uint32_t base, uint32_t lane, uint64_t lt_mask,
                                            FieldRun& fr, RecStats& st, uint32_t expect)
{
    const uint32_t pos = base + (e >> 1);
    const uint64_t m = __ballot(lane < cnt && (e & 1u));
    const uint64_t below = m & lt_mask;
    const uint32_t rec =
        fr.rec + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const uint32_t col = below ? lane - (uint32_t)(63 - __clzll((long long)below)) - 1u : fr.col + lane;
    const uint32_t prev = dpp_t<0x138, 0xf>(0u, pos);  // wave_shr:1: the previous lane's terminator
    const uint32_t off = lane ? prev + 1u : fr.off;
    const bool ends_record = (m >> lane) & 1ull;
    if (ends_record) note_record(st, col + 1u, rec, expect);
    g0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)g0);  // (wave-uniform: the store addresses stay scalar)
    if (rel + lane < slots) {
        store_u32(o.rec + g0, lane, rec);
        store_u32(o.col + g0, lane, col);
        store_u32(o.off + g0, lane, off);
        store_u32(o.len + g0, lane, pos - off);
    }
    fr.rec += (uint32_t)__popcll(m);
    fr.col = m ? (cnt - 1u) - (uint32_t)(63 - __clzll((long long)m)) : fr.col + cnt;
    fr.off = (uint32_t)__builtin_amdgcn_readlane((int)pos, (int)cnt - 1) + 1u;
}

// Per-wave list of the wave's terminators (LDS): entry = position within the
// super-tile << 1 | record-delimiter bit, in field order. A wave with more
// fields in a super-tile lists and writes them in several passes. With 4-byte
// groups the list is shorter, so that four workgroups fit a CU's LDS.
template <int CB>
constexpr int kWaveList = CB == 2 ? 768 : 1024;

// emit: tags from each span's start state; every field's record, column,
// offset and length; the last range writes the unterminated final field and
// the result counts.
//
// Fields are written by waves, 64 consecutive fields per round: each lane first
// lists its terminators in the wave's LDS list, then lane l of a round takes
// field r + l: its record and column follow from a ballot of the record bits
// of the round's fields, its offset from the previous field's terminator (the
// lane before, by DPP). The four output arrays are written with consecutive
// addresses across the lanes.
template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock, (kEmitWavesPerSimd<CB, V8>)) csv_emit_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    __shared__ Pass2Shared<V8, Gm::PAR> sh;
    __shared__ GCarry s_wc[kSpanScratch];
    __shared__ GCarry s_wg[kFastWaves];
    __shared__ uint32_t s_list[kFastWaves][kWaveList<CB>];
    __shared__ uint32_t s_err[kFastWaves];
    __shared__ uint32_t s_cols[4 * kFastWaves];

    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t b = blockIdx.x;
    RecStats rs = rec_stats_none();  // fields per record, over the records this lane's fields end
    uint32_t s0, s1;
    range_of(p, b, s0, s1);
    const Vec ident = fast_ident<V8>(p.nt);
    uint32_t run = p.range_state[b];
    const OutArrays& o = p.out;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    uint32_t* list = s_list[wv];
    load_pass2<CB, V8>(p, sh);
    const GCarryComb gcomb;
    // the count prefix of the range (the input starts in record 0, at column start_col)
    GCarry P = gcomb(GCarry{0u, 0u, p.start_col, 0u}, carries_before(p, b, s_wg));  // (its barrier publishes sh)
    if (b == 0) {  // the first INVALID byte: the smallest of the ranges' (stored by the carries kernel)
        const uint32_t i0 = 2 * threadIdx.x, i1 = i0 + 1;
        uint32_t e = i0 < p.num_ranges ? p.range_err[i0] : kNone;
        if (i1 < p.num_ranges) e = min(e, p.range_err[i1]);
        e = wave_min_defined(e);
        if (lane == 0) s_err[wv] = e;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 1; i < kFastWaves; ++i) e = min(e, s_err[i]);
            p.hdr->err_min = e;
        }
    }

    auto step = [&](auto full_tag, uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) {
        constexpr bool FULL = decltype(full_tag)::value;
        const PairPos c = pair_pos(p, st);
        Vec v0, v1;
        super_vecs<V8>(p, st, in.tvl, ident, v0, v1);
        const uint32_t ts1 = vat(v0, run);
        uint32_t xa = 0, xb = 0;
        const bool ba = kSpeculates<CB, V8> && tile_bits<V8>(p, 2 * st, v0, xa);
        const bool bb = kSpeculates<CB, V8> && tile_bits<V8>(p, 2 * st + 1, v1, xb);
        const bool upper = threadIdx.x >= kFastBlock / 2;
        const int mode = span_mode<CB, V8>(upper ? bb : ba, upper ? vat(v1, ts1) == xb : vat(v0, run) == xa,
                                           in.cvlo, in.cvhi);
        uint64_t T[2], RD[2];
        span_tags<CB, V8, FULL>(p, c, in, run, ts1, sh, T, RD, nullptr, true, mode);
        const SpanCarry sc = span_carry(T, RD, c.abs, s_wc);

        // the wave's fields: super-tile-local indices [wfirst, wend); the state at its first field
        const uint32_t mine = sc.mine, first = sc.wave_excl.nf + sc.excl_nf;
        const uint32_t wfirst = sc.wave_excl.nf;
        const uint32_t wend = __builtin_amdgcn_readlane(first + mine, kWave - 1);
        FieldRun fr{P.nr + sc.wave_excl.nr, col_after(P.col, sc.wave_excl.col, sc.wave_excl.nr),
                    (uint32_t)max(P.lt, sc.wave_excl.lt)};
        const uint32_t st_abs = st * (uint32_t)(2 * kFastTile);
        const uint32_t rel0 = c.abs - st_abs;
        for (uint32_t w0 = wfirst; w0 < wend; w0 += kWaveList<CB>) {
            const uint32_t w1 = min(w0 + (uint32_t)kWaveList<CB>, wend);
            // (1) each lane lists its terminators that fall in [w0, w1)
            {
                const uint32_t tw[4] = {(uint32_t)T[0], (uint32_t)(T[0] >> 32), (uint32_t)T[1], (uint32_t)(T[1] >> 32)};
                const uint32_t rw[4] = {(uint32_t)RD[0], (uint32_t)(RD[0] >> 32), (uint32_t)RD[1],
                                        (uint32_t)(RD[1] >> 32)};
                list_terminators<4>(list, tw, rw, rel0, first, mine, w0, w1);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // (2) rounds of 64 fields: the round's output slices are uniform base pointers,
            // each lane stores at its own 4-byte offset
            const uint32_t slots = slots_from(o.cap, (uint64_t)P.nf + w0, w1 - w0);
            for (uint32_t r = w0; r < w1; r += kWave) {
                const uint32_t cnt = min((uint32_t)kWave, w1 - r);
                field_round(o, P.nf + r, r - w0, slots, cnt, list[r - w0 + min(lane, cnt - 1u)], st_abs, lane, lt_mask,
                            fr, rs, p.expect_cols);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        P = gcomb(P, sc.total);
        run = vat(v1, ts1);
    };
    walk_supers<CB, V8>(
        p, s0, s1, [&](uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) { step(std::true_type{}, st, in, it); },
        [&](uint32_t st, const IdxIn<CB, V8>& in, uint32_t it) { step(std::false_type{}, st, in, it); });
    if (threadIdx.x == 0 && b == p.num_ranges - 1) {
        const uint32_t final_field = (p.partial || p.hdr->last_rec) ? 0u : 1u;
        p.hdr->tail_start = P.lt;
        p.hdr->tail_col = P.col;
        if (final_field && P.nf < o.cap) {
            o.rec[P.nf] = P.nr;
            o.col[P.nf] = P.col;
            o.off[P.nf] = P.lt;
            o.len[P.nf] = p.n - P.lt;
        }
        if (final_field) note_record(rs, P.col + 1u, P.nr, p.expect_cols);  // the final field ends the last record
        p.hdr->n_fields = (uint64_t)P.nf + final_field;
        p.hdr->n_records = (uint64_t)P.nr + final_field;
    }
    // the range's per-record counts, into the call's
    publish_rec_stats<kFastWaves>(rs.cmin, rs.cmax, rs.bad, rs.fbad, s_cols, &p.hdr->cols_min, &p.hdr->cols_max,
                                  &p.hdr->bad_records, &p.hdr->first_bad);
}

// ================================================================ fused single pass
//
// One kernel runs every step of the method per 32 KiB tile: classify, the
// chunk vectors and their block scan, the tile's start state by a decoupled
// look-back over the tile vectors, pass 2 from each chunk's start state, the
// block scan of the count carries, the tile's count prefix by a second
// look-back, and the field emission. The input is read once and the fields are
// written once; nothing per byte or per chunk goes to memory.
//
// Workgroups are persistent and take tiles in increasing order from an atomic
// counter, so a tile only ever waits for tiles that running workgroups already
// hold, and a workgroup never waits for one that is not resident.
//
// Each workgroup runs a three-stage software pipeline over its tiles. One
// round does phase 1 of its newest tile (classify, chunk vectors, block scan,
// publish the tile's vector aggregate), phase 2 of the previous one (vector
// look-back, pass 2, count carries, publish their aggregate) and phase 3 of the
// one before (count look-back, fields). A look-back thus reads statuses that
// were published about a round earlier, instead of waiting for tiles that
// started at the same time; and a tile's aggregate is published right after it
// is taken, never behind a wait, so waits do not feed back into later tiles.

// Count-carry statuses. Aggregate (tile-local): nf | nr << 16 (a 32 KiB tile
// has at most 2^15 of each), col (absolute when nr > 0), lt. Inclusive prefix:
// nf, nr, col, lt, all absolute.
__device__ __forceinline__ void publish_gagg(StatB& s, const GCarry& c, uint32_t epoch)
{
    st_relaxed(&s.agg[0], ew(epoch, c.nf | (c.nr << 16)));
    st_relaxed(&s.agg[1], ew(epoch, c.col));
    st_relaxed(&s.agg[2], ew(epoch, c.lt));
}
__device__ __forceinline__ void publish_gincl(StatB& s, const GCarry& c, uint32_t epoch)
{
    st_relaxed(&s.incl[0], ew(epoch, c.nf));
    st_relaxed(&s.incl[1], ew(epoch, c.nr));
    st_relaxed(&s.incl[2], ew(epoch, c.col));
    st_relaxed(&s.incl[3], ew(epoch, c.lt));
}

// count-carry status of one tile: the seven words are loaded at once
struct GCarryPoll {
    const StatB* stat;
    uint32_t epoch;
    struct Raw {
        uint64_t i[4], a[3];
    };
    __device__ __forceinline__ Raw load(int64_t u) const
    {
        const StatB& s = stat[u];
        Raw r;
#pragma unroll
        for (int k = 0; k < 4; ++k) r.i[k] = ld_relaxed(&s.incl[k]);
#pragma unroll
        for (int k = 0; k < 3; ++k) r.a[k] = ld_relaxed(&s.agg[k]);
        return r;
    }
    __device__ __forceinline__ uint32_t decode(const Raw& r, GCarry& out) const
    {
        if (ew_ok(r.i[0], epoch) && ew_ok(r.i[1], epoch) && ew_ok(r.i[2], epoch) && ew_ok(r.i[3], epoch)) {
            out = {(uint32_t)r.i[0], (uint32_t)r.i[1], (uint32_t)r.i[2], (uint32_t)r.i[3]};
            return kFlagIncl;
        }
        if (ew_ok(r.a[0], epoch) && ew_ok(r.a[1], epoch) && ew_ok(r.a[2], epoch)) {
            const uint32_t x0 = (uint32_t)r.a[0];
            out = {x0 & 0xffffu, x0 >> 16, (uint32_t)r.a[1], (uint32_t)r.a[2]};
            return kFlagAgg;
        }
        return 0;
    }
};

// Vector statuses: the aggregate is the tile's packed vector, the inclusive
// prefix the state after the tile, read back as a constant vector.
struct FVecPoll {
    const uint64_t* stat;
    uint32_t epoch;
    using Raw = uint64_t;
    __device__ __forceinline__ Raw load(int64_t u) const { return ld_relaxed(&stat[u]); }
    __device__ __forceinline__ uint32_t decode(Raw w, Vec& out) const
    {
        const uint32_t f = status_flag(w, epoch);
        if (f == kFlagAgg) out = vunpack(status_payload(w));
        if (f == kFlagIncl) {
            const uint32_t k = status_payload(w) * 0x01010101u;
            out = {k, k};
        }
        return f;
    }
};

// pass 2 over a ragged chunk (the input's last bytes), one byte at a time
template <int CB>
__device__ void pass2_ragged_chunk(const FastParams& p, const ChunkPos& c, uint32_t s, uint32_t nt,
                                   const uint8_t* s_nxt, const uint8_t* s_tag, uint64_t& T, uint64_t& RD,
                                   uint32_t& err)
{
    T = RD = 0;
    for (uint32_t j = 0; j < c.my_len; ++j) {
        const uint32_t code = classify1<CB>(p.in[c.chunk_abs + j], p);
        const uint32_t row = min(s, nt);
        const uint32_t t = s_tag[row * 16 + code];
        s = s_nxt[row * 16 + code];
        T |= (uint64_t)(t == PPR_TAG_FIELD || t == PPR_TAG_RECORD) << j;
        RD |= (uint64_t)(t == PPR_TAG_RECORD) << j;
        if (t == PPR_TAG_INVALID && err == kNone) err = c.chunk_abs + j;
    }
}

constexpr int kFusedList = 1024;  // per-wave terminator list entries (LDS)
constexpr int kFusedWavesPerSimd = 4;  // 2 resident workgroups per CU (8 waves each): the register budget the kernel is cut to

template <int CB, bool V8>
struct FusedShared {
    uint32_t t1[V8 ? 2 * Geo<CB>::E : Geo<CB>::E];
    Pass2Shared<V8, Geo<CB>::PAR> p2;
    Vec wv[kFastWaves];
    Vec pv[kFastWaves];
    GCarry wc[kSpanScratch];
    GCarry pc[kFastWaves];
    int first[kFastWaves];
    uint32_t next, state, last_rec;
    uint32_t cols[4 * kFastWaves];
    uint32_t list[kFastWaves][kFusedList];
};

template <int CB, bool V8>
__global__ void __launch_bounds__(kFastBlock, kFusedWavesPerSimd) csv_fused_kernel(FastParams p)
{
    using Gm = Geo<CB>;
    constexpr int NI = Gm::NI, ND = Gm::ND, NP = Gm::NP;
    __shared__ FusedShared<CB, V8> sh;

    const int tid = threadIdx.x;
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t nt = p.nt, num_tiles = p.num_tiles;
    const OutArrays& o = p.out;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const GCarryComb gcomb;
    RecStats rs = rec_stats_none();  // fields per record, over the records this lane's fields end
    const GCarry zero{0u, 0u, 0u, 0u};
    if (tid == 0) {
        sh.next = atomicAdd(&p.hdr->tile_counter, 1u);
        sh.last_rec = 0;
    }
    for (int i = tid; i < (V8 ? 2 : 1) * Gm::E; i += kFastBlock) sh.t1[i] = p.tabs[i];
    load_pass2<CB, V8>(p, sh.p2);
    __syncthreads();
    const Vec ident = fast_ident<V8>(nt);

    // this thread's 64 bytes of a tile, if its chunk is full (16-byte loads)
    auto load_chunk = [&](uint32_t t, uint32_t (&w)[ND]) {
        const uint32_t pos = t * (uint32_t)kFastTile + (uint32_t)tid * (uint32_t)kFastChunk;
        if (pos + (uint32_t)kFastChunk <= p.n) {
            const uint4* src = reinterpret_cast<const uint4*>(p.in + pos);
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

    // The pipeline: t0 in phase 1 (bytes loaded), t1 in phase 2, t2 in phase 3
    // (num_tiles: no tile). Each tile's state is handed from phase to phase in
    // registers.
    uint32_t t0 = sh.next, t1 = num_tiles, t2 = num_tiles;
    uint32_t w[ND];
    if (t0 < num_tiles) load_chunk(t0, w);
    uint32_t pw1[NP];  // phase 2 input: group indices, vector of the tile's earlier chunks, tile vector
    Vec excl1 = ident, tot1 = ident;
    uint64_t T2 = 0, RD2 = 0;  // phase 3 input: tag bitmaps, count carries, end state
    SpanCarry sc2{0u, 0u, zero, zero};
    uint32_t end2 = 0;
#pragma unroll
    for (int q = 0; q < NP; ++q) pw1[q] = 0;

    const FVecPoll vpoll{p.stat_vec, p.epoch};
    const GCarryPoll cpoll{p.stat_carry, p.epoch};
    while (t0 < num_tiles || t1 < num_tiles || t2 < num_tiles) {
        // ---- phase 1 (tile t0): classify, chunk vectors, block scan, aggregate
        uint32_t pw0[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q) pw0[q] = 0;
        Vec excl0 = ident, tot0 = ident;
        uint32_t tn = num_tiles;
        if (t0 < num_tiles) {
            if (tid == 0) sh.next = atomicAdd(&p.hdr->tile_counter, 1u);  // read after the block scan's barrier
            const ChunkPos c = chunk_pos(p.n, t0);
            Vec v = ident;
            if (c.full) {
                uint32_t ia[NI];
                chunk_codes<CB>(w, p, ia, pw0);
                v = tree_vector<CB, V8>(ia, sh.t1);
            } else if (c.my_len) {
                v = ragged_vector<CB, V8>(p, c, ident, sh.p2.nxt);
            }
            block_scan<kFastWaves>(v, ident, excl0, tot0, sh.wv, VecComb<V8>{});
            tn = sh.next;
            if (tid == 0)
                st_relaxed(&p.stat_vec[t0], t0 == 0 ? status_word(p.epoch, kFlagIncl, vat(tot0, p.start_code))
                                                    : status_word(p.epoch, kFlagAgg, vpack(tot0)));
        }

        // ---- phase 2 (tile t1): start state, pass 2, count carries, their aggregate
        uint64_t T1 = 0, RD1 = 0;
        SpanCarry sc1{0u, 0u, zero, zero};
        uint32_t end1 = 0;
        if (t1 < num_tiles) {
            if (t1 == 0) {
                if (tid == 0) sh.state = p.start_code;
            } else {
                const Vec acc = lookback_pre<kFastWaves>(t1, ident, vpoll, VecComb<V8>{}, sh.pv, sh.first,
                                                         &p.hdr->fault, look_first<kFastWaves>(t1, vpoll));
                if (tid == 0) {
                    const uint32_t st = vat(acc, 0);  // a constant vector: the state after all earlier tiles
                    sh.state = st;
                    st_relaxed(&p.stat_vec[t1], status_word(p.epoch, kFlagIncl, vat(tot1, st)));
                }
            }
            __syncthreads();
            const uint32_t ts = sh.state;
            end1 = vat(tot1, ts);
            const ChunkPos c = chunk_pos(p.n, t1);
            const uint32_t s = vat(excl1, ts);
            uint32_t err = kNone;
            uint64_t T[1] = {0}, RD[1] = {0};
            if (c.full) {
                const uint32_t any = pass2_run<CB, 1>(pw1, s, nt, sh.p2.t2, T, RD);
                if (any & kP2Invalid) err = first_invalid<CB, 1>(pw1, s, nt, sh.p2.t2, c.chunk_abs);
            } else if (c.my_len) {
                pass2_ragged_chunk<CB>(p, c, s, nt, sh.p2.nxt, sh.p2.tag, T[0], RD[0], err);
            }
            wave_lower_min(&p.hdr->err_min, err);
            if (c.my_len && c.chunk_abs + c.my_len == p.n)
                sh.last_rec = (uint32_t)((RD[0] >> (c.my_len - 1)) & 1u);
            sc1 = span_carry<1>(T, RD, c.chunk_abs, sh.wc);
            T1 = T[0];
            RD1 = RD[0];
            if (tid == 0) {
                if (t1 == 0)  // the input starts in record 0 at column start_col
                    publish_gincl(p.stat_carry[0], gcomb(GCarry{0u, 0u, p.start_col, 0u}, sc1.total), p.epoch);
                else
                    publish_gagg(p.stat_carry[t1], sc1.total, p.epoch);
            }
        }

        // ---- phase 3 (tile t2): count prefix, fields
        if (t2 < num_tiles) {
            GCarry P{0u, 0u, p.start_col, 0u};
            if (t2 != 0) {
                P = lookback_pre<kFastWaves>(t2, zero, cpoll, gcomb, sh.pc, sh.first, &p.hdr->fault,
                                             look_first<kFastWaves>(t2, cpoll));
                if (tid == 0) publish_gincl(p.stat_carry[t2], gcomb(P, sc2.total), p.epoch);
            }
            const uint32_t tile_start = t2 * (uint32_t)kFastTile;
            // the wave lists its terminators, then writes 64 fields per round
            uint32_t* list = sh.list[wv];
            const uint32_t mine = sc2.mine, first = sc2.wave_excl.nf + sc2.excl_nf;
            const uint32_t wfirst = sc2.wave_excl.nf;
            const uint32_t wend = __builtin_amdgcn_readlane(first + mine, kWave - 1);
            FieldRun fr{P.nr + sc2.wave_excl.nr, col_after(P.col, sc2.wave_excl.col, sc2.wave_excl.nr),
                        (uint32_t)max(P.lt, sc2.wave_excl.lt)};
            const uint32_t rel0 = (uint32_t)tid * (uint32_t)kFastChunk;
            for (uint32_t w0 = wfirst; w0 < wend; w0 += kFusedList) {
                const uint32_t w1 = min(w0 + (uint32_t)kFusedList, wend);
                {
                    const uint32_t tw[2] = {(uint32_t)T2, (uint32_t)(T2 >> 32)};
                    const uint32_t rw[2] = {(uint32_t)RD2, (uint32_t)(RD2 >> 32)};
                    list_terminators<2>(list, tw, rw, rel0, first, mine, w0, w1);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const uint32_t slots = slots_from(o.cap, (uint64_t)P.nf + w0, w1 - w0);
                for (uint32_t r = w0; r < w1; r += kWave) {
                    const uint32_t cnt = min((uint32_t)kWave, w1 - r);
                    field_round(o, P.nf + r, r - w0, slots, cnt, list[r - w0 + min(lane, cnt - 1u)], tile_start,
                                lane, lt_mask, fr, rs, p.expect_cols);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            // the input's last tile: the unterminated final field and the results
            if (t2 == num_tiles - 1 && tid == 0) {
                const GCarry I = gcomb(P, sc2.total);
                const uint32_t final_field = (p.partial || sh.last_rec) ? 0u : 1u;
                p.hdr->tail_start = I.lt;
                p.hdr->tail_col = I.col;
                if (final_field && I.nf < o.cap) {
                    o.rec[I.nf] = I.nr;
                    o.col[I.nf] = I.col;
                    o.off[I.nf] = I.lt;
                    o.len[I.nf] = p.n - I.lt;
                }
                if (final_field) note_record(rs, I.col + 1u, I.nr, p.expect_cols);  // the final field ends the last record
                const uint32_t e = min(end2, 8u);
                p.hdr->n_fields = (uint64_t)I.nf + final_field;
                p.hdr->n_records = (uint64_t)I.nr + final_field;
                p.hdr->end_state = p.state_of[e];
                p.hdr->error_pos =
                    (p.partial || ((p.accept_codes >> e) & 1u)) ? (int64_t)-1 : (int64_t)p.n;  // before err_min
            }
        }

        // hand the tiles on
        t2 = t1;
        T2 = T1;
        RD2 = RD1;
        sc2 = sc1;
        end2 = end1;
        t1 = t0;
#pragma unroll
        for (int q = 0; q < NP; ++q) pw1[q] = pw0[q];
        excl1 = excl0;
        tot1 = tot0;
        t0 = tn;
        if (t0 < num_tiles) load_chunk(t0, w);
        __syncthreads();  // sh.next and the scan scratch are rewritten next round
    }
    // the workgroup's per-record counts, into the call's
    publish_rec_stats<kFastWaves>(rs.cmin, rs.cmax, rs.bad, rs.fbad, sh.cols, &p.hdr->cols_min, &p.hdr->cols_max,
                                  &p.hdr->bad_records, &p.hdr->first_bad);
}

// workgroups of the codes kernel (all resident at once: 4 per CU)
constexpr uint32_t kCodesGrid = 1024;

template <int CB, bool V8>
static void launch(const FastParams& f, const ppr_parse_opts_t* o, hipStream_t s)
{
    const dim3 grid(f.num_ranges), block(kFastBlock);
    stage_event(o, 0, s);
    hipLaunchKernelGGL((csv_codes_kernel<CB, V8>), dim3(std::min<uint32_t>(f.num_tiles, kCodesGrid)), block, 0, s, f);
    hipLaunchKernelGGL((csv_range_vec_kernel<V8>), grid, dim3(kWave), 0, s, f);
    stage_event(o, 1, s);
    hipLaunchKernelGGL((csv_carries_kernel<CB, V8>), grid, block, 0, s, f);
    stage_event(o, 2, s);
    hipLaunchKernelGGL((csv_emit_kernel<CB, V8>), grid, block, 0, s, f);
    stage_event(o, 3, s);
}

// Persistent grid of the fused kernel: as many workgroups as the device holds at
// once (more would only wait for a slot; fewer would leave CUs idle).
template <int CB, bool V8>
static uint32_t fused_grid()
{
    static int per_cu = 0;
    static int cus = 0;
    if (per_cu == 0) {
        int dev = 0, b = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, csv_fused_kernel<CB, V8>, kFastBlock, 0) == hipSuccess &&
            b > 0 && n > 0) {
            cus = n;
            per_cu = b;
        } else {
            cus = 256;
            per_cu = 1;
        }
    }
    return (uint32_t)(cus * per_cu);
}

template <int CB, bool V8>
static void launch_fused(const FastParams& f, const ppr_parse_opts_t* o, hipStream_t s)
{
    stage_event(o, 0, s);
    hipLaunchKernelGGL((csv_fast_tables_kernel<CB, V8>), dim3(clear_grid((uint64_t)f.num_tiles * (8 + sizeof(StatB)))),
                       dim3(256), 0, s, f);
    stage_event(o, 1, s);
    const uint32_t grid = std::min<uint32_t>(f.num_tiles, fused_grid<CB, V8>());
    hipLaunchKernelGGL((csv_fused_kernel<CB, V8>), dim3(grid), dim3(kFastBlock), 0, s, f);
    stage_event(o, 2, s);
}

int launch_csv_fast(const FastParams& f, int cb, bool v8, const ppr_parse_opts_t* o, hipStream_t s)
{
    if (f.path == PPR_PATH_FUSED) {
        if (cb == 2) v8 ? launch_fused<2, true>(f, o, s) : launch_fused<2, false>(f, o, s);
        else if (cb == 3) v8 ? launch_fused<3, true>(f, o, s) : launch_fused<3, false>(f, o, s);
        else v8 ? launch_fused<4, true>(f, o, s) : launch_fused<4, false>(f, o, s);
    } else {
        if (cb == 2) v8 ? launch<2, true>(f, o, s) : launch<2, false>(f, o, s);
        else if (cb == 3) v8 ? launch<3, true>(f, o, s) : launch<3, false>(f, o, s);
        else v8 ? launch<4, true>(f, o, s) : launch<4, false>(f, o, s);
    }
    return hipGetLastError() == hipSuccess ? PPR_OK : PPR_EHIP;
}

}  // namespace ppr
