// Types and helpers shared by the CSV kernels (generic and fast paths).
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", Sec. 3: per-chunk state-transition vectors (Fig. 2), their composite
// and exclusive scan, re-simulation and tagging, record counts and
// relative/absolute column offsets (Fig. 4).
#pragma once

#include "ppr.h"
#include "ppr_device.h"
#include "ppr_host.h"
#include "ppr_slots.h"

namespace ppr {

constexpr int kBlock = 1024;     // generic path: threads per tile (a look-back round covers as many tiles as the
                                 // device holds at once: 2 workgroups per CU)
constexpr int kWaves = kBlock / kWave;
constexpr int kFastBlock = 512;  // fast path: threads per tile
constexpr int kFastWaves = kFastBlock / kWave;
constexpr int kMaxChunk = 64;
constexpr int kFastChunk = 64;   // fast path: bytes per thread
constexpr int kFastTile = kFastBlock * kFastChunk;
constexpr uint32_t kNone = 0xffffffffu;
constexpr uint32_t kAbs = 0xffu;                // state code of the absorbing state (fast path)
constexpr int kTabWords = 2 * 256 + 2 * 9 * 256;  // largest step tables (pass 1 + pass 2), 32-bit words

// Carries of a run of bytes [ParPaRaw Sec. 3, offsets, Fig. 4]:
//   nf terminators, nr record delimiters,
//   column offset handed to what follows: absolute (a record delimiter was seen:
//     field delimiters after the last one) or relative (field delimiters seen),
//   lt = 1 + position of the last terminator (0: none),
//   err = first INVALID byte (kNone: none; only the generic path scans it).
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

struct CarryComb {
    __device__ Carry operator()(const Carry& a, const Carry& b) const { return carry_op(a, b); }
};

// Composite of vectors; with V8 false only entries 0-3 are live (lo).
template <bool V8>
__device__ __forceinline__ Vec comp(Vec a, Vec b)
{
    if constexpr (V8) return compose(a, b);
    else return {perm(b.lo, b.lo, a.lo), 0xffffffffu};  // (entries 4-7 are never read with 4 tracked states)
}

template <bool V8>
struct VecComb {
    __device__ Vec operator()(const Vec& a, const Vec& b) const { return comp<V8>(a, b); }
};

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

// Fields per record, over the records whose last field a lane writes
// [ParPaRaw, "Inferring or validating number of columns"]: the fewest and the
// most, and, given an expected number (expect > 0), how many records have
// another number and the index of the first of them.
struct RecStats {
    uint32_t cmin, cmax, bad, fbad;
};

__device__ __forceinline__ RecStats rec_stats_none() { return {kNone, 0u, 0u, kNone}; }

// record `rec` ends with this field and has `fields` fields
__device__ __forceinline__ void note_record(RecStats& st, uint32_t fields, uint32_t rec, uint32_t expect)
{
    st.cmin = min(st.cmin, fields);
    st.cmax = max(st.cmax, fields);
    const bool bad = expect != 0u && fields != expect;
    st.bad += bad ? 1u : 0u;
    st.fbad = bad ? min(st.fbad, rec) : st.fbad;
}

struct OutArrays {
    uint32_t* rec;
    uint32_t* col;
    uint32_t* off;
    uint32_t* len;
    uint64_t cap;
};

// ---------------------------------------------------------------- fast path
//
// Symbol codes: the catch-all class has code 2^CB - 1; every other class a
// smaller code. States are coded 0..nt-1 (tracked) and kAbs (absorbing). The
// table index of a group of G symbols is c0 + 4 c1 + 16 c2 + 64 c3 (CB = 2,
// G = 4) or c0 + 16 c1 (CB = 3 or 4, G = 2); one byte per group.
struct FastParams {
    const uint8_t* in;
    uint32_t n, num_tiles;
    uint32_t start_code, accept_codes;  // bit i: tracked code i accepting; bit 8: absorbing state accepting
    uint32_t nt;                        // tracked states
    SlotTables slots;                   // symbol classification (ppr_slots.h)
    OutArrays out;
    WsHeader* hdr;
    uint32_t* tabs;        // step tables built for this call
    uint32_t num_super;    // super-tiles: pairs of tiles (the last may hold one)
    uint32_t num_ranges;   // workgroups of the streaming kernels, each owning a contiguous run of super-tiles
    uint8_t* idx;          // group indices, NI bytes per full chunk
    uint32_t* cvec_lo;     // per even chunk: vector of the tile's bytes before it (entries 0-3)
    uint32_t* cvec_hi;     // (entries 4-7)
    uint64_t* tile_vec;    // per tile: state-transition vector (lo | hi << 32)
    uint64_t* range_vec;   // per range: composite of its tile vectors
    uint32_t* range_state; // per range: state code before its first byte
    uint4* range_carry;    // per range: nf, nr, col (absolute when nr > 0), lt
    uint32_t* range_err;   // per range: its first INVALID byte (kNone: none)
    uint64_t* stat_vec;    // fused path: per tile, vector look-back status
    StatB* stat_carry;     // fused path: per tile, count-carry look-back status
    uint32_t* spec;        // streaming path (the same memory): per tile, the carry of its agreed chunks (8 words)
    uint32_t epoch;        // fused path: call epoch carried by the status words
    uint32_t path;         // PPR_PATH_* the call runs
    uint32_t expect_cols;  // expected fields per record (0: none)
    uint32_t start_col;    // column of the field open at the input's start (0: a record starts there)
    uint32_t partial;      // more input follows: no final field, the end state may be non-accepting
    uint32_t quiet_abs;    // the absorbing state tags no byte FIELD or RECORD (tag bitmaps may replace indices)
    uint8_t state_of[16];  // DFA state of each code (index 8: absorbing)
    uint8_t nxt[9][16];    // [state code, row nt = absorbing][symbol code] -> next code
    uint8_t tag[9][16];
};

constexpr uint32_t kMaxRanges = 1024;

struct FastLayout {
    uint64_t tiles, tabs, tile_vec, range_vec, range_state, range_carry, range_err, stat_vec, stat_carry, cvec_lo,
        cvec_hi, idx, total;
};

// workspace of the fast path for n bytes (idx sized for 2-byte groups)
inline FastLayout fast_layout(uint64_t n)
{
    FastLayout L;
    L.tiles = (n + kFastTile - 1) / kFastTile;
    L.tabs = 256;
    L.tile_vec = align_up(L.tabs + kTabWords * 4, 256);
    L.range_vec = align_up(L.tile_vec + L.tiles * 8, 256);
    L.range_state = align_up(L.range_vec + kMaxRanges * 8, 256);
    L.range_carry = align_up(L.range_state + kMaxRanges * 4, 256);
    L.range_err = align_up(L.range_carry + kMaxRanges * 16, 256);
    L.stat_vec = align_up(L.range_err + kMaxRanges * 4, 256);
    L.stat_carry = align_up(L.stat_vec + L.tiles * 8, 256);
    L.cvec_lo = align_up(L.stat_carry + L.tiles * sizeof(StatB), 256);
    L.cvec_hi = align_up(L.cvec_lo + L.tiles * (kFastBlock / 2) * 4, 256);
    L.idx = align_up(L.cvec_hi + L.tiles * (kFastBlock / 2) * 4, 256);
    L.total = align_up(L.idx + L.tiles * (uint64_t)kFastTile / 2, 256);
    return L;
}

// workspace of the fused path alone (header, step tables, look-back statuses;
// the streaming kernels' arrays are left out: their offsets repeat the last one)
inline FastLayout fused_layout(uint64_t n)
{
    FastLayout L;
    L.tiles = (n + kFastTile - 1) / kFastTile;
    L.tabs = 256;
    L.stat_vec = align_up(L.tabs + kTabWords * 4, 256);
    L.stat_carry = align_up(L.stat_vec + L.tiles * 8, 256);
    L.total = align_up(L.stat_carry + L.tiles * sizeof(StatB), 256);
    L.tile_vec = L.range_vec = L.range_state = L.range_carry = L.range_err = L.cvec_lo = L.cvec_hi = L.idx = L.total;
    return L;
}

// Enqueue the fast path (CB symbol-code bits, V8: more than 4 tracked states).
int launch_csv_fast(const FastParams& f, int cb, bool v8, const ppr_parse_opts_t* opts, hipStream_t s);

// Enqueue one parse into the workspace d_ws (see ppr_parse_async); compact:
// d_ws is a fixed scratch buffer, so only the single-pass paths (fused kernel
// for table-driven inputs, else the generic kernel) are used.
int parse_enqueue(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                  const ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream,
                  bool compact);

}  // namespace ppr
