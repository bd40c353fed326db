// Streaming lexer kernels on gfx950.
//
// Method: "Lexing on the GPU: the scan is the easy part", section "A lexer is a
// prefix scan" (identifiers of transition functions, composed through the k x k
// merge table; the state after each prefix is an inclusive scan) and section
// "Does it produce the same tokens?" (a flag on a merged identifier ends a token
// before that byte; its kind is the final-state entry of the state before it).
//
// Four kernels, none of which waits on another workgroup:
//   lex_ids_kernel    pass 1: each thread folds its 40-byte chunk from the
//                     identity through the fold rows held in LDS (identifiers
//                     whose fold rows are equal share a row), a block scan of
//                     the chunk identifiers under the merge table; stores each
//                     chunk's tile-exclusive identifier and each tile's.
//   lex_range_kernel  one wave per range (a contiguous run of tiles) composes
//                     its tile identifiers.
//   lex_count_kernel  per range, in tile order: each chunk's start identifier
//                     (the range prefix, the tiles before, the chunk's tile
//                     prefix), pass 2 through the minimal automaton in LDS,
//                     boundary counts and the last boundary, one per range.
//   lex_emit_kernel   the same pass 2 with token kinds, a block scan of the
//                     counts, and the tokens written by waves, 64 per round
//                     with consecutive addresses; the last range writes the
//                     final token and the count.
// The device-wide scans run over the range aggregates only, in each workgroup's
// prologue.
#include "ppr_lex_common.h"
#include "ppr_scan.h"

namespace ppr {

// a earlier, b later
struct LexIdComb {
    const uint16_t* merge;
    uint32_t k, id_mask;
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const
    {
        return (uint32_t)merge[(uint64_t)a * k + b] & id_mask;
    }
};

// boundaries counted, the last one's position (0: none; position 0 is never one)
struct LexTok {
    uint32_t nt, lb;
};

struct LexTokComb {
    __device__ LexTok operator()(const LexTok& a, const LexTok& b) const { return {a.nt + b.nt, max(a.lb, b.lb)}; }
};

constexpr int kLexWords = kLexFastChunk / 4;  // dwords per chunk
constexpr int kLexList = 1024;                // per-wave token list entries (LDS)

__device__ __forceinline__ uint32_t chunk_byte(const uint32_t (&w)[kLexWords], int j)
{
    return (w[j >> 2] >> (8 * (j & 3))) & 0xffu;
}

// A thread's chunk: full (8-byte loads) or the input's ragged end (bytes < len).
template <bool FULL>
__device__ __forceinline__ void load_lex_chunk(const uint8_t* src, uint32_t len, uint32_t (&w)[kLexWords])
{
    if constexpr (FULL) {
        const uint2* s = reinterpret_cast<const uint2*>(src);
#pragma unroll
        for (int q = 0; q < kLexWords / 2; ++q) {
            const uint2 x = s[q];
            w[2 * q] = x.x;
            w[2 * q + 1] = x.y;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kLexWords; ++q) w[q] = 0;
#pragma unroll
        for (int j = 0; j < kLexFastChunk; ++j) {
            const uint32_t b = (uint32_t)j < len ? (uint32_t)src[j] : 0u;
            w[j >> 2] |= b << (8 * (j & 3));
        }
    }
}

// u16 at byte a of an LDS table
__device__ __forceinline__ uint32_t lds_u16_at(const uint16_t* base, uint32_t a)
{
    return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + a);
}

// Pass 1: the chunk's identifier, folded from the identity. All but the last
// byte step through the fold rows in LDS (entries: the next row times m); the
// last byte reads the identifier itself from the same row in global memory.
// s_col2 holds each byte's column times 2, and the rows lie at LDS address 0,
// so a step's address is one v_lshl_add of the entry and the column.
template <bool FULL>
__device__ __forceinline__ uint32_t fold_lex_chunk(const LexFastParams& p, const uint32_t (&w)[kLexWords], uint32_t len,
                                                   const uint16_t* s_rows, const uint8_t* s_col2)
{
    if (!FULL && len == 0) return p.identity;
    uint32_t r = p.row0, c = 0;
#pragma unroll
    for (int j = 0; j < kLexFastChunk; ++j) {
        const uint32_t cj = s_col2[chunk_byte(w, j)];
        if (FULL ? j + 1 < kLexFastChunk : (uint32_t)j + 1u < len) r = lds_u16_at(s_rows, 2u * r + cj);
        else if (FULL || (uint32_t)j + 1u == len) c = cj >> 1;
    }
    return p.row_id[r + c];
}

// Pass 1 for N full chunks at once: their folds step in lockstep, so each
// step's N row reads are independent and wait on the LDS once.
template <int N>
__device__ __forceinline__ void fold_lex_chunks(const LexFastParams& p, const uint32_t (&w)[N][kLexWords],
                                                const uint16_t* s_rows, const uint8_t* s_col2, uint32_t (&id)[N])
{
    uint32_t r[N];
#pragma unroll
    for (int k = 0; k < N; ++k) r[k] = p.row0;
#pragma unroll
    for (int j = 0; j + 1 < kLexFastChunk; ++j)
#pragma unroll
        for (int k = 0; k < N; ++k) r[k] = lds_u16_at(s_rows, 2u * r[k] + s_col2[chunk_byte(w[k], j)]);
#pragma unroll
    for (int k = 0; k < N; ++k) id[k] = p.row_id[r[k] + (s_col2[chunk_byte(w[k], kLexFastChunk - 1)] >> 1)];
}

// Pass 2 from the automaton state whose row starts at byte q4 of the step
// table: bit j of the result is set when a token ends before byte j. Entries
// are addressed by byte: entry = the successor's row offset | flag << 16 |
// kind of the state before the byte << 24; s_col4 holds each byte's column
// times 4 (one byte each: the 256-byte table is one word per LDS bank, so its
// reads never conflict). The step table sits at LDS address 0, so a step is
// one add of the entry's low half and the column (v_add_u32 with a 16-bit
// source select) and one LDS read. A full chunk reads all its columns before
// the chain of steps (they do not depend on the state) and gathers the flag
// bytes, and with kinds the kind bytes, four per word by v_perm; the kind words
// go to kinds32 (garbage where no token ends: only flagged bytes' kinds are
// read).
template <bool KINDS>
__device__ __forceinline__ uint64_t lex_pass2_full(const uint32_t (&w)[kLexWords], uint32_t q4, const uint32_t* s_step,
                                                   const uint8_t* s_col4, uint32_t* kinds32)
{
    uint32_t c[kLexFastChunk];
#pragma unroll
    for (int j = 0; j < kLexFastChunk; ++j) c[j] = s_col4[chunk_byte(w, j)];
    uint32_t e = q4, fw = 0, kw = 0, b0 = 0, b1 = 0;
#pragma unroll
    for (int j = 0; j < kLexFastChunk; ++j) {
        e = lds_at(s_step, (e & 0xffffu) + c[j]);
        const int i = j & 3;
        const uint32_t keep = 0x03020100u & ~(0xffu << (8 * i));
        fw = perm(e, fw, keep | (6u << (8 * i)));  // byte i <- the entry's flag byte
        if (KINDS) kw = perm(e, kw, keep | (7u << (8 * i)));  // byte i <- the entry's kind byte
        if (i == 3) {
            const uint32_t nib = __builtin_amdgcn_udot4(fw, 0x08040201u, 0u, false);  // flag bytes (0/1) -> 4 bits
            if (j < 32) b0 |= nib << (j - 3);
            else b1 |= nib << (j - 35);
            if (KINDS) kinds32[j >> 2] = kw;
        }
    }
    return (uint64_t)b0 | ((uint64_t)b1 << 32);
}

// Pass 2 over the input's ragged last chunk (bytes < len), one byte at a time.
template <bool KINDS>
__device__ __forceinline__ uint64_t lex_pass2_ragged(const uint32_t (&w)[kLexWords], uint32_t len, uint32_t q4,
                                                     const uint32_t* s_step, const uint8_t* s_col4, uint8_t* kinds)
{
    uint64_t bits = 0;
    uint32_t e = q4;
    for (uint32_t j = 0; j < len; ++j) {
        e = lds_at(s_step, (e & 0xffffu) + (uint32_t)s_col4[chunk_byte(w, (int)j)]);
        const uint32_t f = (e >> 16) & 1u;
        if (KINDS && f) kinds[j] = (uint8_t)(e >> 24);
        bits |= (uint64_t)f << j;
    }
    return bits;
}

__device__ __forceinline__ void lex_range_of(const LexFastParams& p, uint32_t b, uint32_t& t0, uint32_t& t1)
{
    t0 = (uint32_t)((uint64_t)b * p.num_tiles / p.num_ranges);
    t1 = (uint32_t)((uint64_t)(b + 1) * p.num_tiles / p.num_ranges);
}

// What a thread of the count and emit kernels reads per tile: its chunk's
// bytes, its chunk's tile-exclusive identifier and the tile's identifier.
struct LexIn {
    uint32_t w[kLexWords];
    uint32_t cid, tid;
};

__device__ __forceinline__ LexIn load_lex_in(const LexFastParams& p, uint32_t tile)
{
    LexIn in;
    load_lex_chunk<true>(p.in + (size_t)tile * kLexFastTile + threadIdx.x * kLexFastChunk, kLexFastChunk, in.w);
    in.cid = p.chunk_id[(size_t)tile * kLexFastBlock + threadIdx.x];
    in.tid = p.tile_id[tile];
    return in;
}

// Runs full(tile, in, it) over the entirely full tiles of [t0, t1) in order,
// with two register buffers used in turn and an unconditional prefetch (the
// last full tile is read again at the end), then tail(tile, it) for the input's
// ragged last tile if the range holds it. it counts the tiles from 0.
template <typename Full, typename Tail>
__device__ __forceinline__ void walk_lex_tiles(const LexFastParams& p, uint32_t t0, uint32_t t1, const Full& full,
                                               const Tail& tail)
{
    const uint32_t tf = min(t1, p.n / (uint32_t)kLexFastTile);
    uint32_t t = t0;
    LexIn a, b;
    if (t < tf) a = load_lex_in(p, t);
    while (t < tf) {
        b = load_lex_in(p, min(t + 1, tf - 1));
        full(t, a, t - t0);
        if (++t >= tf) break;
        a = load_lex_in(p, min(t + 1, tf - 1));
        full(t, b, t - t0);
        ++t;
    }
    if (t < t1) tail(t, t - t0);
}

// identifier of the bytes of ranges 0..b-1 (thread i takes ranges 2i, 2i+1)
__device__ uint32_t lex_ranges_before(const LexFastParams& p, uint32_t b, uint32_t* s_wave, const LexIdComb& idc)
{
    const uint32_t i0 = 2 * threadIdx.x, i1 = i0 + 1;
    const uint32_t a = i0 < b ? p.range_id[i0] : p.identity;
    const uint32_t c = i1 < b ? p.range_id[i1] : p.identity;
    return block_reduce<kLexFastWaves>(idc(a, c), p.identity, s_wave, idc);
}

// boundaries of ranges 0..b-1
__device__ LexTok lex_tokens_before(const LexFastParams& p, uint32_t b, LexTok* s_wave)
{
    const uint32_t i0 = 2 * threadIdx.x, i1 = i0 + 1;
    const uint2 x = i0 < b ? p.range_tok[i0] : make_uint2(0u, 0u);
    const uint2 y = i1 < b ? p.range_tok[i1] : make_uint2(0u, 0u);
    return block_reduce<kLexFastWaves>(LexTok{x.x + y.x, max(x.y, y.y)}, LexTok{0u, 0u}, s_wave, LexTokComb{});
}

// The pass-2 kernels' LDS, one object so that the step table lies at LDS
// address 0 (the entries' row offsets are then the addresses themselves).
template <typename Rest>
struct LexPass2Shared {
    uint32_t step[kLexStepLds / 4];    // the minimal automaton (below)
    uint16_t state[kLexStateLds / 2];  // row offset of each identifier's state
    uint8_t col4[256];                 // each byte's column times 4
    Rest rest;                         // the kernel's own
};

// The minimal automaton in LDS, by byte offset: entry = the successor's row
// offset (successor * m * 4) | flag << 16 | kind of the row's state << 24;
// the row offset of each identifier's state; and each byte's column times 4.
// (Row offsets stay below 2^16: the table is held to 16 KiB; columns times 4
// fit a byte: the streaming kernels take m <= 64.)
template <typename Rest>
__device__ __forceinline__ void load_lex_automaton(const LexFastParams& p, LexPass2Shared<Rest>& sh)
{
    const uint32_t m4 = p.m * 4u;
    for (uint32_t i = threadIdx.x; i < p.nq * p.m; i += kLexFastBlock) {
        const uint32_t e = p.step[i];
        sh.step[i] = (e & 0xffffu) * m4 | (e & 0x10000u) | ((uint32_t)p.state_kind[i / p.m] << 24);
    }
    for (uint32_t i = threadIdx.x; i < p.k; i += kLexFastBlock) sh.state[i] = (uint16_t)(p.state_of[i] * m4);
    if (threadIdx.x < 256) sh.col4[threadIdx.x] = (uint8_t)(p.col[threadIdx.x] << 2);
}

// Several tiles' chunk identifiers, scanned together: the merges of the scans
// are independent gathers, so each level of the scan waits once for all.
constexpr int kIdsTiles = 4;

struct IdSet {
    uint32_t v[kIdsTiles];
};

struct LexIdSetComb {
    LexIdComb c;
    __device__ IdSet operator()(const IdSet& x, const IdSet& y) const
    {
        IdSet r;
#pragma unroll
        for (int k = 0; k < kIdsTiles; ++k) r.v[k] = c(x.v[k], y.v[k]);
        return r;
    }
};

// The rest of the pass-1 kernel's LDS, after the fold rows (all of it is
// dynamic, so the rows lie at LDS address 0).
struct IdsShared {
    uint8_t col2[256];  // each byte's column times 2
    IdSet set[2][kLexFastWaves];
    uint32_t wave[kLexFastWaves];
};

__global__ void __launch_bounds__(kLexFastBlock) lex_ids_kernel(LexFastParams p)
{
    extern __shared__ __align__(16) uint16_t s_rows[];
    const uint32_t row_vecs = (p.n_rows * p.m + 7u) / 8u;  // (the rows are padded to 16 bytes)
    IdsShared& sh = *reinterpret_cast<IdsShared*>(reinterpret_cast<uint4*>(s_rows) + row_vecs);
    uint8_t* const s_col = sh.col2;
    uint32_t* const s_wave = sh.wave;
    const uint32_t tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) {  // (no kernel of the call has read the header yet)
        p.hdr->tile_counter = 0;
        p.hdr->n_fields = 0;
        p.hdr->fault = 0;
        p.hdr->path = PPR_PATH_STREAMING;
    }
    for (uint32_t i = tid; i < row_vecs; i += kLexFastBlock)
        reinterpret_cast<uint4*>(s_rows)[i] = reinterpret_cast<const uint4*>(p.next_row)[i];
    if (tid < 256) s_col[tid] = (uint8_t)(p.col[tid] << 1);
    __syncthreads();
    const LexIdComb idc{p.merge, p.k, p.id_mask};
    const LexIdSetComb scomb{idc};
    const uint32_t tfull = p.n / (uint32_t)kLexFastTile;  // tiles [0, tfull) are entirely full
    const uint32_t stride = gridDim.x;
    // Workgroup b takes the full tiles b, b + G, b + 2G, ... (G = the grid),
    // kIdsTiles at a time: t, t + G, ... (t itself again in place of one that is
    // not a full tile; its copy then stores the same values).
    auto nth = [&](uint32_t t, uint32_t k) { return t + k * stride < tfull ? t + k * stride : t; };
    uint32_t it = 0;
    auto load_set = [&](uint32_t tile, uint32_t (&w)[kIdsTiles][kLexWords]) {
#pragma unroll
        for (int k = 0; k < kIdsTiles; ++k)
            load_lex_chunk<true>(p.in + (size_t)nth(tile, k) * kLexFastTile + tid * kLexFastChunk, kLexFastChunk,
                                 w[k]);
    };
    uint32_t w[kIdsTiles][kLexWords];
    if (blockIdx.x < tfull) load_set(blockIdx.x, w);
    for (uint32_t tile = blockIdx.x; tile < tfull; tile += kIdsTiles * stride, ++it) {
        // the next set's bytes load while this one is folded and scanned (the
        // empty asm keeps the compiler from sinking the loads below the fold;
        // the registers are free: the fold rows in LDS already hold the kernel
        // to two workgroups per CU)
        uint32_t wn[kIdsTiles][kLexWords];
        const uint32_t next = tile + kIdsTiles * stride;
        load_set(next < tfull ? next : tile, wn);
        asm volatile("" ::: "memory");
        IdSet v, ident, excl, tot;
        fold_lex_chunks<kIdsTiles>(p, w, s_rows, s_col, v.v);
#pragma unroll
        for (int k = 0; k < kIdsTiles; ++k) ident.v[k] = p.identity;
#pragma unroll
        for (int k = 0; k < kIdsTiles; ++k)
#pragma unroll
            for (int q = 0; q < kLexWords; ++q) w[k][q] = wn[k][q];
        block_scan<kLexFastWaves>(v, ident, excl, tot, sh.set[it & 1], scomb);
#pragma unroll
        for (int k = 0; k < kIdsTiles; ++k) {
            p.chunk_id[(size_t)nth(tile, k) * kLexFastBlock + tid] = (uint16_t)excl.v[k];
            if (tid == 0) p.tile_id[nth(tile, k)] = tot.v[k];
        }
    }
    if (tfull < p.num_tiles && blockIdx.x == tfull % stride) {  // the input's ragged last tile
        const uint32_t pos = tfull * (uint32_t)kLexFastTile + tid * (uint32_t)kLexFastChunk;
        const uint32_t len = pos < p.n ? min((uint32_t)kLexFastChunk, p.n - pos) : 0u;
        uint32_t w[kLexWords];
        load_lex_chunk<false>(p.in + pos, len, w);
        uint32_t excl, tot;
        block_scan<kLexFastWaves>(fold_lex_chunk<false>(p, w, len, s_rows, s_col), p.identity, excl, tot, s_wave,
                                  idc);
        p.chunk_id[(size_t)tfull * kLexFastBlock + tid] = (uint16_t)excl;
        if (tid == 0) p.tile_id[tfull] = tot;
    }
}

__global__ void __launch_bounds__(kWave) lex_range_kernel(LexFastParams p)
{
    const LexIdComb idc{p.merge, p.k, p.id_mask};
    uint32_t t0, t1;
    lex_range_of(p, blockIdx.x, t0, t1);
    uint32_t rv = p.identity;
    for (uint32_t t = t0; t < t1; t += kWave) {
        const uint32_t i = t + threadIdx.x;
        const uint32_t x = i < t1 ? p.tile_id[i] : p.identity;
        rv = idc(rv, readlane_t(wave_scan(x, p.identity, idc), kWave - 1));
    }
    if (threadIdx.x == 0) p.range_id[blockIdx.x] = rv;
}

__global__ void __launch_bounds__(kLexFastBlock) lex_count_kernel(LexFastParams p)
{
    struct Own {
        uint32_t wave[kLexFastWaves];
        LexTok tw[kLexFastWaves];
    };
    __shared__ __align__(16) LexPass2Shared<Own> sh;
    const uint32_t* s_step = sh.step;
    const uint16_t* s_state = sh.state;
    const uint8_t* s_col4 = sh.col4;
    uint32_t* s_wave = sh.rest.wave;
    LexTok* s_tw = sh.rest.tw;
    const uint32_t tid = threadIdx.x, b = blockIdx.x;
    load_lex_automaton(p, sh);
    const LexIdComb idc{p.merge, p.k, p.id_mask};
    uint32_t run = lex_ranges_before(p, b, s_wave, idc);  // (its barrier publishes the tables)
    uint32_t t0, t1;
    lex_range_of(p, b, t0, t1);
    LexTok acc{0u, 0u};
    auto count = [&](uint32_t tile, uint64_t B) {
        const uint32_t pos = tile * (uint32_t)kLexFastTile + tid * (uint32_t)kLexFastChunk;
        if (pos == 0) B &= ~1ull;  // a flag at the input's first byte ends no token
        acc.nt += (uint32_t)__popcll(B);
        if (B) acc.lb = pos + (uint32_t)(63 - __clzll((long long)B));
    };
    walk_lex_tiles(
        p, t0, t1,
        [&](uint32_t tile, const LexIn& in, uint32_t) {
            const uint32_t q = s_state[idc(run, in.cid)];
            count(tile, lex_pass2_full<false>(in.w, q, s_step, s_col4, nullptr));
            run = idc(run, in.tid);
        },
        [&](uint32_t tile, uint32_t) {
            const uint32_t pos = tile * (uint32_t)kLexFastTile + tid * (uint32_t)kLexFastChunk;
            const uint32_t len = pos < p.n ? min((uint32_t)kLexFastChunk, p.n - pos) : 0u;
            uint32_t w[kLexWords];
            load_lex_chunk<false>(p.in + pos, len, w);
            const uint32_t q = s_state[idc(run, p.chunk_id[(size_t)tile * kLexFastBlock + tid])];
            count(tile, lex_pass2_ragged<false>(w, len, q, s_step, s_col4, nullptr));
            run = idc(run, p.tile_id[tile]);
        });
    const LexTok r = block_reduce<kLexFastWaves>(acc, LexTok{0u, 0u}, s_tw, LexTokComb{});
    if (tid == 0) p.range_tok[b] = make_uint2(r.nt, r.lb);
}

__global__ void __launch_bounds__(kLexFastBlock) lex_emit_kernel(LexFastParams p)
{
    struct Own {
        uint32_t kind32[kLexFastTile / 4];  // kind of the token ending before each byte of the tile
        uint32_t list[kLexFastWaves][kLexList];
        uint32_t wave[kLexFastWaves];
        LexTok pre[kLexFastWaves];
        LexTok tw[2][kLexFastWaves];
    };
    __shared__ __align__(16) LexPass2Shared<Own> sh;
    const uint32_t* s_step = sh.step;
    const uint16_t* s_state = sh.state;
    const uint8_t* s_col4 = sh.col4;
    uint32_t* s_kind32 = sh.rest.kind32;
    uint32_t* s_wave = sh.rest.wave;
    LexTok* s_pre = sh.rest.pre;
    const uint32_t tid = threadIdx.x, b = blockIdx.x;
    const uint32_t lane = (uint32_t)lane_id();
    uint8_t* const s_kind = reinterpret_cast<uint8_t*>(s_kind32);
    load_lex_automaton(p, sh);
    const LexIdComb idc{p.merge, p.k, p.id_mask};
    uint32_t run = lex_ranges_before(p, b, s_wave, idc);  // (its barrier publishes the tables)
    LexTok P = lex_tokens_before(p, b, s_pre);
    uint32_t* list = sh.rest.list[tid / kWave];
    const uint32_t pos0 = tid * (uint32_t)kLexFastChunk;  // the chunk's first byte in the tile
    uint32_t t0, t1;
    lex_range_of(p, b, t0, t1);
    // one tile's tokens from its boundary bitmaps (pass 2 done, kinds in s_kind)
    auto emit = [&](uint32_t tile, uint64_t B, uint32_t it) {
        const uint32_t tile_start = tile * (uint32_t)kLexFastTile;
        const uint32_t pos = tile_start + pos0;
        if (pos == 0) B &= ~1ull;  // a flag at the input's first byte ends no token
        const LexTok c{(uint32_t)__popcll(B), B ? pos + (uint32_t)(63 - __clzll((long long)B)) : 0u};
        LexTok cex, ctot;
        block_scan<kLexFastWaves>(c, LexTok{0u, 0u}, cex, ctot, sh.rest.tw[it & 1u], LexTokComb{});  // (publishes s_kind)

        // Tokens, written by waves: each lane lists its boundaries (tile
        // positions) in the wave's list, then lane l of a round takes token
        // r + l: its end is its boundary, its start the previous boundary (the
        // lane before, by DPP).
        const uint32_t mine = c.nt;
        const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)cex.nt);  // tile tokens before the wave
        const uint32_t first = cex.nt - wbase;
        const uint32_t wcnt = (uint32_t)__builtin_amdgcn_readlane((int)(first + mine), kWave - 1);
        uint32_t off_run = max(P.lb, (uint32_t)__builtin_amdgcn_readfirstlane((int)cex.lb));
        const uint32_t tw[2] = {(uint32_t)B, (uint32_t)(B >> 32)}, rw[2] = {0u, 0u};
        for (uint32_t w0 = 0; w0 < wcnt; w0 += kLexList) {
            const uint32_t w1 = min(w0 + (uint32_t)kLexList, wcnt);
            list_terminators<2>(list, tw, rw, pos0, first, mine, w0, w1);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint32_t slots = slots_from(p.cap, (uint64_t)P.nt + wbase + w0, w1 - w0);
            for (uint32_t r = w0; r < w1; r += kWave) {
                const uint32_t cnt = min((uint32_t)kWave, w1 - r);
                const uint32_t e = list[r - w0 + min(lane, cnt - 1u)] >> 1;
                const uint32_t end = tile_start + e;
                const uint32_t prev = dpp_t<0x138, 0xf>(0u, end);  // wave_shr:1: the previous lane's boundary
                const uint32_t st = lane ? prev : off_run;
                const uint32_t g0 = P.nt + wbase + r;  // (token counts < n < 2^32)
                if (r - w0 + lane < slots) {
                    store_u32(p.kind + g0, lane, s_kind[e]);
                    store_u32(p.start + g0, lane, st);
                    store_u32(p.len + g0, lane, end - st);
                }
                off_run = (uint32_t)__builtin_amdgcn_readlane((int)end, (int)cnt - 1);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        P = LexTokComb{}(P, ctot);
        __syncthreads();  // the next tile's pass 2 rewrites s_kind
    };
    walk_lex_tiles(
        p, t0, t1,
        [&](uint32_t tile, const LexIn& in, uint32_t it) {
            const uint32_t q = s_state[idc(run, in.cid)];
            emit(tile, lex_pass2_full<true>(in.w, q, s_step, s_col4, s_kind32 + pos0 / 4u), it);
            run = idc(run, in.tid);
        },
        [&](uint32_t tile, uint32_t it) {
            const uint32_t pos = tile * (uint32_t)kLexFastTile + pos0;
            const uint32_t len = pos < p.n ? min((uint32_t)kLexFastChunk, p.n - pos) : 0u;
            uint32_t w[kLexWords];
            load_lex_chunk<false>(p.in + pos, len, w);
            const uint32_t q = s_state[idc(run, p.chunk_id[(size_t)tile * kLexFastBlock + tid])];
            emit(tile, lex_pass2_ragged<true>(w, len, q, s_step, s_col4, s_kind + pos0), it);
            run = idc(run, p.tile_id[tile]);
        });
    if (b == p.num_ranges - 1 && tid == 0) {  // the final token: from the last boundary to n
        if (P.nt < p.cap) {
            p.kind[P.nt] = p.final_[run];
            p.start[P.nt] = P.lb;
            p.len[P.nt] = p.n - P.lb;
        }
        p.hdr->n_fields = (uint64_t)P.nt + 1u;
    }
}

// workgroups of the pass-1 kernel (two per CU hold the fold rows in LDS)
constexpr uint32_t kLexIdsGrid = 512;

int launch_lex_fast(const LexFastParams& p, const ppr_parse_opts_t* o, hipStream_t s)
{
    const size_t ids_lds = (size_t)(p.n_rows * p.m + 7u) / 8u * 16u + sizeof(IdsShared);
    stage_event(o, 0, s);
    hipLaunchKernelGGL(lex_ids_kernel, dim3(std::min<uint32_t>(p.num_tiles, kLexIdsGrid)), dim3(kLexFastBlock), ids_lds,
                       s, p);
    hipLaunchKernelGGL(lex_range_kernel, dim3(p.num_ranges), dim3(kWave), 0, s, p);
    stage_event(o, 1, s);
    hipLaunchKernelGGL(lex_count_kernel, dim3(p.num_ranges), dim3(kLexFastBlock), 0, s, p);
    stage_event(o, 2, s);
    hipLaunchKernelGGL(lex_emit_kernel, dim3(p.num_ranges), dim3(kLexFastBlock), 0, s, p);
    stage_event(o, 3, s);
    return hipGetLastError() == hipSuccess ? PPR_OK : PPR_EHIP;
}

}  // namespace ppr
