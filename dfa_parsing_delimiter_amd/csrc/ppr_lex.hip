// Table-driven data-parallel lexer on gfx950.
//
// Method: "Lexing on the GPU: the scan is the easy part", section "A lexer is a
// prefix scan": bytes map to identifiers of partially applied transition
// functions, composition is one load from a k x k table of 16-bit identifiers,
// and the lexer state after every prefix is an inclusive scan under that
// composition. A flag bit on a merged identifier marks a token boundary; the
// final-state table gives the kind of the token ending just before it (section
// "Does it produce the same tokens?").
//
// MI355X mapping (not the page's Futhark map/scan/filter/gather pipeline, which
// materialises ~20 bytes of state per input byte):
//   * nothing per byte is materialised in HBM: a tile of 512*L bytes is staged
//     once into LDS, each thread folds its chunk sequentially (a chunk only ever
//     merges with single-byte elements, so the fold reads a k x m "fold" table —
//     the merge table restricted to the m distinct byte identifiers — that fits
//     in L2, instead of the k x k table);
//   * chunk identifiers are scanned in the workgroup with the merge table, then
//     across tiles by decoupled look-back (16-bit payloads);
//   * each thread re-folds its chunk from its true prefix identifier, marks token
//     boundaries in a bitmap, and a second look-back scans token counts; tokens
//     are written as (kind, start, length) directly.
#include <map>
#include <vector>

#include "ppr.h"
#include "ppr_device.h"
#include "ppr_host.h"
#include "ppr_lex_common.h"
#include "ppr_scan.h"

namespace ppr {

constexpr int kLexBlock = 512;  // threads per tile: a look-back round covers 512 tiles
constexpr int kLexWaves = kLexBlock / kWave;
constexpr int kLexMaxChunk = 64;
constexpr int kLexLdsKinds = 4096;  // final-state tables up to this many entries are read from LDS
constexpr uint32_t kLexLdsStep = 48u << 10;  // minimal automata up to this size are stepped from LDS

struct LexParams {
    const uint8_t* in;
    uint32_t n, L, tile_bytes, num_tiles, epoch;
    uint32_t k, m;
    uint32_t id_mask, flag_mask;
    uint32_t identity, reserved;
    const uint16_t* merge;  // k x k
    const uint16_t* fold;   // k x m
    const uint16_t* final_;
    const uint16_t* state_of;  // minimal automaton (nq > 0): state of each identifier,
    const uint32_t* step;      //   per state and column: successor | flag << 16,
    const uint16_t* state_kind;  //   per state: token kind
    uint32_t nq;                 // its states; 0: pass 2 re-folds the identifiers
    uint32_t* kind;
    uint32_t* start;
    uint32_t* len;
    uint64_t cap;
    WsHeader* hdr;
    uint64_t* statA;
    StatB* statB;  // payload words: token count, last boundary
    uint8_t col[256];
};

__device__ __forceinline__ uint32_t merge_ids(const LexParams& p, uint32_t a, uint32_t b)
{
    return (uint32_t)p.merge[(uint64_t)a * p.k + b] & p.id_mask;
}

// token-count carry: nt tokens ended, lb = last boundary position (0 when none:
// the first token starts at 0 either way). Both combine commutatively.
struct TokCarry {
    uint32_t nt, lb;
};

struct IdComb {
    const uint16_t* merge;
    uint32_t k, id_mask;
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const
    {
        return (uint32_t)merge[(uint64_t)a * k + b] & id_mask;
    }
};
struct TokComb {
    __device__ TokCarry operator()(const TokCarry& a, const TokCarry& b) const
    {
        return {a.nt + b.nt, max(a.lb, b.lb)};
    }
};

// one tile's identifier status: aggregate = the tile's identifier, inclusive =
// the identifier of everything through the tile
struct IdPoll {
    const uint64_t* statA;
    uint32_t epoch;
    __device__ uint32_t operator()(int64_t u, uint32_t& out) const
    {
        const uint64_t w = ld_relaxed(&statA[u]);
        const uint32_t f = status_flag(w, epoch);
        if (f) out = status_payload(w);
        return f;
    }
};

// one tile's token-count status (two self-validating words per kind)
struct TokPoll {
    const StatB* statB;
    uint32_t epoch;
    __device__ uint32_t operator()(int64_t u, TokCarry& out) const
    {
        const StatB& s = statB[u];
        const uint64_t i0 = ld_relaxed(&s.incl[0]), i1 = ld_relaxed(&s.incl[1]);
        if (ew_ok(i0, epoch) && ew_ok(i1, epoch)) {
            out = {(uint32_t)i0, (uint32_t)i1};
            return kFlagIncl;
        }
        const uint64_t a0 = ld_relaxed(&s.agg[0]), a1 = ld_relaxed(&s.agg[1]);
        if (ew_ok(a0, epoch) && ew_ok(a1, epoch)) {
            out = {(uint32_t)a0, (uint32_t)a1};
            return kFlagAgg;
        }
        return 0;
    }
};

__device__ __forceinline__ void publish_tok(StatB& s, TokCarry c, uint32_t epoch, uint32_t flag)
{
    uint64_t* w = flag == kFlagIncl ? s.incl : s.agg;
    st_relaxed(&w[0], ew(epoch, c.nt));
    st_relaxed(&w[1], ew(epoch, c.lb));
}

// Resets the workspace header (workgroup 0) and clears the look-back statuses
// (all workgroups: n_stat 16-byte words from stat).
__global__ void lex_reset_kernel(WsHeader* hdr, uint4* stat, uint64_t n_stat)
{
    clear_status(stat, n_stat);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr->tile_counter = 0;
        hdr->n_fields = 0;
        hdr->fault = 0;
        hdr->path = PPR_PATH_SINGLE_PASS;
    }
}

__global__ void __launch_bounds__(kLexBlock) lex_kernel(LexParams p)
{
    // dynamic LDS, sized for the call's chunk length L: the tile's bytes, then the
    // kind of the token ending before each byte (3 L bytes per thread, so that
    // short chunks leave room for more workgroups per CU)
    // (and, when k <= kLexLdsKinds, the final-state table after them)
    extern __shared__ __align__(16) uint8_t s_dyn[];
    uint8_t* s_bytes = s_dyn;
    uint16_t* s_kind = reinterpret_cast<uint16_t*>(s_dyn + kLexBlock * p.L);
    uint16_t* s_final = s_kind + kLexBlock * p.L;
    const bool use_min = p.nq != 0;
    const bool lds_final = !use_min && p.k <= (uint32_t)kLexLdsKinds;
    uint32_t* s_step = reinterpret_cast<uint32_t*>(s_final);  // (use_min: in place of the final-state table)
    uint16_t* s_qkind = reinterpret_cast<uint16_t*>(s_step + (use_min ? p.nq * p.m : 0u));
    __shared__ uint8_t s_col[256];
    __shared__ uint32_t s_wid[kLexWaves], s_pid[kLexWaves];
    __shared__ TokCarry s_wtok[kLexWaves], s_ptok[kLexWaves];
    __shared__ int s_first[kLexWaves];
    __shared__ uint32_t s_tile, s_prefix_id;
    __shared__ TokCarry s_prefix;

    const int tid = threadIdx.x;
    // tiles in the order workgroups start (not blockIdx order): a tile only waits
    // in its look-backs on tiles that running workgroups already hold
    if (tid == 0) s_tile = atomicAdd(&p.hdr->tile_counter, 1u);
    if (tid < 256) s_col[tid] = p.col[tid];
    if (lds_final)
        for (uint32_t i = tid; i < p.k; i += kLexBlock) s_final[i] = p.final_[i];
    if (use_min) {
        for (uint32_t i = tid; i < p.nq * p.m; i += kLexBlock) s_step[i] = p.step[i];
        for (uint32_t i = tid; i < p.nq; i += kLexBlock) s_qkind[i] = p.state_kind[i];
    }
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint32_t tile_start = tile * p.tile_bytes;
    const uint32_t tile_len = min(p.tile_bytes, p.n - tile_start);

    const uint8_t* src = p.in + tile_start;
    if ((((uintptr_t)src) & 15u) == 0) {
        const uint32_t nvec = tile_len >> 4;
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(s_bytes);
        for (uint32_t i = tid; i < nvec; i += kLexBlock) d4[i] = s4[i];
        for (uint32_t i = (nvec << 4) + tid; i < tile_len; i += kLexBlock) s_bytes[i] = src[i];
    } else {
        for (uint32_t i = tid; i < tile_len; i += kLexBlock) s_bytes[i] = src[i];
    }
    __syncthreads();

    const uint32_t L = p.L;
    const uint32_t pos0 = tid * L;
    const uint32_t my_len = pos0 < tile_len ? min(L, tile_len - pos0) : 0u;
    const uint32_t chunk_abs = tile_start + pos0;
    const uint32_t m = p.m;

    // pass 1: fold the chunk from the identity (flags are ignored here)
    uint32_t x = p.identity;
    for (uint32_t j = 0; j < my_len; ++j) x = (uint32_t)p.fold[x * m + s_col[s_bytes[pos0 + j]]] & p.id_mask;
    const IdComb idc{p.merge, p.k, p.id_mask};
    uint32_t excl, tot;
    block_scan<kLexWaves>(x, p.identity, excl, tot, s_wid, idc);

    if (tile == 0) {
        if (tid == 0) {
            s_prefix_id = p.identity;
            st_relaxed(&p.statA[0], status_word(p.epoch, kFlagIncl, tot));
        }
    } else {
        if (tid == 0) st_relaxed(&p.statA[tile], status_word(p.epoch, kFlagAgg, tot));
        const uint32_t pre = lookback<kLexWaves>(tile, p.identity, IdPoll{p.statA, p.epoch}, idc, s_pid, s_first,
                                                 &p.hdr->fault);
        if (tid == 0) {
            s_prefix_id = pre;
            st_relaxed(&p.statA[tile], status_word(p.epoch, kFlagIncl, merge_ids(p, pre, tot)));
        }
    }
    __syncthreads();
    const uint32_t tile_prefix = s_prefix_id;

    // pass 2: from the true prefix, mark boundaries. With the minimal automaton
    // this steps a few states in LDS; otherwise it re-folds the identifiers.
    uint32_t prev = merge_ids(p, tile_prefix, excl);
    uint64_t B = 0;
    if (use_min) {
        uint32_t qs = p.state_of[prev];
        for (uint32_t j = 0; j < my_len; ++j) {
            const uint32_t e = s_step[qs * m + s_col[s_bytes[pos0 + j]]];
            if ((e >> 16) && (chunk_abs + j) != 0u) {
                B |= 1ull << j;
                s_kind[pos0 + j] = s_qkind[qs];
            }
            qs = e & 0xffffu;
        }
    } else {
        for (uint32_t j = 0; j < my_len; ++j) {
            const uint32_t y = p.fold[prev * m + s_col[s_bytes[pos0 + j]]];
            if ((y & p.flag_mask) && (chunk_abs + j) != 0u) {
                B |= 1ull << j;
                s_kind[pos0 + j] = lds_final ? s_final[prev] : p.final_[prev];
            }
            prev = y & p.id_mask;
        }
    }
    TokCarry c{(uint32_t)__popcll(B), B ? chunk_abs + (uint32_t)(63 - __clzll((long long)B)) : 0u};
    TokCarry cex, ctot;
    block_scan<kLexWaves>(c, TokCarry{0, 0}, cex, ctot, s_wtok, TokComb{});

    if (tile == 0) {
        if (tid == 0) {
            s_prefix = TokCarry{0, 0};
            publish_tok(p.statB[0], ctot, p.epoch, kFlagIncl);
        }
    } else {
        if (tid == 0) publish_tok(p.statB[tile], ctot, p.epoch, kFlagAgg);
        const TokCarry pre = lookback<kLexWaves>(tile, TokCarry{0, 0}, TokPoll{p.statB, p.epoch}, TokComb{}, s_ptok,
                                                 s_first, &p.hdr->fault);
        if (tid == 0) {
            s_prefix = pre;
            publish_tok(p.statB[tile], TokCarry{pre.nt + ctot.nt, max(pre.lb, ctot.lb)}, p.epoch, kFlagIncl);
        }
    }
    __syncthreads();
    const TokCarry P = s_prefix;

    // Tokens, written by waves: each lane lists its boundaries (tile positions)
    // in the wave's LDS list, laid over the tile's bytes (pass 2 is done with
    // them: barriers since), then lane l of a round takes token r + l. Its end
    // is its boundary, its start the previous one (the lane before, by DPP), so
    // the three output arrays are written with consecutive addresses.
    {
        const uint32_t lane = (uint32_t)lane_id();
        const uint32_t lcap = kLexBlock * L / 4u / kLexWaves;  // per-wave list entries over the tile's bytes
        uint32_t* list = reinterpret_cast<uint32_t*>(s_bytes) + (tid / kWave) * lcap;
        const uint32_t mine = c.nt;
        const uint32_t wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)cex.nt);  // tokens before the wave
        const uint32_t first = cex.nt - wbase;
        const uint32_t wcnt = (uint32_t)__builtin_amdgcn_readlane((int)(first + mine), kWave - 1);
        uint32_t off_run = max(P.lb, (uint32_t)__builtin_amdgcn_readfirstlane((int)cex.lb));
        const uint32_t tw[2] = {(uint32_t)B, (uint32_t)(B >> 32)}, rw[2] = {0u, 0u};
        for (uint32_t w0 = 0; w0 < wcnt; w0 += lcap) {
            const uint32_t w1 = min(w0 + lcap, wcnt);
            list_terminators<2>(list, tw, rw, pos0, first, mine, w0, w1);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint32_t slots = slots_from(p.cap, (uint64_t)P.nt + wbase + w0, w1 - w0);
            for (uint32_t r = w0; r < w1; r += kWave) {
                const uint32_t cnt = min((uint32_t)kWave, w1 - r);
                const uint32_t e = list[r - w0 + min(lane, cnt - 1u)] >> 1;
                const uint32_t pos = tile_start + e;
                const uint32_t prev = dpp_t<0x138, 0xf>(0u, pos);  // wave_shr:1: the previous lane's boundary
                const uint32_t st = lane ? prev : off_run;
                const uint32_t kd = s_kind[e];
                const uint32_t g0 = P.nt + wbase + r;  // (token counts < n < 2^32)
                if (r - w0 + lane < slots) {
                    store_u32(p.kind + g0, lane, kd);
                    store_u32(p.start + g0, lane, st);
                    store_u32(p.len + g0, lane, pos - st);
                }
                off_run = (uint32_t)__builtin_amdgcn_readlane((int)pos, (int)cnt - 1);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    if (tile == p.num_tiles - 1 && tid == 0) {
        const uint32_t nt = P.nt + ctot.nt;
        const uint32_t lb = max(P.lb, ctot.lb);
        const uint32_t last = merge_ids(p, tile_prefix, tot);
        if (nt < p.cap) {
            p.kind[nt] = p.final_[last];
            p.start[nt] = lb;
            p.len[nt] = p.n - lb;
        }
        p.hdr->n_fields = (uint64_t)nt + 1u;
    }
}

// sets *bad if any merge entry's identifier is >= k
__global__ void lex_check_kernel(const uint16_t* merge, uint64_t count, uint32_t k, uint32_t id_mask, uint32_t* bad)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count && ((uint32_t)merge[i] & id_mask) >= k) atomicOr(bad, 1u);
}

struct ColumnIds {
    uint16_t id[256];
};

// fold[x][j] = merge[x][identifier of column j]
__global__ void lex_fold_kernel(const uint16_t* merge, uint32_t k, ColumnIds cols, uint32_t m, uint16_t* fold)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (uint64_t)k * m) return;
    const uint64_t x = i / m, j = i % m;
    fold[i] = merge[x * k + cols.id[j]];
}

// Where the minimal automaton sits in the prepared buffer (after the k x m fold
// entries): byte offsets of the state of each identifier, the step table and the
// state kinds, and the end. Fits when end <= ppr_lex_fold_bytes(k).
struct MinLayout {
    uint64_t state_of, step, kind, end;
};

static MinLayout min_layout(uint32_t k, uint32_t m, uint32_t nq)
{
    MinLayout L;
    L.state_of = align_up((uint64_t)k * m * 2u, 256);
    L.step = align_up(L.state_of + (uint64_t)k * 2u, 256);
    L.kind = align_up(L.step + (uint64_t)nq * m * 4u, 256);
    L.end = L.kind + (uint64_t)nq * 2u;
    return L;
}

// Where the fold rows of the streaming kernels sit, after the minimal
// automaton: the next row (times m) and the identifier reached, n_rows x m
// entries each, padded to 16 bytes.
struct RowLayout {
    uint64_t next_row, row_id, end;
};

static RowLayout row_layout(uint32_t k, uint32_t m, uint32_t nq, uint32_t n_rows)
{
    RowLayout L;
    const uint64_t bytes = align_up((uint64_t)n_rows * m * 2u, 16);
    L.next_row = align_up(min_layout(k, m, nq).end, 256);
    L.row_id = align_up(L.next_row + bytes, 256);
    L.end = L.row_id + bytes;
    return L;
}

// Fold rows [L, "A lexer is a prefix scan": the chunk fold is a walk through
// the fold table]: identifiers whose rows of the fold table name the same
// identifiers share a row. Pass 1 only needs the row it is in until the last
// byte, so it walks the (fewer) rows and reads the identifier at the end.
// Returns the row count; row_of[x] is the row of identifier x, rep[r] one
// identifier of row r.
static uint32_t lex_fold_rows(const std::vector<uint16_t>& fold, uint32_t k, uint32_t m, uint32_t id_mask,
                              std::vector<uint32_t>& row_of, std::vector<uint32_t>& rep)
{
    std::map<std::vector<uint16_t>, uint32_t> rows;
    std::vector<uint16_t> key(m);
    row_of.assign(k, 0);
    rep.clear();
    for (uint32_t x = 0; x < k; ++x) {
        for (uint32_t j = 0; j < m; ++j) key[j] = (uint16_t)(fold[(size_t)x * m + j] & id_mask);
        const auto it = rows.emplace(key, (uint32_t)rows.size());
        if (it.second) rep.push_back(x);
        row_of[x] = it.first->second;
    }
    return (uint32_t)rows.size();
}

// Minimal automaton of the identifier fold [L, "A lexer is a prefix scan": the
// fold is a DFA over identifiers]. States are identifiers, symbols are columns;
// reading column j in x outputs the flag of fold[x][j] and, with the flag, the
// kind final[x] of the token it ends; final[x] is also the kind of a last token.
// Refinement starts from the partition by (final[x], the flags of row x) and
// splits by successor states until no state splits. Returns the state count.
static uint32_t lex_minimize(const std::vector<uint16_t>& fold, const std::vector<uint16_t>& fin, uint32_t k,
                             uint32_t m, uint32_t flag, uint32_t id_mask, std::vector<uint32_t>& cls)
{
    cls.assign(k, 0);
    std::vector<uint32_t> sig(m + 1);
    std::map<std::vector<uint32_t>, uint32_t> ids;
    for (uint32_t x = 0; x < k; ++x) {
        sig[0] = fin[x];
        for (uint32_t j = 0; j < m; ++j) sig[1 + j] = (fold[(size_t)x * m + j] & flag) ? 1u : 0u;
        cls[x] = ids.emplace(sig, (uint32_t)ids.size()).first->second;
    }
    uint32_t n = (uint32_t)ids.size();
    std::vector<uint32_t> next(k);
    for (;;) {
        std::map<std::vector<uint32_t>, uint32_t> nids;
        for (uint32_t x = 0; x < k; ++x) {
            sig[0] = cls[x];
            for (uint32_t j = 0; j < m; ++j) sig[1 + j] = cls[fold[(size_t)x * m + j] & id_mask];
            next[x] = nids.emplace(sig, (uint32_t)nids.size()).first->second;
        }
        if ((uint32_t)nids.size() == n) return n;  // no state split: the partition is stable
        n = (uint32_t)nids.size();
        cls.swap(next);
    }
}

constexpr uint64_t kLexStreamMinAuto = 8ull << 20;

static uint32_t lex_chunk_of(const ppr_parse_opts_t* o)
{
    uint32_t L = o ? o->chunk_bytes : 0u;
    if (L == 0) L = 40;  // the default: measured fastest on the 40-rule token stream (32 to 56 within 10%)
    return L <= (uint32_t)kLexMaxChunk ? L : 0u;
}

static WsLayout lex_layout(uint64_t n, uint32_t L)
{
    const uint64_t tile = (uint64_t)kLexBlock * L;
    const uint64_t tiles = (n + tile - 1) / tile;
    WsLayout w;
    w.tiles = tiles;
    w.off_a = 256;
    w.off_b = align_up(w.off_a + tiles * sizeof(uint64_t), 256);
    w.total = align_up(w.off_b + tiles * sizeof(StatB), 256);
    return w;
}

WsHeader* pinned_header();  // ppr_csv.hip: the blocking calls' pinned header buffer

}  // namespace ppr

using namespace ppr;

extern "C" size_t ppr_lex_fold_bytes(uint32_t k) { return (size_t)k * 256u * sizeof(uint16_t); }

extern "C" int ppr_lex_prepare(const ppr_lex_tables_t* t, ppr_lex_prepared_t* prep, void* stream)
{
    if (!t || !prep || !t->initial_state || !t->merge_table || !t->final_states || !prep->d_fold) return PPR_EINVAL;
    if (t->k == 0 || t->k > t->flag_mask || t->flag_mask != 0x8000u || t->identity >= t->k) return PPR_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    uint16_t init[256];
    if (hipMemcpyAsync(init, t->initial_state, sizeof init, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    ColumnIds cols;
    memset(&cols, 0, sizeof cols);
    uint32_t m = 0;
    for (int b = 0; b < 256; ++b) {
        const uint16_t id = (uint16_t)(init[b] & (uint16_t)~t->flag_mask);
        if (id >= t->k) return PPR_EINVAL;
        uint32_t j = 0;
        while (j < m && cols.id[j] != id) ++j;
        if (j == m) cols.id[m++] = id;
        prep->column_of[b] = (uint8_t)j;
    }
    prep->k = t->k;
    prep->m = m;
    prep->identity = t->identity;
    prep->flag_mask = t->flag_mask;
    {
        // every merge entry must name an identifier below k; the prepared fold
        // buffer's first word serves as the flag (it is overwritten below)
        uint32_t* d_bad = reinterpret_cast<uint32_t*>(prep->d_fold);
        uint32_t bad = 0;
        if (hipMemsetAsync(d_bad, 0, sizeof(uint32_t), s) != hipSuccess) return PPR_EHIP;
        const uint64_t count = (uint64_t)t->k * t->k;
        hipLaunchKernelGGL(lex_check_kernel, dim3((uint32_t)((count + 255) / 256)), dim3(256), 0, s, t->merge_table,
                           count, t->k, (uint32_t)(uint16_t)~t->flag_mask, d_bad);
        if (hipGetLastError() != hipSuccess) return PPR_EHIP;
        if (hipMemcpyAsync(&bad, d_bad, sizeof bad, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
        if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
        if (bad) return PPR_EINVAL;
    }
    const uint64_t total = (uint64_t)t->k * m;
    const uint32_t blocks = (uint32_t)((total + 255) / 256);
    hipLaunchKernelGGL(lex_fold_kernel, dim3(blocks), dim3(256), 0, s, t->merge_table, t->k, cols, m, prep->d_fold);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;

    // the minimal automaton of the fold, stored after it in the same buffer
    prep->n_states = 0;
    prep->n_rows = 0;
    prep->row0 = 0;
    std::vector<uint16_t> fold(total), fin(t->k);
    if (hipMemcpy(fold.data(), prep->d_fold, total * 2u, hipMemcpyDeviceToHost) != hipSuccess) return PPR_EHIP;
    if (hipMemcpy(fin.data(), t->final_states, (size_t)t->k * 2u, hipMemcpyDeviceToHost) != hipSuccess)
        return PPR_EHIP;
    std::vector<uint32_t> cls;
    const uint32_t id_mask = (uint32_t)(uint16_t)~t->flag_mask;
    const uint32_t nq = lex_minimize(fold, fin, t->k, m, t->flag_mask, id_mask, cls);
    const MinLayout ml = min_layout(t->k, m, nq);
    if (ml.end <= ppr_lex_fold_bytes(t->k)) {
        std::vector<uint16_t> state_of(t->k), qkind(nq);
        std::vector<uint32_t> step((size_t)nq * m), rep(nq, 0xffffffffu);
        for (uint32_t x = 0; x < t->k; ++x) {
            state_of[x] = (uint16_t)cls[x];
            if (rep[cls[x]] == 0xffffffffu) rep[cls[x]] = x;
        }
        for (uint32_t q = 0; q < nq; ++q) {
            const uint32_t x = rep[q];
            qkind[q] = fin[x];
            for (uint32_t j = 0; j < m; ++j) {
                const uint32_t y = fold[(size_t)x * m + j];
                step[(size_t)q * m + j] = cls[y & id_mask] | ((y & t->flag_mask) ? 0x10000u : 0u);
            }
        }
        uint8_t* base = reinterpret_cast<uint8_t*>(prep->d_fold);
        if (hipMemcpy(base + ml.state_of, state_of.data(), (size_t)t->k * 2u, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(base + ml.step, step.data(), step.size() * 4u, hipMemcpyHostToDevice) != hipSuccess ||
            hipMemcpy(base + ml.kind, qkind.data(), (size_t)nq * 2u, hipMemcpyHostToDevice) != hipSuccess)
            return PPR_EHIP;
        prep->n_states = nq;

        // the streaming kernels' fold rows, where their tables fit the LDS budgets
        // (the automaton's entries carry the 8-bit kinds, its states times m 16
        // bits; a column times 4 is one byte, so m <= 64)
        uint32_t max_kind = 0;
        for (uint32_t q = 0; q < nq; ++q) max_kind = std::max<uint32_t>(max_kind, qkind[q]);
        std::vector<uint32_t> row_of, rrep;
        const uint32_t nr = lex_fold_rows(fold, t->k, m, id_mask, row_of, rrep);
        const RowLayout rl = row_layout(t->k, m, nq, nr);
        if (max_kind < 256u && m <= 64u && (uint64_t)nq * m * 4u <= kLexStepLds && (uint64_t)t->k * 2u <= kLexStateLds &&
            (uint64_t)nr * m * 2u <= kLexRowLds && rl.end <= ppr_lex_fold_bytes(t->k)) {
            const size_t cells = align_up((uint64_t)nr * m * 2u, 16) / 2u;
            std::vector<uint16_t> next_row(cells, 0), row_id(cells, 0);
            for (uint32_t r = 0; r < nr; ++r)
                for (uint32_t j = 0; j < m; ++j) {
                    const uint32_t y = fold[(size_t)rrep[r] * m + j] & id_mask;
                    next_row[(size_t)r * m + j] = (uint16_t)(row_of[y] * m);
                    row_id[(size_t)r * m + j] = (uint16_t)y;
                }
            if (hipMemcpy(base + rl.next_row, next_row.data(), cells * 2u, hipMemcpyHostToDevice) != hipSuccess ||
                hipMemcpy(base + rl.row_id, row_id.data(), cells * 2u, hipMemcpyHostToDevice) != hipSuccess)
                return PPR_EHIP;
            prep->n_rows = nr;
            prep->row0 = row_of[t->identity] * m;
        }
    }
    return PPR_OK;
}

extern "C" size_t ppr_lex_workspace_bytes(uint64_t n, const ppr_parse_opts_t* opts)
{
    const uint32_t L = lex_chunk_of(opts);
    if (!L || n > kMaxInput) return 0;
    uint64_t total = lex_layout(n, L).total;
    if (L == (uint32_t)kLexFastChunk) total = std::max(total, lex_fast_layout(n).total);
    return (size_t)total;
}

extern "C" int ppr_lex_async(const uint8_t* d_bytes, uint64_t n, const ppr_lex_tables_t* t,
                             const ppr_lex_prepared_t* prep, const ppr_tokens_out_t* out, void* d_ws, size_t ws_bytes,
                             const ppr_parse_opts_t* opts, void* stream)
{
    if (!t || !prep || !out || !d_ws || (n && !d_bytes)) return PPR_EINVAL;
    if (!t->merge_table || !t->final_states || !prep->d_fold || prep->k != t->k || prep->m == 0) return PPR_EINVAL;
    if (t->k == 0 || t->flag_mask != 0x8000u || t->identity >= t->k) return PPR_EINVAL;
    if (out->cap_tokens && (!out->kind || !out->start || !out->length)) return PPR_EINVAL;
    if (n > kMaxInput) return PPR_ETOOBIG;
    const uint32_t L = lex_chunk_of(opts);
    if (!L) return PPR_EINVAL;
    const uint32_t want = opts ? opts->path : 0u;
    if (want > PPR_PATH_FUSED) return PPR_EINVAL;
    const WsLayout lay = lex_layout(n, L);
    if (ws_bytes < lay.total || ((uintptr_t)d_ws & 255u)) return PPR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    WsHeader* hdr = (WsHeader*)ws;

    // the streaming kernels: 40-byte chunks, 8-byte aligned input, prepared fold rows;
    // chosen automatically
    // above kLexStreamMinAuto bytes, where their four launches pay off (the
    // single-pass kernel: 56 against 65 us at 1 MiB, 74 against 81 us at 8 MiB;
    // equal at 16 MiB, 176 against 135 us at 32 MiB)
    const bool asked = want == PPR_PATH_STREAMING || want == PPR_PATH_FUSED;
    if (n && (asked || (want == 0 && n > kLexStreamMinAuto)) && L == (uint32_t)kLexFastChunk &&
        ((uintptr_t)d_bytes & 7u) == 0 && prep->n_rows && prep->n_states) {
        const LexFastLayout fl = lex_fast_layout(n);
        if (ws_bytes < fl.total) return PPR_EWORKSPACE;
        const MinLayout ml = min_layout(prep->k, prep->m, prep->n_states);
        const RowLayout rl = row_layout(prep->k, prep->m, prep->n_states, prep->n_rows);
        const uint8_t* base = reinterpret_cast<const uint8_t*>(prep->d_fold);
        LexFastParams f;
        memset(&f, 0, sizeof f);
        f.in = d_bytes;
        f.n = (uint32_t)n;
        f.num_tiles = (uint32_t)fl.tiles;
        f.num_ranges = (uint32_t)fl.ranges;
        f.k = t->k;
        f.m = prep->m;
        f.identity = t->identity;
        f.id_mask = (uint32_t)(uint16_t)~t->flag_mask;
        f.row0 = prep->row0;
        f.n_rows = prep->n_rows;
        f.nq = prep->n_states;
        f.merge = t->merge_table;
        f.final_ = t->final_states;
        f.next_row = reinterpret_cast<const uint16_t*>(base + rl.next_row);
        f.row_id = reinterpret_cast<const uint16_t*>(base + rl.row_id);
        f.state_of = reinterpret_cast<const uint16_t*>(base + ml.state_of);
        f.step = reinterpret_cast<const uint32_t*>(base + ml.step);
        f.state_kind = reinterpret_cast<const uint16_t*>(base + ml.kind);
        f.chunk_id = reinterpret_cast<uint16_t*>(ws + fl.chunk_id);
        f.tile_id = reinterpret_cast<uint32_t*>(ws + fl.tile_id);
        f.range_id = reinterpret_cast<uint32_t*>(ws + fl.range_id);
        f.range_tok = reinterpret_cast<uint2*>(ws + fl.range_tok);
        f.kind = out->kind;
        f.start = out->start;
        f.len = out->length;
        f.cap = out->cap_tokens;
        f.hdr = hdr;
        memcpy(f.col, prep->column_of, 256);
        return launch_lex_fast(f, opts, s);
    }
    stage_event(opts, 0, s);
    const uint64_t stat_bytes = lay.total - lay.off_a;  // statuses A and B, with their padding
    hipLaunchKernelGGL(lex_reset_kernel, dim3(clear_grid(stat_bytes)), dim3(256), 0, s, hdr, (uint4*)(ws + lay.off_a),
                       stat_bytes / 16);
    stage_event(opts, 1, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    if (n == 0) return PPR_OK;
    LexParams p;
    memset(&p, 0, sizeof p);
    p.in = d_bytes;
    p.n = (uint32_t)n;
    p.L = L;
    p.tile_bytes = kLexBlock * L;
    p.num_tiles = (uint32_t)lay.tiles;
    p.epoch = next_epoch();
    p.k = t->k;
    p.m = prep->m;
    p.flag_mask = t->flag_mask;
    p.id_mask = (uint32_t)(uint16_t)~t->flag_mask;
    p.identity = t->identity;
    p.merge = t->merge_table;
    p.fold = prep->d_fold;
    p.final_ = t->final_states;
    p.kind = out->kind;
    p.start = out->start;
    p.len = out->length;
    p.cap = out->cap_tokens;
    p.hdr = hdr;
    p.statA = (uint64_t*)(ws + lay.off_a);
    p.statB = (StatB*)(ws + lay.off_b);
    memcpy(p.col, prep->column_of, 256);
    // the minimal automaton steps pass 2 when it fits the LDS budget
    p.nq = 0;
    if (prep->n_states && (uint64_t)prep->n_states * prep->m * 4u + prep->n_states * 2u <= kLexLdsStep &&
        min_layout(prep->k, prep->m, prep->n_states).end <= ppr_lex_fold_bytes(prep->k)) {
        const MinLayout ml = min_layout(prep->k, prep->m, prep->n_states);
        const uint8_t* base = reinterpret_cast<const uint8_t*>(prep->d_fold);
        p.nq = prep->n_states;
        p.state_of = reinterpret_cast<const uint16_t*>(base + ml.state_of);
        p.step = reinterpret_cast<const uint32_t*>(base + ml.step);
        p.state_kind = reinterpret_cast<const uint16_t*>(base + ml.kind);
    }
    const size_t lds = (size_t)kLexBlock * L * 3u +
                       (p.nq ? (size_t)p.nq * p.m * 4u + p.nq * 2u
                             : (p.k <= (uint32_t)kLexLdsKinds ? (size_t)p.k * 2u : 0u));
    hipLaunchKernelGGL(lex_kernel, dim3(p.num_tiles), dim3(kLexBlock), lds, s, p);
    stage_event(opts, 2, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    return PPR_OK;
}

extern "C" int ppr_lex_results(const void* d_ws, uint64_t n, ppr_tokens_out_t* out, void* stream)
{
    (void)n;
    if (!d_ws || !out) return PPR_EINVAL;
    WsHeader local;
    WsHeader* dst = pinned_header();  // (per host thread, pinned: one DMA)
    if (!dst) dst = &local;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(dst, d_ws, sizeof(WsHeader), hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    const WsHeader h = *dst;
    out->n_tokens = h.n_fields;
    out->path = h.path;
    if (h.fault) return PPR_EHIP;
    return out->n_tokens > out->cap_tokens ? PPR_ECAPACITY : PPR_OK;
}

extern "C" int ppr_lex(const uint8_t* d_bytes, uint64_t n, const ppr_lex_tables_t* t, const ppr_lex_prepared_t* prep,
                       ppr_tokens_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream)
{
    int rc = ppr_lex_async(d_bytes, n, t, prep, out, d_ws, ws_bytes, opts, stream);
    if (rc) return rc;
    return ppr_lex_results(d_ws, n, out, stream);
}
