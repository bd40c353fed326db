// Data-parallel DFA parse of delimiter-separated bytes on gfx950: the C-ABI
// entry points and the single-pass generic kernel.
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
// Two implementations of these steps:
//   * the streaming path (ppr_csv_fast.hip) for 64-byte chunks, 16-byte aligned
//     input and a class map with one catch-all class and at most 8 other bytes:
//     five kernels with no inter-workgroup waiting;
//   * the generic single-pass kernel here (any table, chunk size 1..64): one
//     workgroup per tile of 1024 chunks, bytes staged through LDS, the two
//     device-wide scans (state vectors, then count carries) as decoupled
//     look-backs in which every wave reads 64 predecessors per round; a
//     state-transition vector is one byte per state in two VGPRs, so a composite
//     is two v_perm_b32 byte selects (ParPaRaw keeps such small arrays in
//     registers with bit-field insert/extract, Fig. 8).
#include <algorithm>

#include "ppr_csv_common.h"
#include "ppr_scan.h"

namespace ppr {

struct LookCtx {
    WsHeader* hdr;
    uint64_t* statA;
    StatB* statB;
    uint32_t epoch;
    uint32_t expect_cols;  // expected fields per record (0: none)
    uint32_t start_col;    // column of the field open at the input's start (0: a record starts there)
    uint32_t partial;      // more input follows: no final field, the end state may be non-accepting
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
    uint32_t cols[4 * NW];
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
    wave_lower_min(&c.hdr->err_min, err);  // chunks holding an INVALID byte: one atomic per wave at most
    Carry cex, ctot;
    block_scan<NW>(cr, carry_identity(), cex, ctot, sh->wcar, CarryComb{});

    if (tile == 0) {
        if (tid == 0) {
            Carry z = carry_identity();
            z.colabs = 1;  // the input starts in record 0 at column start_col
            z.colv = c.start_col;
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
        RecStats st = rec_stats_none();  // fields per record, over the records this chunk's fields end
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
                note_record(st, col + 1u, rec, c.expect_cols);
                ++rec;
                col = 0;
            } else {
                ++col;
            }
            bits &= bits - 1;
        }
        if (tile == num_tiles - 1 && tid == 0 && !sh->last_rec && !c.partial) {  // the final field ends the last record
            const Carry I = carry_op(P, ctot);
            note_record(st, I.colv + 1u, I.nr, c.expect_cols);
        }
        // the tile's per-record counts, into the call's
        publish_rec_stats<NW>(st.cmin, st.cmax, st.bad, st.fbad, sh->cols, &c.hdr->cols_min, &c.hdr->cols_max,
                              &c.hdr->bad_records, &c.hdr->first_bad);
    }

    if (tile == num_tiles - 1 && tid == 0) {
        const Carry I = carry_op(P, ctot);
        const uint32_t final_field = (c.partial || sh->last_rec) ? 0u : 1u;
        c.hdr->tail_start = I.lt;
        c.hdr->tail_col = I.colv;
        if (final_field && I.nf < o.cap) {
            o.rec[I.nf] = I.nr;
            o.col[I.nf] = I.colv;
            o.off[I.nf] = I.lt;
            o.len[I.nf] = n - I.lt;
        }
        c.hdr->n_fields = (uint64_t)I.nf + final_field;
        c.hdr->n_records = (uint64_t)I.nr + final_field;
        c.hdr->end_state = end_state;
        c.hdr->error_pos = (c.partial || end_accepting) ? (int64_t)-1 : (int64_t)n;  // before err_min is applied
    }
}

// Resets the workspace header (workgroup 0) and clears the look-back statuses
// (all workgroups: n_stat 16-byte words from stat).
__global__ void csv_reset_kernel(WsHeader* hdr, uint32_t n, uint32_t start_state, uint32_t accept_mask,
                                 uint32_t start_col, uint32_t partial, uint4* stat, uint64_t n_stat)
{
    clear_status(stat, n_stat);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        hdr->tile_counter = 0;
        hdr->fault = 0;
        hdr->err_min = 0xffffffffu;
        hdr->last_rec = 0;
        hdr->path = PPR_PATH_SINGLE_PASS;
        hdr->cols_min = 0xffffffffu;
        hdr->cols_max = 0;
        hdr->bad_records = 0;
        hdr->first_bad = 0xffffffffu;
        if (n == 0) {  // nothing to parse: the results of an empty input
            hdr->n_fields = 0;
            hdr->n_records = 0;
            hdr->end_state = start_state;
            hdr->error_pos = (partial || ((accept_mask >> start_state) & 1u)) ? -1 : 0;
            hdr->tail_start = 0;
            hdr->tail_col = start_col;
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
        // tiles in the order workgroups start (not blockIdx order): a tile only
        // waits in its look-backs on tiles that running workgroups already hold
        s_tile = atomicAdd(&p.look.hdr->tile_counter, 1u);
        sh.last_rec = 0;
    }
    if (tid < 256) s_cls[tid] = p.cls[tid];
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

// The table-driven path an automatic choice takes, the faster one on MI355X:
// the fused kernel (two launches) for inputs up to kFusedMaxAuto bytes, where
// the streaming kernels' four launches cost more than their throughput gains
// (measured on the quote-heavy CSV: 42 against 50 us at 1 MiB, 47 against
// 49 us at 8 MiB, 64 against 56 us at 16 MiB); the streaming kernels above.
constexpr uint64_t kFusedMaxAuto = 8ull << 20;

static uint32_t auto_table_path(uint64_t n) { return n <= kFusedMaxAuto ? PPR_PATH_FUSED : PPR_PATH_STREAMING; }

static uint32_t chunk_of(const ppr_parse_opts_t* o)
{
    uint32_t L = o ? o->chunk_bytes : 0u;
    if (L == 0) L = kFastChunk;  // the default: 64 bytes per thread
    return L <= (uint32_t)kMaxChunk ? L : 0u;
}

// generic path: header (256 B), then the two status arrays
static WsLayout csv_layout(uint64_t n, uint32_t L)
{
    const uint64_t tile = (uint64_t)kBlock * L;
    const uint64_t tiles = (n + tile - 1) / tile;
    WsLayout w;
    w.tiles = tiles;
    w.off_a = 256;
    w.off_b = align_up(w.off_a + tiles * sizeof(uint64_t), 256);
    w.total = align_up(w.off_b + tiles * sizeof(StatB), 256);
    return w;
}

// Fast-path eligibility and its tables: a catch-all class, at most 8 other
// bytes separable by a 3-bit slot of two bit fields (ppr_slots.h), at most 8
// tracked states.
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
    cb = d->n_classes <= 4 ? 2 : d->n_classes <= 8 ? 3 : 4;
    const uint32_t catch_code = (1u << cb) - 1u;
    uint8_t code_of[PPR_MAX_CLASSES];
    uint32_t next_code = 0;
    for (uint32_t c = 0; c < d->n_classes; ++c) code_of[c] = c == K ? (uint8_t)catch_code : (uint8_t)next_code++;
    uint8_t special_code[8];
    for (int i = 0; i < ns; ++i) special_code[i] = code_of[cm[specials[i]]];
    if (!build_slot_tables(specials, special_code, ns, catch_code, f.slots)) return false;
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
    f.quiet_abs = 1;
    for (int c = 0; c < 16; ++c)
        if (f.tag[nt][c] == PPR_TAG_FIELD || f.tag[nt][c] == PPR_TAG_RECORD) f.quiet_abs = 0;
    return true;
}

}  // namespace ppr

using namespace ppr;

extern "C" size_t ppr_parse_workspace_bytes(uint64_t n, const ppr_parse_opts_t* opts)
{
    const uint32_t L = chunk_of(opts);
    if (!L || n > kMaxInput) return 0;
    uint64_t total = csv_layout(n, L).total;
    if (L == (uint32_t)kFastChunk) total = std::max(total, fast_layout(n).total);
    return (size_t)total;
}

namespace ppr {

// Enqueues one parse. compact: the workspace is a fixed scratch buffer that
// only holds the single-pass paths' statuses, so the streaming kernels (whose
// intermediates take a quarter of the input) are never chosen; a
// table-driven input then runs the fused kernel, whose workspace is the
// header, the step tables and 72 bytes per 32 KiB tile.
int parse_enqueue(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                  const ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream,
                  bool compact)
{
    int rc = validate_dfa(dfa, class_map);
    if (rc) return rc;
    // a parse that continues an earlier call's input: its start state and the open field's column
    const uint32_t flags = opts ? opts->flags : 0u;
    if (flags & ~(uint32_t)(PPR_PARSE_CONTINUE | PPR_PARSE_PARTIAL)) return PPR_EINVAL;
    ppr_dfa_t dfa_cont;
    uint32_t start_col = 0;
    if (flags & PPR_PARSE_CONTINUE) {
        if (opts->start_state >= dfa->n_states) return PPR_EINVAL;
        dfa_cont = *dfa;
        dfa_cont.start_state = opts->start_state;
        dfa = &dfa_cont;
        start_col = opts->start_column;
    }
    const uint32_t partial = (flags & PPR_PARSE_PARTIAL) ? 1u : 0u;
    if (!out || !d_ws || (n && !d_bytes)) return PPR_EINVAL;
    if (n > kMaxInput) return PPR_ETOOBIG;
    const uint32_t L = chunk_of(opts);
    if (!L) return PPR_EINVAL;
    if (out->cap_fields && (!out->record_idx || !out->column_ids || !out->field_offsets || !out->field_lengths))
        return PPR_EINVAL;
    if ((uintptr_t)d_ws & 255u) return PPR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    WsHeader* hdr = (WsHeader*)ws;
    const uint32_t accept = dfa->accept_mask & ((1u << dfa->n_states) - 1u);
    OutArrays oa{out->record_idx, out->column_ids, out->field_offsets, out->field_lengths, out->cap_fields};

    const uint32_t want = opts ? opts->path : 0u;
    if (want > PPR_PATH_FUSED) return PPR_EINVAL;
    const uint32_t expect = opts ? opts->expected_columns : 0u;
    // table-driven paths: 64-byte chunks, 16-byte aligned input, a table they can encode
    if (n && want != PPR_PATH_SINGLE_PASS && L == (uint32_t)kFastChunk && ((uintptr_t)d_bytes & 15u) == 0) {
        FastParams f;
        memset(&f, 0, sizeof f);
        int cb = 0;
        bool v8 = false;
        if (prepare_fast(dfa, class_map, f, cb, v8)) {
            const uint32_t path =
                compact ? PPR_PATH_FUSED
                        : want == PPR_PATH_STREAMING || want == PPR_PATH_FUSED ? want : auto_table_path(n);
            const FastLayout fl = path == PPR_PATH_FUSED ? fused_layout(n) : fast_layout(n);
            if (ws_bytes < fl.total) return PPR_EWORKSPACE;
            f.in = d_bytes;
            f.n = (uint32_t)n;
            f.num_tiles = (uint32_t)fl.tiles;
            f.out = oa;
            f.hdr = hdr;
            f.tabs = (uint32_t*)(ws + fl.tabs);
            f.idx = ws + fl.idx;
            f.cvec_lo = (uint32_t*)(ws + fl.cvec_lo);
            f.cvec_hi = (uint32_t*)(ws + fl.cvec_hi);
            f.num_super = (uint32_t)((fl.tiles + 1) / 2);
            f.num_ranges = (uint32_t)std::min<uint64_t>(f.num_super, kMaxRanges);
            f.tile_vec = (uint64_t*)(ws + fl.tile_vec);
            f.range_vec = (uint64_t*)(ws + fl.range_vec);
            f.range_state = (uint32_t*)(ws + fl.range_state);
            f.range_carry = (uint4*)(ws + fl.range_carry);
            f.range_err = (uint32_t*)(ws + fl.range_err);
            f.stat_vec = (uint64_t*)(ws + fl.stat_vec);
            f.stat_carry = (StatB*)(ws + fl.stat_carry);
            f.spec = (uint32_t*)(ws + fl.stat_carry);  // (8 of its 16 words per tile)
            f.epoch = next_epoch();
            f.path = path;
            f.expect_cols = expect;
            f.start_col = start_col;
            f.partial = partial;
            return launch_csv_fast(f, cb, v8, opts, s);
        }
    }

    const WsLayout lay = csv_layout(n, L);
    if (ws_bytes < lay.total) return PPR_EWORKSPACE;
    stage_event(opts, 0, s);
    const uint64_t stat_bytes = lay.total - lay.off_a;  // statuses A and B, with their padding
    hipLaunchKernelGGL(csv_reset_kernel, dim3(clear_grid(stat_bytes)), dim3(256), 0, s, hdr, (uint32_t)n,
                       dfa->start_state, accept, start_col, partial, (uint4*)(ws + lay.off_a), stat_bytes / 16);
    stage_event(opts, 1, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    if (n == 0) return PPR_OK;
    LookCtx lc{hdr, (uint64_t*)(ws + lay.off_a), (StatB*)(ws + lay.off_b), next_epoch(), expect, start_col, partial};

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
    stage_event(opts, 2, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    return PPR_OK;
}

}  // namespace ppr

extern "C" int ppr_parse_async(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                               const ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts,
                               void* stream)
{
    return parse_enqueue(d_bytes, n, dfa, class_map, out, d_ws, ws_bytes, opts, stream, false);
}

namespace ppr {

// The workspace header's host copy for blocking calls: one pinned buffer per
// host thread, allocated on the thread's first call and kept until the process
// ends (256 bytes). The copy is then one DMA into it; a pageable destination is
// staged through the runtime's own pinned buffer, a second copy with its own
// latency on every call. A thread's calls use it one at a time (each waits for
// its copy). nullptr if the allocation failed: the caller reads into the stack.
WsHeader* pinned_header()
{
    thread_local WsHeader* p = nullptr;
    thread_local bool tried = false;
    if (!tried) {
        tried = true;
        if (hipHostMalloc((void**)&p, sizeof(WsHeader), hipHostMallocPortable) != hipSuccess) {
            p = nullptr;
            (void)hipGetLastError();  // not left for a later launch check to report
        }
    }
    return p;
}

// ppr_parse_results; may_alloc = false (the entry point that allocates nothing)
// reads the header into the stack instead of the pinned buffer.
int parse_results(const void* d_ws, ppr_parse_out_t* out, hipStream_t s, bool may_alloc)
{
    if (!d_ws || !out) return PPR_EINVAL;
    WsHeader local;
    WsHeader* dst = may_alloc ? pinned_header() : nullptr;
    if (!dst) dst = &local;
    if (hipMemcpyAsync(dst, d_ws, sizeof(WsHeader), hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    const WsHeader h = *dst;
    out->n_fields = h.n_fields;
    out->n_records = h.n_records;
    // the first INVALID byte wins over a non-accepting end state
    out->error_pos = h.err_min != 0xffffffffu ? (int64_t)h.err_min : h.error_pos;
    out->end_state = h.end_state;
    out->path = h.path;
    out->min_columns = h.cols_min != 0xffffffffu ? h.cols_min : 0u;
    out->max_columns = h.cols_max;
    out->bad_records = h.bad_records;
    out->first_bad_record = h.first_bad != 0xffffffffu ? (int64_t)h.first_bad : (int64_t)-1;
    out->tail_start = h.tail_start;
    out->tail_column = h.tail_col;
    if (h.fault) return PPR_EHIP;
    return out->n_fields > out->cap_fields ? PPR_ECAPACITY : PPR_OK;
}

}  // namespace ppr

extern "C" int ppr_parse_results(const void* d_ws, uint64_t n, ppr_parse_out_t* out, void* stream)
{
    (void)n;
    return parse_results(d_ws, out, (hipStream_t)stream, true);
}

extern "C" int ppr_parse(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                         ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream)
{
    int rc = ppr_parse_async(d_bytes, n, dfa, class_map, out, d_ws, ws_bytes, opts, stream);
    if (rc) return rc;
    return ppr_parse_results(d_ws, n, out, stream);
}
