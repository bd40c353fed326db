// Single-pass data-parallel DFA parse of delimiter-separated bytes on gfx950.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", Sec. 3. Every thread owns a chunk of L bytes and runs one DFA instance
// per state over it, producing its state-transition vector (Fig. 2). An
// exclusive scan of the vectors under composition, seeded with the identity,
// gives each chunk its true start state. Each thread then re-simulates its chunk
// from that state and tags every byte (record delimiter, field delimiter,
// value, invalid), keeping the two delimiter bitmaps. Record counts (POPCNT +
// exclusive sum) and relative/absolute column offsets (Fig. 4) are scanned the
// same way, and every field is written out with its record, column, offset and
// length.
//
// MI355X mapping (not the page's CUDA design):
//   * one workgroup of 256 threads = one tile of 256*L bytes, staged once from
//     HBM into LDS with 16-byte loads; the tile is never re-read from HBM;
//   * tiles take their index from an atomic counter (dispatch order is not
//     assumed), and the device-wide scan is a decoupled look-back: each tile
//     publishes its aggregate, then its inclusive prefix; a 64-lane wave reads
//     64 predecessors per step;
//   * two look-backs in one kernel: the state vectors first (known right after
//     the first pass), then the field/record/column counts (known only after
//     the re-simulation);
//   * vectors are 8 bytes in two VGPRs and compose with v_perm_b32.
#include "ppr.h"
#include "ppr_device.h"
#include "ppr_host.h"

namespace ppr {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxChunk = 64;
constexpr uint32_t kNone = 0xffffffffu;

struct CsvParams {
    const uint8_t* in;
    uint32_t n, L, tile_bytes, num_tiles;
    uint32_t start_state, accept_mask, epoch, reserved;
    uint32_t* rec;
    uint32_t* col;
    uint32_t* off;
    uint32_t* len;
    uint64_t cap;
    WsHeader* hdr;
    uint64_t* statA;
    StatB* statB;
    uint32_t row_lo[PPR_MAX_CLASSES], row_hi[PPR_MAX_CLASSES];  // next-state vector of each class
    uint8_t nt[PPR_MAX_STATES][PPR_MAX_CLASSES];                // next | tag << 4
    uint8_t cls[256];
};

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

// exclusive scan over the block in thread order; total = composite of all threads
__device__ void block_scan_vec(Vec v, Vec& excl, Vec& total, Vec* s_wave)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    Vec inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        Vec o = shfl_up_vec(inc, d);
        if (lane >= d) inc = compose(o, inc);
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    Vec pre = vec_identity(), tot = vec_identity();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        Vec a = s_wave[i];
        if (i < w) pre = compose(pre, a);
        tot = compose(tot, a);
    }
    Vec ex = shfl_up_vec(inc, 1);
    if (lane == 0) ex = vec_identity();
    excl = compose(pre, ex);
    total = tot;
}

__device__ void block_scan_carry(const Carry& c, Carry& excl, Carry& total, Carry* s_wave)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    Carry inc = c;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        Carry o = shfl_up_carry(inc, d);
        if (lane >= d) inc = carry_op(o, inc);
    }
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    Carry pre = carry_identity(), tot = carry_identity();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        Carry a = s_wave[i];
        if (i < w) pre = carry_op(pre, a);
        tot = carry_op(tot, a);
    }
    Carry ex = shfl_up_carry(inc, 1);
    if (lane == 0) ex = carry_identity();
    excl = carry_op(pre, ex);
    total = tot;
}

// Wave 0 only. State before the first byte of `tile` (tile > 0).
__device__ uint32_t lookback_state(const CsvParams& p, uint32_t tile)
{
    const int lane = lane_id();
    Vec acc = vec_identity();  // composite of the tiles between the frontier and `tile`
    int64_t base = (int64_t)tile - 1;
    uint32_t spins = 0;
    for (;;) {
        const int64_t u = base - lane;
        const bool valid = u >= 0;
        uint64_t w = 0;
        uint32_t f = kFlagIncl;
        if (valid) {
            w = ld_relaxed(&p.statA[u]);
            f = status_flag(w, p.epoch);
        }
        while (!__all(f != 0)) {
            if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(&p.hdr->fault, 1u);
                return 0u;
            }
            __builtin_amdgcn_s_sleep(1);
            if (f == 0) {
                w = ld_relaxed(&p.statA[u]);
                f = status_flag(w, p.epoch);
            }
        }
        const uint64_t incl = __ballot(valid && f == kFlagIncl);
        const int j = incl ? __ffsll((unsigned long long)incl) - 1 : kWave;
        Vec a = (valid && lane < j) ? vec_unpack(status_payload(w)) : vec_identity();
        // ordered reduction: lane l+d holds an earlier tile than lane l
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            Vec o = shfl_down_vec(a, d);
            if (lane + d < kWave) a = compose(o, a);
        }
        acc = compose(shfl_vec(a, 0), acc);
        if (j < kWave) return vec_at(acc, shfl(status_payload(w), j));
        base -= kWave;
    }
}

__device__ __forceinline__ Carry load_carry(const StatB& s, uint32_t flag)
{
    const uint32_t* v = flag == kFlagIncl ? s.incl : s.agg;
    return {v[0], v[1], v[2], v[3], v[4], v[5]};
}

__device__ __forceinline__ void store_carry(StatB& s, const Carry& c, uint32_t epoch, uint32_t flag)
{
    uint32_t* v = flag == kFlagIncl ? s.incl : s.agg;
    v[0] = c.nf;
    v[1] = c.nr;
    v[2] = c.colv;
    v[3] = c.colabs;
    v[4] = c.lt;
    v[5] = c.err;
    st_release(&s.flag, status_word(epoch, flag, 0));
}

// Wave 0 only. Carry of all bytes before `tile` (tile > 0).
__device__ Carry lookback_carry(const CsvParams& p, uint32_t tile)
{
    const int lane = lane_id();
    Carry acc = carry_identity();
    int64_t base = (int64_t)tile - 1;
    uint32_t spins = 0;
    for (;;) {
        const int64_t u = base - lane;
        const bool valid = u >= 0;
        uint32_t f = kFlagIncl;
        if (valid) f = status_flag(ld_acquire(&p.statB[u].flag), p.epoch);
        while (!__all(f != 0)) {
            if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(&p.hdr->fault, 2u);
                return carry_identity();
            }
            __builtin_amdgcn_s_sleep(1);
            if (f == 0) f = status_flag(ld_acquire(&p.statB[u].flag), p.epoch);
        }
        const uint64_t incl = __ballot(valid && f == kFlagIncl);
        const int j = incl ? __ffsll((unsigned long long)incl) - 1 : kWave;
        Carry c = (valid && lane <= j) ? load_carry(p.statB[u], f) : carry_identity();
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            Carry o = shfl_down_carry(c, d);
            if (lane + d < kWave) c = carry_op(o, c);
        }
        acc = carry_op(shfl_carry(c, 0), acc);
        if (j < kWave) return acc;
        base -= kWave;
    }
}

__global__ void csv_reset_kernel(WsHeader* hdr, uint32_t n, uint32_t start_state, uint32_t accept_mask)
{
    if (threadIdx.x == 0) {
        hdr->tile_counter = 0;
        hdr->fault = 0;
        if (n == 0) {  // nothing to parse: the results of an empty input
            hdr->n_fields = 0;
            hdr->n_records = 0;
            hdr->end_state = start_state;
            hdr->error_pos = ((accept_mask >> start_state) & 1u) ? -1 : 0;
        }
    }
}

__global__ void __launch_bounds__(kBlock) csv_parse_kernel(CsvParams p)
{
    __shared__ __align__(16) uint8_t s_bytes[kBlock * kMaxChunk];
    __shared__ uint8_t s_cls[256];
    __shared__ uint8_t s_nt[PPR_MAX_STATES * PPR_MAX_CLASSES];
    __shared__ uint32_t s_rlo[PPR_MAX_CLASSES], s_rhi[PPR_MAX_CLASSES];
    __shared__ Vec s_wvec[kWaves];
    __shared__ Carry s_wcar[kWaves];
    __shared__ uint32_t s_tile, s_state, s_last_rec;
    __shared__ Carry s_prefix;

    const int tid = threadIdx.x;
    if (tid == 0) {
        s_tile = atomicAdd(&p.hdr->tile_counter, 1u);
        s_last_rec = 0;
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
    block_scan_vec(v, excl, tot, s_wvec);

    // the tile's start state
    if (tile == 0) {
        if (tid == 0) {
            s_state = p.start_state;
            st_relaxed(&p.statA[0], status_word(p.epoch, kFlagIncl, vec_at(tot, p.start_state)));
        }
    } else {
        if (tid == 0) st_relaxed(&p.statA[tile], status_word(p.epoch, kFlagAgg, vec_pack(tot)));
        if (tid < kWave) {
            const uint32_t s = lookback_state(p, tile);
            if (tid == 0) {
                s_state = s;
                st_relaxed(&p.statA[tile], status_word(p.epoch, kFlagIncl, vec_at(tot, s)));
            }
        }
    }
    __syncthreads();
    const uint32_t tile_state = s_state;

    // pass 2: one instance from the known state, tagging every byte
    uint32_t s = vec_at(excl, tile_state);
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
    if (my_len && chunk_abs + my_len == p.n) s_last_rec = (uint32_t)((RD >> (my_len - 1)) & 1u);

    const uint64_t T = FD | RD;
    Carry c;
    c.nf = (uint32_t)__popcll(T);
    c.nr = (uint32_t)__popcll(RD);
    if (RD) {
        const int hi = 63 - __clzll((long long)RD);
        const uint64_t above = hi == 63 ? 0ull : (~0ull << (hi + 1));
        c.colv = (uint32_t)__popcll(FD & above);
        c.colabs = 1;
    } else {
        c.colv = (uint32_t)__popcll(FD);
        c.colabs = 0;
    }
    c.lt = T ? chunk_abs + (uint32_t)(63 - __clzll((long long)T)) + 1u : 0u;
    c.err = err;
    Carry cex, ctot;
    block_scan_carry(c, cex, ctot, s_wcar);

    if (tile == 0) {
        if (tid == 0) {
            Carry z = carry_identity();
            z.colabs = 1;  // the input starts at column 0 of record 0
            s_prefix = z;
            store_carry(p.statB[0], carry_op(z, ctot), p.epoch, kFlagIncl);
        }
    } else {
        if (tid == 0) store_carry(p.statB[tile], ctot, p.epoch, kFlagAgg);
        if (tid < kWave) {
            Carry pre = lookback_carry(p, tile);
            if (tid == 0) {
                s_prefix = pre;
                store_carry(p.statB[tile], carry_op(pre, ctot), p.epoch, kFlagIncl);
            }
        }
    }
    __syncthreads();
    const Carry P = s_prefix;

    // emit this thread's fields
    {
        const Carry base = carry_op(P, cex);
        uint64_t fi = base.nf;
        uint32_t rec = base.nr, col = base.colv, off = base.lt;
        uint64_t bits = T;
        while (bits) {
            const uint32_t j = (uint32_t)__ffsll((unsigned long long)bits) - 1u;
            const uint32_t pos = chunk_abs + j;
            if (fi < p.cap) {
                p.rec[fi] = rec;
                p.col[fi] = col;
                p.off[fi] = off;
                p.len[fi] = pos - off;
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

    // the last tile closes the input: unterminated final field and the scalars
    if (tile == p.num_tiles - 1 && tid == 0) {
        const Carry I = carry_op(P, ctot);
        const uint32_t end_state = vec_at(tot, tile_state);
        const uint32_t final_field = s_last_rec ? 0u : 1u;
        if (final_field && I.nf < p.cap) {
            p.rec[I.nf] = I.nr;
            p.col[I.nf] = I.colv;
            p.off[I.nf] = I.lt;
            p.len[I.nf] = p.n - I.lt;
        }
        p.hdr->n_fields = (uint64_t)I.nf + final_field;
        p.hdr->n_records = (uint64_t)I.nr + final_field;
        p.hdr->end_state = end_state;
        p.hdr->error_pos = I.err != kNone ? (int64_t)I.err
                                          : (((p.accept_mask >> end_state) & 1u) ? (int64_t)-1 : (int64_t)p.n);
    }
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
    if (L == 0) L = 32;
    return L <= (uint32_t)kMaxChunk ? L : 0u;
}

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

    CsvParams p;
    memset(&p, 0, sizeof p);
    p.in = d_bytes;
    p.n = (uint32_t)n;
    p.L = L;
    p.tile_bytes = kBlock * L;
    p.num_tiles = (uint32_t)lay.tiles;
    p.start_state = dfa->start_state;
    p.accept_mask = accept;
    p.epoch = next_epoch();
    p.rec = out->record_idx;
    p.col = out->column_ids;
    p.off = out->field_offsets;
    p.len = out->field_lengths;
    p.cap = out->cap_fields;
    p.hdr = hdr;
    p.statA = (uint64_t*)(ws + lay.off_a);
    p.statB = (StatB*)(ws + lay.off_b);
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
    hipLaunchKernelGGL(csv_parse_kernel, dim3(p.num_tiles), dim3(kBlock), 0, s, p);
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
    out->error_pos = h.error_pos;
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
