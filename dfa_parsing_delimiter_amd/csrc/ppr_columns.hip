// Columnar partition of parsed fields: per-column concatenated symbol strings
// (CSS) and their index.
//
// Method: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw
// Data", Sec. 3 (the symbols partitioned by column with a stable sort on their
// column tags: a histogram of the partitions, an exclusive sum over it, a
// scatter; each column's symbols then lie together, its CSS; an index gives
// each field's record, offset into the CSS and number of symbols, from a
// run-length encoding of the record tags and an exclusive sum, Fig. 5) and the
// specialisations passage (an inline-terminated CSS, each field followed by a
// terminator byte, and a vector-delimited CSS with an auxiliary boolean
// vector, Fig. 6).
//
// MI355X mapping. The parse already gives one entry per field (record, column,
// offset, length), so the partition moves fields, not bytes, until the very
// last step, and it needs one pass per step rather than one per digit (columns
// fit one key of at most 12 bits):
//   hist     per block of fields, a count per column (LDS atomics), stored
//            column-major: entry (c, b);
//   scan     exclusive sum over those counts in column-major order (single
//            pass, decoupled look-back): where block b's fields of column c go;
//   scatter  per block, rounds of 256 fields: a field's place among the
//            round's fields of its column (wave multisplit: ballots over the
//            key bits, then the waves' counts in LDS), plus the running count
//            of its column in the block; its index entry is written there
//            (record, length, source offset), which keeps each column's fields
//            in input order;
//   scan     exclusive sum of length (+1 per field with a terminator slot)
//            over the partitioned entries: every field's CSS offset, and the
//            CSS size;
//   copy     one lane per field copies its bytes in 16-byte pieces (unaligned
//            global loads and stores), then its slot.
#include <algorithm>

#include "ppr_scan.h"

namespace ppr {
namespace {

constexpr int kColBlock = 256;  // threads of every kernel here
constexpr int kColWaves = kColBlock / kWave;
constexpr uint32_t kColMaxColumns = 4096;
constexpr int kScanPer = 16;  // elements per thread of the scan kernel
constexpr int kScanTile = kColBlock * kScanPer;

struct ColHeader {
    uint32_t bad_column;  // a field's column id was not below n_columns
    uint32_t fault;       // a look-back gave up (never expected)
    uint32_t ctr[2];      // tile counters of the two scans
    uint32_t total[2];    // the scans' totals
};

// fields per block of the histogram and scatter kernels: 16 per thread, more
// for many columns, so that the column-major histogram stays near a byte per
// field
inline uint32_t fields_per_block(uint32_t n_columns)
{
    uint32_t per = 16;
    while ((uint64_t)per * kColBlock < (uint64_t)n_columns * 8 && per < 1024) per *= 2;
    return per * kColBlock;
}

struct ColLayout {
    uint64_t blocks, tiles, hist, scan_stat, ent_src, total;
};

inline ColLayout col_layout(uint64_t nf, uint32_t n_columns)
{
    ColLayout L;
    const uint32_t B = fields_per_block(n_columns);
    L.blocks = (nf + B - 1) / B;
    const uint64_t hist_n = L.blocks * n_columns;
    L.tiles = std::max<uint64_t>(
        std::max((hist_n + kScanTile - 1) / kScanTile, (nf + kScanTile - 1) / kScanTile), 1);
    L.hist = 256;
    L.scan_stat = align_up(L.hist + std::max<uint64_t>(hist_n, 1) * 4, 256);
    L.ent_src = align_up(L.scan_stat + 2 * L.tiles * 8, 256);
    L.total = align_up(L.ent_src + std::max<uint64_t>(nf, 1) * 4, 256);
    return L;
}

// Resets the header (workgroup 0) and clears both scans' look-back statuses
// (all workgroups: n_stat 16-byte words from stat).
__global__ void cols_reset_kernel(ColHeader* h, uint4* stat, uint64_t n_stat)
{
    clear_status(stat, n_stat);
    if (blockIdx.x == 0 && threadIdx.x == 0) *h = ColHeader{0u, 0u, {0u, 0u}, {0u, 0u}};
}

// per block of B fields, the count of each column, into hist[c * blocks + b]
__global__ void __launch_bounds__(kColBlock) cols_hist_kernel(const uint32_t* col, uint64_t nf, uint32_t n_columns,
                                                              uint32_t B, uint64_t blocks, uint32_t* hist,
                                                              ColHeader* h)
{
    __shared__ uint32_t s_h[kColMaxColumns];
    for (uint32_t c = threadIdx.x; c < n_columns; c += kColBlock) s_h[c] = 0;
    __syncthreads();
    const uint64_t f0 = (uint64_t)blockIdx.x * B, f1 = std::min<uint64_t>(f0 + B, nf);
    uint32_t bad = 0;
    for (uint64_t i = f0 + threadIdx.x; i < f1; i += kColBlock) {
        const uint32_t c = col[i];
        if (c < n_columns) atomicAdd(&s_h[c], 1u);
        else bad = 1;
    }
    if (__ballot(bad) && lane_id() == 0) atomicOr(&h->bad_column, 1u);
    __syncthreads();
    for (uint32_t c = threadIdx.x; c < n_columns; c += kColBlock) hist[(uint64_t)c * blocks + blockIdx.x] = s_h[c];
}

// Single-pass exclusive scan of x[i] + add over n elements into y (in place
// allowed), the total into *total. Tiles in the order workgroups start (an
// atomic counter), decoupled look-back over 32-bit sum statuses.
struct SumPoll {
    const uint64_t* stat;
    uint32_t epoch;
    __device__ uint32_t operator()(int64_t u, uint32_t& out) const
    {
        const uint64_t w = ld_relaxed(&stat[u]);
        const uint32_t f = status_flag(w, epoch);
        if (f) out = status_payload(w);
        return f;
    }
};

__global__ void __launch_bounds__(kColBlock) cols_scan_kernel(const uint32_t* x, uint32_t* y, uint64_t n, uint32_t add,
                                                              uint64_t* stat, uint32_t epoch, uint32_t* ctr,
                                                              uint32_t* total, uint32_t* fault)
{
    __shared__ uint32_t s_tile, s_wave[kColWaves], s_part[kColWaves];
    __shared__ int s_first[kColWaves];
    if (threadIdx.x == 0) s_tile = atomicAdd(ctr, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t base = (uint64_t)tile * kScanTile + (uint64_t)threadIdx.x * kScanPer;
    uint32_t v[kScanPer], sum = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
        v[k] = base + k < n ? x[base + k] + add : 0u;
        sum += v[k];
    }
    uint32_t excl, tot;
    block_scan<kColWaves>(sum, 0u, excl, tot, s_wave, AddU32{});
    uint32_t pre = 0;
    if (tile == 0) {
        if (threadIdx.x == 0) st_relaxed(&stat[0], status_word(epoch, kFlagIncl, tot));
    } else {
        if (threadIdx.x == 0) st_relaxed(&stat[tile], status_word(epoch, kFlagAgg, tot));
        pre = lookback<kColWaves>(tile, 0u, SumPoll{stat, epoch}, AddU32{}, s_part, s_first, fault);
        if (threadIdx.x == 0) st_relaxed(&stat[tile], status_word(epoch, kFlagIncl, pre + tot));
    }
    uint32_t run = pre + excl;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
        if (base + k < n) y[base + k] = run;
        run += v[k];
    }
    const uint64_t tiles = (n + kScanTile - 1) / kScanTile;
    if (tile == tiles - 1 && threadIdx.x == 0) *total = pre + tot;
}

// Scatter: the index entries of block b's fields, each at
//   (fields of lower columns) + (this column's fields in earlier blocks)   [the scanned histogram]
//   + (its column's fields earlier in the block)                           [running counts, LDS]
// so that each column's entries keep the fields' order.
__global__ void __launch_bounds__(kColBlock) cols_scatter_kernel(const uint32_t* rec, const uint32_t* col,
                                                                 const uint32_t* off, const uint32_t* len, uint64_t nf,
                                                                 uint32_t n_columns, uint32_t key_bits, uint32_t B,
                                                                 uint64_t blocks, const uint32_t* hist_excl,
                                                                 uint32_t* ent_rec, uint32_t* ent_len,
                                                                 uint32_t* ent_src)
{
    __shared__ uint32_t s_base[kColMaxColumns];
    __shared__ uint16_t s_wc[kColWaves][kColMaxColumns];
    const uint32_t lane = (uint32_t)lane_id(), w = threadIdx.x / kWave;
    for (uint32_t c = threadIdx.x; c < n_columns; c += kColBlock) {
        s_base[c] = hist_excl[(uint64_t)c * blocks + blockIdx.x];
#pragma unroll
        for (int k = 0; k < kColWaves; ++k) s_wc[k][c] = 0;
    }
    __syncthreads();
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t f0 = (uint64_t)blockIdx.x * B, f1 = std::min<uint64_t>(f0 + B, nf);
    for (uint64_t r0 = f0; r0 < f1; r0 += kColBlock) {
        const uint64_t i = r0 + threadIdx.x;
        uint32_t key = i < f1 ? col[i] : 0u;
        // (a column id out of range was reported by the histogram kernel; its field is left out here)
        const bool valid = i < f1 && key < n_columns;
        key = valid ? key : 0u;
        // the lanes of this wave with the same key (a column id below n_columns: checked by the histogram)
        uint64_t peers = __ballot(valid);
        for (uint32_t bit = 0; bit < key_bits; ++bit) {
            const uint64_t m = __ballot((key >> bit) & 1u);
            peers &= ((key >> bit) & 1u) ? m : ~m;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & lt), cnt = (uint32_t)__popcll(peers);
        const bool last = valid && (peers >> lane) == 1ull;  // the wave's last lane with this key
        if (last) s_wc[w][key] = (uint16_t)cnt;
        __syncthreads();
        uint32_t pre = 0, later = 0;
        if (valid) {
#pragma unroll
            for (int k = 0; k < kColWaves; ++k) {
                const uint32_t wc = s_wc[k][key];
                if (k < (int)w) pre += wc;
                if (k > (int)w) later += wc;
            }
            const uint32_t j = s_base[key] + pre + rank;
            ent_rec[j] = rec[i];
            ent_len[j] = len[i];
            ent_src[j] = off[i];
        }
        __syncthreads();
        if (last) {
            if (later == 0) s_base[key] += pre + cnt;  // the round's last field of this key advances its count
            s_wc[w][key] = 0;
        }
        __syncthreads();
    }
}

// the columns' first entries and first CSS bytes
__global__ void cols_bounds_kernel(const uint32_t* hist_excl, uint64_t blocks, uint32_t n_columns, uint64_t nf,
                                   const uint32_t* ent_off, const uint32_t* css_total, uint32_t* first_field,
                                   uint32_t* first_byte)
{
    for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c <= n_columns; c += gridDim.x * blockDim.x) {
        const uint32_t f = c < n_columns ? (blocks ? hist_excl[(uint64_t)c * blocks] : 0u) : (uint32_t)nf;
        first_field[c] = f;
        first_byte[c] = f < nf ? ent_off[f] : *css_total;
    }
}

// one lane per field: its bytes to css[ent_off[j] ...] in 16-byte pieces, then
// its slot (terminator, or 0 with aux = 1); aux = 0 over the field's bytes.
// Nothing is written at or beyond css_cap.
__global__ void __launch_bounds__(kColBlock) cols_copy_kernel(const uint8_t* in, uint64_t n, const uint32_t* ent_src,
                                                              const uint32_t* ent_len, const uint32_t* ent_off,
                                                              uint64_t nf, uint8_t* css, uint8_t* aux, uint64_t cap,
                                                              uint32_t slot, uint32_t term, const ColHeader* h)
{
    const uint64_t j = (uint64_t)blockIdx.x * kColBlock + threadIdx.x;
    if (j >= nf || h->bad_column) return;  // (with a bad column id some entries were never written)
    const uint32_t L = ent_len[j];
    if ((uint64_t)ent_src[j] + L > n) return;  // (never for a parse's own fields)
    const uint8_t* s = in + ent_src[j];
    const uint64_t d0 = ent_off[j];
    const uint64_t room = d0 < cap ? cap - d0 : 0;
    const uint32_t L_in = (uint32_t)std::min<uint64_t>(L, room);
    uint8_t* d = css + d0;
    uint32_t k = 0;
    for (; k + 16 <= L_in; k += 16) {
        uint4 x;
        __builtin_memcpy(&x, s + k, 16);
        __builtin_memcpy(d + k, &x, 16);
        if (aux) {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            __builtin_memcpy(aux + d0 + k, &z, 16);
        }
    }
    for (; k < L_in; ++k) {
        d[k] = s[k];
        if (aux) aux[d0 + k] = 0;
    }
    if (slot && L < room) {
        d[L] = (uint8_t)term;
        if (aux) aux[d0 + L] = 1;
    }
}

}  // namespace
}  // namespace ppr

using namespace ppr;

extern "C" PPR_API size_t ppr_columns_workspace_bytes(uint64_t n_fields, uint32_t n_columns)
{
    if (n_columns > kColMaxColumns || n_fields >= 0xffffffffull) return 0;
    return (size_t)col_layout(n_fields, n_columns).total;
}

extern "C" PPR_API int ppr_columns(const uint8_t* d_bytes, uint64_t n, const uint32_t* d_rec, const uint32_t* d_col,
                                   const uint32_t* d_off, const uint32_t* d_len, uint64_t n_fields, uint32_t n_columns,
                                   uint32_t mode, uint32_t terminator, ppr_columns_out_t* out, void* d_ws,
                                   size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream)
{
    if (!out || mode > PPR_CSS_VECTOR || terminator > 255 || n_columns > kColMaxColumns) return PPR_EINVAL;
    // every CSS offset (at most n bytes plus a slot per field) fits 32 bits
    if (n_fields >= 0xffffffffull || n + (mode == PPR_CSS_INDEXED ? 0u : n_fields) >= 0xffffffffull)
        return PPR_ETOOBIG;
    if (n_fields && (!d_bytes || !d_rec || !d_col || !d_off || !d_len || !n_columns)) return PPR_EINVAL;
    if (!out->rec || !out->css_off || !out->length || !out->col_first_field || !out->col_first_byte || !d_ws)
        return PPR_EINVAL;
    if ((out->css_cap && !out->css) || (mode == PPR_CSS_VECTOR && out->css_cap && !out->aux)) return PPR_EINVAL;
    if ((uintptr_t)d_ws & 255u) return PPR_EWORKSPACE;
    const ColLayout L = col_layout(n_fields, n_columns);
    if (ws_bytes < L.total) return PPR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    ColHeader* h = (ColHeader*)ws;
    uint32_t* hist = (uint32_t*)(ws + L.hist);
    uint64_t* stat = (uint64_t*)(ws + L.scan_stat);  // two arrays of L.tiles statuses, one per scan
    uint32_t* ent_src = (uint32_t*)(ws + L.ent_src);
    const uint32_t B = fields_per_block(n_columns);
    const uint32_t slot = mode == PPR_CSS_INDEXED ? 0u : 1u;
    uint32_t key_bits = 0;
    while ((1u << key_bits) < n_columns) ++key_bits;
    const uint32_t e1 = next_epoch(), e2 = next_epoch();

    stage_event(opts, 0, s);
    hipLaunchKernelGGL(cols_reset_kernel, dim3(clear_grid(2 * L.tiles * 8)), dim3(256), 0, s, h, (uint4*)stat, L.tiles);
    stage_event(opts, 1, s);
    if (n_fields) {
        hipLaunchKernelGGL(cols_hist_kernel, dim3((uint32_t)L.blocks), dim3(kColBlock), 0, s, d_col, n_fields,
                           n_columns, B, L.blocks, hist, h);
        stage_event(opts, 2, s);
        const uint64_t hist_n = L.blocks * n_columns;
        hipLaunchKernelGGL(cols_scan_kernel, dim3((uint32_t)((hist_n + kScanTile - 1) / kScanTile)), dim3(kColBlock), 0,
                           s, hist, hist, hist_n, 0u, stat, e1, &h->ctr[0], &h->total[0], &h->fault);
        stage_event(opts, 3, s);
        hipLaunchKernelGGL(cols_scatter_kernel, dim3((uint32_t)L.blocks), dim3(kColBlock), 0, s, d_rec, d_col, d_off,
                           d_len, n_fields, n_columns, key_bits, B, L.blocks, hist, out->rec, out->length, ent_src);
        stage_event(opts, 4, s);
        hipLaunchKernelGGL(cols_scan_kernel, dim3((uint32_t)((n_fields + kScanTile - 1) / kScanTile)),
                           dim3(kColBlock), 0, s, out->length, out->css_off, n_fields, slot, stat + L.tiles, e2,
                           &h->ctr[1], &h->total[1], &h->fault);
        stage_event(opts, 5, s);
    } else {
        for (uint32_t i = 2; i <= 5; ++i) stage_event(opts, i, s);
    }
    hipLaunchKernelGGL(cols_bounds_kernel, dim3((n_columns + 256) / 256), dim3(256), 0, s, hist, L.blocks, n_columns,
                       n_fields, out->css_off, &h->total[1], out->col_first_field, out->col_first_byte);
    stage_event(opts, 6, s);
    if (n_fields)
        hipLaunchKernelGGL(cols_copy_kernel, dim3((uint32_t)((n_fields + kColBlock - 1) / kColBlock)), dim3(kColBlock),
                           0, s, d_bytes, n, ent_src, out->length, out->css_off, n_fields, out->css,
                           mode == PPR_CSS_VECTOR ? out->aux : nullptr, out->css_cap, slot,
                           mode == PPR_CSS_VECTOR ? 0u : terminator, h);
    stage_event(opts, 7, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    ColHeader hh;
    if (hipMemcpyAsync(&hh, h, sizeof hh, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    out->css_bytes = hh.total[1];
    if (hh.bad_column) return PPR_EINVAL;
    if (hh.fault) return PPR_EHIP;
    return out->css_bytes > out->css_cap ? PPR_ECAPACITY : PPR_OK;
}
