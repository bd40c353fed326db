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
// offset, length), so the partition sorts fields, not bytes, and only the last
// step touches the bytes. Columns fit one key of at most 12 bits, so one
// counting pass replaces the digit passes of a radix sort:
//   hist   per block of 4096 fields, per column: the number of fields and
//          their CSS bytes (length + slot), stored column-major;
//   scan   exclusive sums over both (single pass, decoupled look-back): where
//          block b's fields of column c start, as an index entry and as a
//          CSS byte;
//   part   per block: a stable counting sort of its fields by column in LDS
//          (wave multisplit by ballots over the key bits), an exclusive sum of
//          the sorted fields' bytes, then the index entries written in sorted
//          order (each column's entries of the block are one run) and the
//          bytes copied in sorted order, 16-byte pieces spread over a wave's
//          lanes. Blocks are mapped to XCDs in contiguous runs, so that the
//          partial cache lines that neighbouring blocks write into a column's
//          run meet in one L2.
#include <algorithm>

#include "ppr_scan.h"

namespace ppr {
namespace {

constexpr int kColBlock = 256;  // threads of every kernel here
constexpr int kColWaves = kColBlock / kWave;
constexpr int kColPer = 16;                           // fields (or scan elements) per thread
constexpr uint32_t kColFields = kColBlock * kColPer;  // fields per block: 4096
constexpr uint32_t kColMaxColumns = 4096;
constexpr uint32_t kNoKey = 0xffffu;  // LDS key of a field left out (past the end, or a bad column id)

struct ColHeader {
    uint32_t bad_column;  // a field's column id was not below n_columns
    uint32_t fault;       // a look-back gave up (never expected)
    uint32_t ctr[2];      // tile counters of the two scans
    uint32_t total[2];    // the scans' totals: fields, CSS bytes
};

struct ColLayout {
    uint64_t blocks, tiles, cnt, bytes, scan_stat, total;
};

// Fields per block: 1024 (small blocks keep more of them resident per CU to
// hide their latency, and their input in L2 while their columns are copied),
// more for wide tables, up to 4096, so that each column has about 8 fields per
// block (runs in the index, and a histogram of at most an eighth of the
// fields).
inline uint32_t fields_per_block(uint32_t n_columns)
{
    uint32_t B = 1024;
    while (B < kColFields && B < 8ull * n_columns) B *= 2;
    return B;
}

inline ColLayout col_layout(uint64_t nf, uint32_t n_columns, uint32_t B)
{
    ColLayout L;
    L.blocks = (nf + B - 1) / B;
    const uint64_t hist_n = L.blocks * n_columns;
    L.tiles = std::max<uint64_t>((hist_n + kColFields - 1) / kColFields, 1);
    L.cnt = 256;
    L.bytes = align_up(L.cnt + std::max<uint64_t>(hist_n, 1) * 4, 256);
    L.scan_stat = align_up(L.bytes + std::max<uint64_t>(hist_n, 1) * 4, 256);
    L.total = align_up(L.scan_stat + 2 * L.tiles * 8, 256);
    return L;
}

// LDS of the partition kernel for blocks of B fields and NW waves: per field
// (length, CSS offset, sorted order, key, first piece), then per column (end,
// two offsets, per-wave counts)
inline size_t part_lds_bytes(uint32_t B, uint32_t n_columns, uint32_t NW)
{
    return (size_t)B * 16 + (size_t)n_columns * (3 * 4 + NW * 2);
}

constexpr size_t kLdsBudget = 150 * 1024;  // of the 160 KiB per CU: the dynamic part of one workgroup

// The block of workgroup `bid` in an XCD-aware order: workgroups are
// dispatched to the 8 XCDs in turn (XCD x runs x, x + 8, ...), and XCD x takes
// the x-th contiguous eighth of the blocks.
__device__ __forceinline__ uint32_t xcd_block(uint32_t bid, uint32_t nblocks)
{
    const uint32_t q = nblocks / 8u, r = nblocks % 8u, x = bid % 8u;
    return x * q + min(x, r) + bid / 8u;
}

// 16 consecutive u32 from a[i0] (0 at and past n); four 16-byte loads when all are in range
__device__ __forceinline__ void load16(const uint32_t* a, uint64_t i0, uint64_t n, uint32_t (&v)[kColPer])
{
    if (i0 + kColPer <= n) {
#pragma unroll
        for (int q = 0; q < kColPer / 4; ++q) {
            uint4 x;
            __builtin_memcpy(&x, a + i0 + 4 * q, 16);
            v[4 * q] = x.x;
            v[4 * q + 1] = x.y;
            v[4 * q + 2] = x.z;
            v[4 * q + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < kColPer; ++k) v[k] = i0 + k < n ? a[i0 + k] : 0u;
    }
}

__device__ __forceinline__ void store16(uint32_t* a, uint64_t i0, uint64_t n, const uint32_t (&v)[kColPer])
{
    if (i0 + kColPer <= n) {
#pragma unroll
        for (int q = 0; q < kColPer / 4; ++q) {
            const uint4 x = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            __builtin_memcpy(a + i0 + 4 * q, &x, 16);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kColPer; ++k)
            if (i0 + k < n) a[i0 + k] = v[k];
    }
}

// Resets the header (workgroup 0) and clears both scans' look-back statuses
// (all workgroups: n_stat 16-byte words from stat).
__global__ void cols_reset_kernel(ColHeader* h, uint4* stat, uint64_t n_stat)
{
    clear_status(stat, n_stat);
    if (blockIdx.x == 0 && threadIdx.x == 0) *h = ColHeader{0u, 0u, {0u, 0u}, {0u, 0u}};
}

// Per block of B fields and per column: the number of fields and their CSS
// bytes (length + slot), into cnt / bytes[c * blocks + b].
__global__ void __launch_bounds__(kColBlock) cols_hist_kernel(const uint32_t* col, const uint32_t* len, uint64_t nf,
                                                              uint32_t B, uint32_t n_columns, uint32_t slot,
                                                              uint64_t blocks, uint32_t* cnt, uint32_t* bytes,
                                                              ColHeader* h)
{
    __shared__ uint32_t s_c[kColMaxColumns], s_b[kColMaxColumns];
    for (uint32_t c = threadIdx.x; c < n_columns; c += kColBlock) s_c[c] = s_b[c] = 0;
    // thread t: fields t, t + 256, ... of the block (consecutive lanes,
    // consecutive fields); blocks in XCD-aware order, so that neighbouring
    // blocks' counts (neighbouring words of each column) meet in one L2
    const uint32_t hb = xcd_block(blockIdx.x, (uint32_t)blocks);
    const uint64_t f0 = (uint64_t)hb * B, f1 = std::min<uint64_t>(f0 + B, nf);
    uint32_t cv[kColPer], lv[kColPer];
#pragma unroll
    for (int k = 0; k < kColPer; ++k) {
        const uint64_t i = f0 + (uint64_t)k * kColBlock + threadIdx.x;
        cv[k] = i < f1 ? col[i] : 0u;
        lv[k] = i < f1 ? len[i] : 0u;
    }
    __syncthreads();
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < kColPer; ++k) {
        if (f0 + (uint64_t)k * kColBlock + threadIdx.x >= f1) continue;
        if (cv[k] < n_columns) {
            atomicAdd(&s_c[cv[k]], 1u);
            atomicAdd(&s_b[cv[k]], lv[k] + slot);
        } else {
            bad = 1;
        }
    }
    if (__ballot(bad) && lane_id() == 0) atomicOr(&h->bad_column, 1u);
    __syncthreads();
    for (uint32_t c = threadIdx.x; c < n_columns; c += kColBlock) {
        cnt[(uint64_t)c * blocks + hb] = s_c[c];
        bytes[(uint64_t)c * blocks + hb] = s_b[c];
    }
}

// Single-pass exclusive scan of x over n elements into y (in place allowed),
// the total into *total. Tiles of 4096 elements (16 consecutive per thread,
// 16-byte loads and stores) in the order workgroups start (an atomic counter),
// decoupled look-back over 32-bit sum statuses.
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

__global__ void __launch_bounds__(kColBlock) cols_scan_kernel(const uint32_t* x, uint32_t* y, uint64_t n,
                                                              uint64_t* stat, uint32_t epoch, uint32_t* ctr,
                                                              uint32_t* total, uint32_t* fault)
{
    __shared__ uint32_t s_tile, s_wave[kColWaves], s_part[kColWaves];
    __shared__ int s_first[kColWaves];
    if (threadIdx.x == 0) s_tile = atomicAdd(ctr, 1u);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t base = (uint64_t)tile * kColFields + (uint64_t)threadIdx.x * kColPer;
    uint32_t v[kColPer], sum = 0;
    load16(x, base, n, v);
#pragma unroll
    for (int k = 0; k < kColPer; ++k) sum += v[k];
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
    for (int k = 0; k < kColPer; ++k) {
        const uint32_t e = run;
        run += v[k];
        v[k] = e;
    }
    store16(y, base, n, v);
    const uint64_t tiles = (n + kColFields - 1) / kColFields;
    if (tile == tiles - 1 && threadIdx.x == 0) *total = pre + tot;
}

// the columns' first entries and first CSS bytes (block 0's scanned count and bytes)
__global__ void cols_bounds_kernel(const uint32_t* cnt_excl, const uint32_t* bytes_excl, uint64_t blocks,
                                   uint32_t n_columns, uint64_t nf, const uint32_t* css_total, uint32_t* first_field,
                                   uint32_t* first_byte)
{
    for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c <= n_columns; c += gridDim.x * blockDim.x) {
        const bool col = c < n_columns;
        first_field[c] = col ? (blocks ? cnt_excl[(uint64_t)c * blocks] : 0u) : (uint32_t)nf;
        first_byte[c] = col ? (blocks ? bytes_excl[(uint64_t)c * blocks] : 0u) : *css_total;
    }
}

struct PartParams {
    const uint8_t* in;
    uint64_t n;
    const uint32_t *rec, *col, *off, *len;
    uint64_t nf, blocks;
    uint32_t B;  // fields per block: 1024, 2048 or 4096
    uint32_t n_columns, key_bits, slot, term;
    const uint32_t *cnt_excl, *bytes_excl;  // scanned histograms, column-major
    uint32_t *ent_rec, *ent_off, *ent_len;  // the index
    uint8_t *css, *aux;
    uint64_t cap;
};

// the first L <= 16 bytes of x to d, as one 16-byte store or 8-, 4-, 2- and 1-byte stores
__device__ __forceinline__ void store_upto16(uint8_t* d, uint32_t L, const uint4& x)
{
    if (L == 16u) {
        __builtin_memcpy(d, &x, 16);
        return;
    }
    uint64_t lo = (uint64_t)x.x | ((uint64_t)x.y << 32);
    const uint64_t hi = (uint64_t)x.z | ((uint64_t)x.w << 32);
    uint32_t o = 0;
    if (L & 8u) {
        __builtin_memcpy(d, &lo, 8);
        lo = hi;
        o = 8;
    }
    if (L & 4u) {
        const uint32_t v = (uint32_t)lo;
        __builtin_memcpy(d + o, &v, 4);
        lo >>= 32;
        o += 4;
    }
    if (L & 2u) {
        const uint16_t v = (uint16_t)lo;
        __builtin_memcpy(d + o, &v, 2);
        lo >>= 16;
        o += 2;
    }
    if (L & 1u) d[o] = (uint8_t)lo;
}

// x with byte t (< 16) replaced by v
__device__ __forceinline__ uint4 put_byte(uint4 x, uint32_t t, uint32_t v)
{
    const uint32_t sh = 8u * (t & 3u), keep = ~(0xffu << sh), b = v << sh, q = t >> 2;
    x.x = q == 0 ? (x.x & keep) | b : x.x;
    x.y = q == 1 ? (x.y & keep) | b : x.y;
    x.z = q == 2 ? (x.z & keep) | b : x.z;
    x.w = q == 3 ? (x.w & keep) | b : x.w;
    return x;
}

__device__ __forceinline__ uint32_t byte_of(const uint4& x, uint32_t t)
{
    const uint32_t wd = t < 4 ? x.x : t < 8 ? x.y : t < 12 ? x.z : x.w;
    return (wd >> (8u * (t & 3u))) & 0xffu;
}

// The first m <= 16 bytes of a field's CSS extent starting at byte o of it:
// the data bytes from src + o (16 loaded at once where the input allows), the
// slot byte at L - o if it falls in the piece.
struct Piece {
    uint4 x;
    uint64_t d;  // CSS offset of the piece
    uint32_t m;  // bytes (0: none)
    uint32_t t;  // slot's place in the piece (16 or more: not in it)
};

__device__ __forceinline__ Piece load_piece(const PartParams& p, uint32_t src, uint32_t dst, uint32_t L, uint32_t o,
                                            uint32_t m)
{
    Piece q;
    q.d = (uint64_t)dst + o;
    q.m = m;
    q.t = L - o;
    if ((uint64_t)src + o + 16u <= p.n) {
        __builtin_memcpy(&q.x, p.in + src + o, 16);
    } else {  // a piece that ends at the input's end: its data bytes one by one
        q.x = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll 1
        for (uint32_t t = 0; t < m && o + t < L; ++t) q.x = put_byte(q.x, t, p.in[src + o + t]);
    }
    return q;
}

__device__ __forceinline__ void store_piece(const PartParams& p, const Piece& q)
{
    if (!q.m) return;
    const bool has_slot = p.slot && q.t < 16u;
    const uint4 v = has_slot ? put_byte(q.x, q.t, p.term) : q.x;
    if (q.d + q.m <= p.cap) {
        store_upto16(p.css + q.d, q.m, v);
        if (p.aux) {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            store_upto16(p.aux + q.d, q.m, has_slot ? put_byte(z, q.t, 1u) : z);
        }
    } else {
#pragma unroll 1
        for (uint32_t t = 0; t < q.m && q.d + t < p.cap; ++t) {
            p.css[q.d + t] = (uint8_t)byte_of(v, t);
            if (p.aux) p.aux[q.d + t] = (uint8_t)(has_slot && t == q.t);
        }
    }
}

// One block of up to B fields, NT threads: stable counting sort by column in
// LDS, the index entries in sorted order, then the CSS bytes.
template <int NT>
__global__ void __launch_bounds__(NT) cols_part_kernel(PartParams p)
{
    constexpr int NW = NT / kWave;
    extern __shared__ __align__(16) uint8_t s_dyn[];
    const uint32_t B = p.B;
    uint32_t* s_len = reinterpret_cast<uint32_t*>(s_dyn);  // [local field] length
    uint32_t* s_css = s_len + B;                             // [sorted] block-local CSS offset
    uint16_t* s_perm = reinterpret_cast<uint16_t*>(s_css + B);  // [sorted] local field
    uint16_t* s_key = s_perm + B;                            // [local field] column (kNoKey: none)
    uint32_t* s_pe = reinterpret_cast<uint32_t*>(s_key + B);  // [sorted] first piece
    uint32_t* s_pos = s_pe + B;                              // [column] end of the column's sorted run
    uint32_t* s_jofs = s_pos + p.n_columns;                  // [column] index entry - sorted position
    uint32_t* s_bofs = s_jofs + p.n_columns;                 // [column] CSS offset - block-local one
    uint16_t* s_wrun = reinterpret_cast<uint16_t*>(s_bofs + p.n_columns);  // [wave][column] count, then base
    __shared__ uint32_t s_wave[NW];

    const uint32_t tid = threadIdx.x, lane = (uint32_t)lane_id(), w = tid / kWave;
    const uint32_t C = p.n_columns;
    const uint32_t b = xcd_block(blockIdx.x, (uint32_t)p.blocks);
    const uint64_t f0 = (uint64_t)b * B;
    const uint32_t nb = (uint32_t)std::min<uint64_t>(B, p.nf - f0);
    const uint32_t fpt = B / NT;              // fields per thread: 1 to 16
    const uint32_t per = (C + NT - 1) / NT;   // columns per thread (thread t: t * per ...), at most 16

    // (1) keys and lengths of the block's fields into LDS (thread t: fields t,
    // t + NT, ...), and the block's entry and byte bases of each column (s_jofs
    // and s_bofs, made relative in (3) and (4)); all loads are issued first
    {
        uint32_t cv[kColPer], lv[kColPer];
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t i = k * NT + tid;
            cv[k] = k < fpt && i < nb ? p.col[f0 + i] : kNoKey;
            lv[k] = k < fpt && i < nb ? p.len[f0 + i] : 0u;
        }
        for (uint32_t c = tid; c < C; c += NT) {
            const uint32_t gj = p.cnt_excl[(uint64_t)c * p.blocks + b], gb = p.bytes_excl[(uint64_t)c * p.blocks + b];
#pragma unroll
            for (int v = 0; v < NW; ++v) s_wrun[v * C + c] = 0;
            s_jofs[c] = gj;
            s_bofs[c] = gb;
        }
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t i = k * NT + tid;
            if (k >= fpt) continue;
            s_key[i] = cv[k] < C ? (uint16_t)cv[k] : (uint16_t)kNoKey;
            s_len[i] = lv[k];
        }
    }
    __syncthreads();
    // (2) stable ranks. Wave w takes the block's w-th NW-th in rounds of 64
    // fields in input order: the lanes with the same key come from ballots over
    // the key bits, the wave's earlier fields of that key from its running count
    // in LDS (read and written by this wave alone, in program order).
    const uint32_t seg = B / NW;  // (rounds: seg / 64 = fpt)
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t rk[kColPer];
    uint16_t* wrun = s_wrun + w * C;
#pragma unroll
    for (uint32_t r = 0; r < (uint32_t)kColPer; ++r) {
        rk[r] = 0;
        if (r >= fpt) continue;
        const uint32_t i = w * seg + r * kWave + lane;
        const uint32_t key = i < nb ? s_key[i] : kNoKey;
        const bool valid = key != kNoKey;
        uint64_t peers = __ballot(valid);
        for (uint32_t bit = 0; bit < p.key_bits; ++bit) {
            const uint64_t m = __ballot((key >> bit) & 1u);
            peers &= ((key >> bit) & 1u) ? m : ~m;
        }
        const uint32_t run = valid ? wrun[key] : 0u;
        rk[r] = run + (uint32_t)__popcll(peers & lt);
        if (valid && (peers >> lane) == 1ull) wrun[key] = (uint16_t)(run + __popcll(peers));
    }
    __syncthreads();
    // (3) each column's sorted run: its start (exclusive sum over the columns of
    // the counts) and, per wave, where that wave's fields of the column begin
    {
        uint32_t sum = 0;
        for (uint32_t k = 0; k < per; ++k) {
            const uint32_t c = tid * per + k;
            if (c < C) {
#pragma unroll
                for (int v = 0; v < NW; ++v) sum += s_wrun[v * C + c];
            }
        }
        uint32_t excl, tot;
        block_scan<NW>(sum, 0u, excl, tot, s_wave, AddU32{});
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t c = tid * per + k;
            if (k >= per || c >= C) continue;
            s_jofs[c] -= excl;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                const uint32_t n_vc = s_wrun[v * C + c];
                s_wrun[v * C + c] = (uint16_t)excl;
                excl += n_vc;
            }
            s_pos[c] = excl;
        }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t r = 0; r < (uint32_t)kColPer; ++r) {
        if (r >= fpt) continue;
        const uint32_t i = w * seg + r * kWave + lane;
        const uint32_t key = i < nb ? s_key[i] : kNoKey;
        if (key != kNoKey) s_perm[wrun[key] + rk[r]] = (uint16_t)i;
    }
    __syncthreads();
    // (4) block-local CSS offsets: exclusive sum of (length + slot) in sorted order
    const uint32_t nv = s_pos[C - 1];  // fields with a valid key
    {
        uint32_t wv[kColPer], sum = 0;
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t q = tid * fpt + k;
            wv[k] = k < fpt && q < nv ? s_len[s_perm[q]] + p.slot : 0u;
            sum += wv[k];
        }
        uint32_t excl, tot;
        block_scan<NW>(sum, 0u, excl, tot, s_wave, AddU32{});
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            if (k < fpt) s_css[tid * fpt + k] = excl;
            excl += wv[k];
        }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
        const uint32_t c = tid * per + k;
        if (k >= per || c >= C) continue;
        const uint32_t first = c ? s_pos[c - 1] : 0u;
        if (first < s_pos[c]) s_bofs[c] -= s_css[first];
    }
    __syncthreads();
    // (5) index entries in sorted order (thread t: sorted fields t, t + NT, ...;
    // each column's entries of the block are one run); the gathers of all of a
    // thread's entries are issued first. Length, source and CSS offset go to
    // LDS for (6).
    uint32_t qL[kColPer], qS[kColPer], qD[kColPer];
    {
        uint32_t qi[kColPer], qr[kColPer];
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t q = tid + k * NT;
            qi[k] = k < fpt && q < nv ? s_perm[q] : 0u;
            qr[k] = k < fpt && q < nv ? p.rec[f0 + qi[k]] : 0u;
            qS[k] = k < fpt && q < nv ? p.off[f0 + qi[k]] : 0u;
        }
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t q = tid + k * NT;
            qL[k] = 0;
            qD[k] = 0;
            if (k >= fpt || q >= nv) continue;
            const uint32_t c = s_key[qi[k]], L = s_len[qi[k]];
            const uint32_t j = q + s_jofs[c], o = s_css[q] + s_bofs[c];
            p.ent_rec[j] = qr[k];
            p.ent_len[j] = L;
            p.ent_off[j] = o;
            qL[k] = (uint64_t)qS[k] + L <= p.n ? L : 0u;  // (a span past the input: never for a parse's own fields)
            qD[k] = o;
        }
    }
    // (6) the CSS bytes. A field takes E = L + slot bytes: its data, then the
    // slot. E >= 16 is ceil(E / 16) pieces of 16 bytes (the last one ending at
    // E), a shorter E one piece. Length, source and CSS offset by sorted
    // position go to the LDS of the local-order arrays (which nothing reads any
    // more), the exclusive sum of the pieces to s_pe. The block's pieces are
    // dealt to the threads in turn (consecutive threads take consecutive
    // pieces, so they write consecutive bytes); a thread finds a piece's field
    // by a binary search over s_pe and keeps 8 pieces in flight.
    uint32_t* s_sl = s_len;                                 // [sorted] length
    uint32_t* s_ss = reinterpret_cast<uint32_t*>(s_perm);  // [sorted] source offset (s_perm and s_key)
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
        const uint32_t q = tid + k * NT;
        if (k >= fpt) continue;
        s_sl[q] = qL[k];
        s_ss[q] = qS[k];
        s_css[q] = qD[k];
    }
    __syncthreads();
    uint32_t n_pieces;
    {
        uint32_t np[kColPer], sum = 0;
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            const uint32_t q = tid * fpt + k;
            const uint32_t E = k < fpt && q < nv ? s_sl[q] + p.slot : 0u;
            np[k] = E >= 16u ? (E + 15u) >> 4 : (E ? 1u : 0u);
            sum += np[k];
        }
        uint32_t excl;
        block_scan<NW>(sum, 0u, excl, n_pieces, s_wave, AddU32{});
#pragma unroll
        for (uint32_t k = 0; k < (uint32_t)kColPer; ++k) {
            if (k < fpt) s_pe[tid * fpt + k] = excl;
            excl += np[k];
        }
    }
    __syncthreads();
    constexpr int kInFlight = 8;
    for (uint32_t k0 = 0; k0 < n_pieces; k0 += kInFlight * NT) {
        Piece pc[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const uint32_t k = k0 + u * NT + tid;
            pc[u].m = 0;
            if (k >= n_pieces) continue;
            uint32_t lo = 0;  // the last field whose first piece is at or before k
#pragma unroll
            for (uint32_t step = kColFields / 2; step >= 1; step >>= 1)
                if (lo + step < nv && s_pe[lo + step] <= k) lo += step;
            const uint32_t L = s_sl[lo], E = L + p.slot;
            const uint32_t o = E >= 16u ? min((k - s_pe[lo]) << 4, E - 16u) : 0u;
            pc[u] = load_piece(p, s_ss[lo], s_css[lo], L, o, min(E, 16u));
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) store_piece(p, pc[u]);
    }
}

}  // namespace
}  // namespace ppr

using namespace ppr;

extern "C" PPR_API size_t ppr_columns_workspace_bytes(uint64_t n_fields, uint32_t n_columns)
{
    if (n_columns > kColMaxColumns || n_fields >= 0xffffffffull) return 0;
    return (size_t)col_layout(n_fields, n_columns, 1024).total;  // (the most blocks)
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
    const uint32_t B = fields_per_block(n_columns);
    const ColLayout L = col_layout(n_fields, n_columns, B);
    if (ws_bytes < L.total) return PPR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    ColHeader* h = (ColHeader*)ws;
    uint32_t* cnt = (uint32_t*)(ws + L.cnt);
    uint32_t* bytes = (uint32_t*)(ws + L.bytes);
    uint64_t* stat = (uint64_t*)(ws + L.scan_stat);  // two arrays of L.tiles statuses, one per scan
    const uint32_t slot = mode == PPR_CSS_INDEXED ? 0u : 1u;
    uint32_t key_bits = 0;
    while ((1u << key_bits) < n_columns) ++key_bits;
    const uint64_t hist_n = L.blocks * n_columns;
    const uint32_t e1 = next_epoch(), e2 = next_epoch();

    stage_event(opts, 0, s);
    hipLaunchKernelGGL(cols_reset_kernel, dim3(clear_grid(2 * L.tiles * 8)), dim3(256), 0, s, h, (uint4*)stat, L.tiles);
    stage_event(opts, 1, s);
    if (n_fields) {
        hipLaunchKernelGGL(cols_hist_kernel, dim3((uint32_t)L.blocks), dim3(kColBlock), 0, s, d_col, d_len, n_fields,
                           B, n_columns, slot, L.blocks, cnt, bytes, h);
        stage_event(opts, 2, s);
        const dim3 sg((uint32_t)((hist_n + kColFields - 1) / kColFields));
        hipLaunchKernelGGL(cols_scan_kernel, sg, dim3(kColBlock), 0, s, cnt, cnt, hist_n, stat, e1, &h->ctr[0],
                           &h->total[0], &h->fault);
        stage_event(opts, 3, s);
        hipLaunchKernelGGL(cols_scan_kernel, sg, dim3(kColBlock), 0, s, bytes, bytes, hist_n, stat + L.tiles, e2,
                           &h->ctr[1], &h->total[1], &h->fault);
        stage_event(opts, 4, s);
        PartParams pp;
        pp.in = d_bytes;
        pp.n = n;
        pp.rec = d_rec;
        pp.col = d_col;
        pp.off = d_off;
        pp.len = d_len;
        pp.nf = n_fields;
        pp.blocks = L.blocks;
        pp.B = B;
        pp.n_columns = n_columns;
        pp.key_bits = key_bits;
        pp.slot = slot;
        pp.term = mode == PPR_CSS_VECTOR ? 0u : terminator;
        pp.cnt_excl = cnt;
        pp.bytes_excl = bytes;
        pp.ent_rec = out->rec;
        pp.ent_off = out->css_off;
        pp.ent_len = out->length;
        pp.css = out->css;
        pp.aux = mode == PPR_CSS_VECTOR ? out->aux : nullptr;
        pp.cap = out->css_cap;
        // blocks of 4096 fields run 1024 threads where their LDS allows (four
        // fields per thread), others 256
        if (B == kColFields && part_lds_bytes(B, n_columns, 16) <= kLdsBudget)
            hipLaunchKernelGGL(cols_part_kernel<1024>, dim3((uint32_t)L.blocks), dim3(1024),
                               part_lds_bytes(B, n_columns, 16), s, pp);
        else
            hipLaunchKernelGGL(cols_part_kernel<kColBlock>, dim3((uint32_t)L.blocks), dim3(kColBlock),
                               part_lds_bytes(B, n_columns, kColWaves), s, pp);
        stage_event(opts, 5, s);
    } else {
        for (uint32_t i = 2; i <= 5; ++i) stage_event(opts, i, s);
    }
    hipLaunchKernelGGL(cols_bounds_kernel, dim3((n_columns + 256) / 256), dim3(256), 0, s, cnt, bytes, L.blocks,
                       n_columns, n_fields, &h->total[1], out->col_first_field, out->col_first_byte);
    stage_event(opts, 6, s);
    if (hipGetLastError() != hipSuccess) return PPR_EHIP;
    ColHeader hh;
    if (hipMemcpyAsync(&hh, h, sizeof hh, hipMemcpyDeviceToHost, s) != hipSuccess) return PPR_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PPR_EHIP;
    out->css_bytes = n_fields ? hh.total[1] : 0u;
    if (hh.bad_column) return PPR_EINVAL;
    if (hh.fault) return PPR_EHIP;
    return out->css_bytes > out->css_cap ? PPR_ECAPACITY : PPR_OK;
}
