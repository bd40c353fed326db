// Wave/workgroup scans and the device-wide decoupled look-back, generic over the
// carried value (state-transition vectors, count carries, lexer identifiers).
//
// ParPaRaw (Sec. 3) computes the chunks' start states and offsets with
// exclusive scans over associative operators; here every such scan is a
// single-pass scan: each workgroup scans its own threads, publishes its tile
// aggregate, then finds its tile's exclusive prefix by looking back over its
// predecessors' published statuses (aggregate or inclusive prefix).
//
// gfx950 specifics:
//   * wave scans use DPP lane moves (row_shr within rows of 16 lanes, then
//     row_bcast:15 and row_bcast:31 across rows) fused into the VALU, not LDS
//     shuffles; the exclusive shift is wave_shr:1;
//   * every wave of the workgroup takes part in a look-back round, so one round
//     (one trip to memory and back, about a microsecond across XCDs) covers
//     64 x waves predecessors, and a wave only waits for the statuses it needs
//     (those between the nearest inclusive prefix and the tile);
//   * statuses are relaxed agent-scope atomics (coherent across XCDs) whose
//     words carry the call epoch, so no release/acquire fences (L2 writeback and
//     invalidate on this target) are needed.
#pragma once

#include "ppr_device.h"
#include "ppr_host.h"
#include "ppr_walk.h"

namespace ppr {

template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_t(const T& old, const T& src)
{
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    constexpr int N = sizeof(T) / 4;
    uint32_t o[N], s[N], r[N];
    __builtin_memcpy(o, &old, sizeof(T));
    __builtin_memcpy(s, &src, sizeof(T));
#pragma unroll
    for (int i = 0; i < N; ++i)
        r[i] = (uint32_t)__builtin_amdgcn_update_dpp((int)o[i], (int)s[i], CTRL, ROW_MASK, 0xf, false);
    T out;
    __builtin_memcpy(&out, r, sizeof(T));
    return out;
}

template <typename T>
__device__ __forceinline__ T readlane_t(const T& v, int lane)
{
    constexpr int N = sizeof(T) / 4;
    uint32_t s[N], r[N];
    __builtin_memcpy(s, &v, sizeof(T));
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = (uint32_t)__builtin_amdgcn_readlane((int)s[i], lane);
    T out;
    __builtin_memcpy(&out, r, sizeof(T));
    return out;
}

// inclusive scan over the 64 lanes of a wave in lane order (comb(a, b): a earlier)
template <typename T, typename Comb>
__device__ __forceinline__ T wave_scan(T x, const T& id, const Comb& comb)
{
    x = comb(dpp_t<0x111, 0xf>(id, x), x);  // row_shr:1
    x = comb(dpp_t<0x112, 0xf>(id, x), x);  // row_shr:2
    x = comb(dpp_t<0x114, 0xf>(id, x), x);  // row_shr:4
    x = comb(dpp_t<0x118, 0xf>(id, x), x);  // row_shr:8
    x = comb(dpp_t<0x142, 0xa>(id, x), x);  // row_bcast:15 into rows 1 and 3
    x = comb(dpp_t<0x143, 0xc>(id, x), x);  // row_bcast:31 into rows 2 and 3
    return x;
}

struct MinU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct MaxU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};

// the wave's minimum of mn and maximum of mx, in every lane
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx)
{
    mn = readlane_t(wave_scan(mn, 0xffffffffu, MinU32{}), kWave - 1);
    mx = readlane_t(wave_scan(mx, 0u, MaxU32{}), kWave - 1);
}

// Widens the stored range [*dmin, *dmax] (it only ever widens) to hold [mn, mx]
// (mn = 0xffffffff, mx = 0: nothing to add). One thread calls it; it makes an
// atomic only where the stored bound would change (a stale read understates the
// range, so at worst an atomic is made that was not needed).
__device__ __forceinline__ void widen_range(uint32_t* dmin, uint32_t* dmax, uint32_t mn, uint32_t mx)
{
    if (mn < __hip_atomic_load(dmin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMin(dmin, mn);
    if (mx > __hip_atomic_load(dmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(dmax, mx);
}

struct AddU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};

// The workgroup's per-record counts (fewest / most fields, records not of the
// expected number, the first of them) into the call's, held at dmin, dmax, dbad
// and dfirst. Every thread calls it; s_stats holds 4 x NW words.
template <int NW>
__device__ __forceinline__ void publish_rec_stats(uint32_t cmin, uint32_t cmax, uint32_t bad, uint32_t fbad,
                                                  uint32_t* s_stats, uint32_t* dmin, uint32_t* dmax, uint32_t* dbad,
                                                  uint32_t* dfirst)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    cmin = readlane_t(wave_scan(cmin, 0xffffffffu, MinU32{}), kWave - 1);
    cmax = readlane_t(wave_scan(cmax, 0u, MaxU32{}), kWave - 1);
    bad = readlane_t(wave_scan(bad, 0u, AddU32{}), kWave - 1);
    fbad = readlane_t(wave_scan(fbad, 0xffffffffu, MinU32{}), kWave - 1);
    if (lane == 0) {
        s_stats[w] = cmin;
        s_stats[NW + w] = cmax;
        s_stats[2 * NW + w] = bad;
        s_stats[3 * NW + w] = fbad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < NW; ++i) {
            cmin = min(cmin, s_stats[i]);
            cmax = max(cmax, s_stats[NW + i]);
            bad += s_stats[2 * NW + i];
            fbad = min(fbad, s_stats[3 * NW + i]);
        }
        widen_range(dmin, dmax, cmin, cmax);
        if (bad) atomicAdd(dbad, bad);
        if (fbad < __hip_atomic_load(dfirst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMin(dfirst, fbad);
    }
}

// value of the previous lane (lane 0: id)
template <typename T>
__device__ __forceinline__ T wave_shr1(const T& id, const T& x)
{
    return dpp_t<0x138, 0xf>(id, x);
}

// inclusive scan over lanes 0..N-1 of each row of 16 (N <= 16)
template <int N, typename T, typename Comb>
__device__ __forceinline__ T row_scan(T x, const T& id, const Comb& comb)
{
    static_assert(N <= 16, "one row");
    if constexpr (N > 1) x = comb(dpp_t<0x111, 0xf>(id, x), x);
    if constexpr (N > 2) x = comb(dpp_t<0x112, 0xf>(id, x), x);
    if constexpr (N > 4) x = comb(dpp_t<0x114, 0xf>(id, x), x);
    if constexpr (N > 8) x = comb(dpp_t<0x118, 0xf>(id, x), x);
    return x;
}

// cond ? a : b, word by word (a conditional between two objects can otherwise
// become a select between their addresses, in different address spaces)
template <typename T>
__device__ __forceinline__ T select_t(bool cond, const T& a, const T& b)
{
    constexpr int N = sizeof(T) / 4;
    uint32_t x[N], y[N];
    __builtin_memcpy(x, &a, sizeof(T));
    __builtin_memcpy(y, &b, sizeof(T));
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = cond ? x[i] : y[i];
    T out;
    __builtin_memcpy(&out, x, sizeof(T));
    return out;
}

// s_wave[lane] in lanes 0..NW-1, id elsewhere. The load is unconditional (a
// clamped index) and the choice is made per word, so that no pointer select
// between LDS and a private copy of id appears.
template <int NW, typename T>
__device__ __forceinline__ T lane_value(const T* s_wave, const T& id)
{
    const int lane = lane_id();
    const T v = s_wave[lane < NW ? lane : NW - 1];
    return select_t(lane < NW, v, id);
}

// Exclusive scan over the workgroup in thread order (comb(a, b): a earlier).
// `total` is the combination of all threads. The wave totals go through LDS and
// are scanned by the first NW lanes of every wave. Uses s_wave[NW]; the caller
// synchronises before reusing it.
template <int NW, typename T, typename Comb>
__device__ void block_scan(const T& v, const T& ident, T& excl, T& total, T* s_wave, const Comb& comb)
{
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const T inc = wave_scan(v, ident, comb);
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    const T ws = row_scan<NW>(lane_value<NW>(s_wave, ident), ident, comb);
    T pre = ident;
    if (w) pre = readlane_t(ws, w - 1);
    total = readlane_t(ws, NW - 1);
    excl = comb(pre, wave_shr1(ident, inc));
}

// Combination of the values of all threads of the workgroup in thread order,
// returned to every thread. Uses s_wave[NW]; the caller synchronises before
// reusing it.
template <int NW, typename T, typename Comb>
__device__ T block_reduce(const T& v, const T& ident, T* s_wave, const Comb& comb)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const T inc = wave_scan(v, ident, comb);
    if (lane == kWave - 1) s_wave[w] = inc;
    __syncthreads();
    return readlane_t(row_scan<NW>(lane_value<NW>(s_wave, ident), ident, comb), NW - 1);
}

// One round of a look-back at `base` (see walk_predecessors): lane l of wave w
// looks at tile base - 64 w - (63 - l). first_raw(u, v) / repoll(u, v) give the
// status of tile u (kFlagIncl: v = inclusive prefix through u, kFlagAgg: v = u's
// aggregate, 0: not yet published). A wave only waits for the statuses it needs
// (those between the nearest inclusive prefix and the tile); after kSpinLimit
// polls (counted in `spins` over the whole walk) the missing ones count as empty
// aggregates and a fault is recorded, so the kernel always finishes. Returns the
// combination of the statuses used; found: one of them was an inclusive prefix.
template <int NW, typename T, typename First, typename Repoll, typename Comb>
__device__ __forceinline__ T lookback_round(int64_t base, const T& ident, const First& first_raw,
                                            const Repoll& repoll, const Comb& comb, T* s_part, int* s_found,
                                            uint32_t* fault, uint32_t& spins, bool& found)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int64_t u = base - (int64_t)(w * kWave + (kWave - 1 - lane));
    const bool valid = u >= 0;
    T v = ident;
    uint32_t f = 0;
    if (valid) f = first_raw(u, v);
    const uint64_t vmask = __ballot(valid);
    for (;;) {
        const uint64_t ready = __ballot(f != 0);
        const uint64_t inclm = __ballot(f == kFlagIncl);
        // statuses needed: from the nearest inclusive prefix up to the tile
        const uint64_t need = inclm ? vmask & (~0ull << (63 - __clzll((long long)inclm))) : vmask;
        if ((ready & need) == need) break;
        if (++spins > kSpinLimit) {
            if (lane == 0) atomicOr(fault, 1u);
            if (valid && f == 0) {
                f = kFlagAgg;
                v = ident;
            }
            break;
        }
        __builtin_amdgcn_s_sleep(1);
        if (valid && f == 0) f = repoll(u, v);
    }
    const uint64_t inclm = __ballot(f == kFlagIncl);
    const int j = inclm ? 63 - __clzll((long long)inclm) : -1;
    if (!(valid && lane >= j)) v = ident;
    const T part = readlane_t(wave_scan(v, ident, comb), kWave - 1);
    if (lane == 0) {
        s_part[w] = part;
        s_found[w] = j >= 0;
    }
    __syncthreads();
    // wave i covers tiles base-64i-63 .. base-64i; the nearest wave holding an
    // inclusive prefix ends the walk, and farther waves are not needed
    int wi = NW;
#pragma unroll
    for (int i = NW - 1; i >= 0; --i)
        if (s_found[i]) wi = i;
    const int last = wi < NW ? wi : NW - 1;
    T r = s_part[last];
    for (int i = last - 1; i >= 0; --i) r = comb(r, s_part[i]);
    __syncthreads();
    found = wi < NW;
    return r;
}

// Decoupled look-back; every thread of the workgroup calls it, tile > 0.
// poll(u, out) returns kFlagIncl (out = inclusive prefix through tile u),
// kFlagAgg (out = tile u's aggregate) or 0 (not yet published). Returns the
// combination of all tiles before `tile`. Bounded: see lookback_round and
// walk_predecessors.
template <int NW, typename T, typename Poll, typename Comb>
__device__ T lookback(uint32_t tile, const T& ident, const Poll& poll, const Comb& comb, T* s_part, int* s_found,
                      uint32_t* fault)
{
    uint32_t spins = 0;
    return walk_predecessors(
        tile, ident, (int64_t)NW * kWave,
        [&](int64_t base, bool& found) {
            return lookback_round<NW>(base, ident, poll, poll, comb, s_part, s_found, fault, spins, found);
        },
        comb);
}

// Look-back whose first round of polls the caller issued earlier (look_first),
// so that those loads travel while the caller does other work. A poller has
// load(u) -> Raw (the status words of tile u, all loads issued at once) and
// decode(raw, out) -> kFlagIncl / kFlagAgg / 0, as poll() above. Otherwise as
// lookback(): every thread calls it, tile > 0, bounded.
template <int NW, typename P>
__device__ __forceinline__ typename P::Raw look_first(uint32_t tile, const P& poller)
{
    const int lane = lane_id(), w = threadIdx.x / kWave;
    const int64_t u = (int64_t)tile - 1 - (int64_t)(w * kWave + (kWave - 1 - lane));
    return poller.load(u >= 0 ? u : 0);  // (a tile before the first is never decoded)
}

template <int NW, typename T, typename P, typename Comb>
__device__ T lookback_pre(uint32_t tile, const T& ident, const P& poller, const Comb& comb, T* s_part, int* s_found,
                          uint32_t* fault, const typename P::Raw& raw0)
{
    uint32_t spins = 0;
    bool first_round = true;
    auto repoll = [&](int64_t u, T& v) { return poller.decode(poller.load(u), v); };
    return walk_predecessors(
        tile, ident, (int64_t)NW * kWave,
        [&](int64_t base, bool& found) {
            const bool fr = first_round;
            first_round = false;
            auto first_raw = [&](int64_t u, T& v) { return fr ? poller.decode(raw0, v) : repoll(u, v); };
            return lookback_round<NW>(base, ident, first_raw, repoll, comb, s_part, s_found, fault, spins, found);
        },
        comb);
}

}  // namespace ppr
