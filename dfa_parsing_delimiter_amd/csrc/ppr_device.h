// Device-side building blocks shared by the CSV and lexer kernels (gfx950).
//
// State-transition vectors [ParPaRaw, Sec. 3, Fig. 2]: entry i is the state a
// chunk ends in when it starts in state i. With at most 8 states, a vector is
// 8 bytes in two VGPRs (entries 0-3 in `lo`, 4-7 in `hi`), so the composite of
// two vectors is two v_perm_b32 byte selects — the register-resident array that
// ParPaRaw builds with bit-field insert/extract (multi-fragment in-register
// array, Fig. 8) becomes one byte permute per four entries on CDNA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ppr {

constexpr int kWave = 64;

struct Vec {
    uint32_t lo, hi;
};

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    // v_perm_b32: byte k of the result is byte sel.k of the 64-bit value {hi, lo} (0-3: lo, 4-7: hi)
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// LDS word at a byte address
__device__ __forceinline__ uint32_t lds_at(const uint32_t* base, uint32_t byte_addr)
{
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(base) + byte_addr);
}

__device__ __forceinline__ Vec vec_identity() { return {0x03020100u, 0x07060504u}; }

// composite: a earlier, b later; result[i] = b[a[i]]
__device__ __forceinline__ Vec compose(Vec a, Vec b) { return {perm(b.hi, b.lo, a.lo), perm(b.hi, b.lo, a.hi)}; }

__device__ __forceinline__ uint32_t vec_at(Vec v, uint32_t s)
{
    uint32_t w = s < 4 ? v.lo : v.hi;
    return (w >> ((s & 3u) * 8u)) & 0xffu;
}

// 8 entries of 3 bits (values < 8) <-> nibble-packed 32-bit word
__device__ __forceinline__ uint32_t vec_pack(Vec v)
{
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r |= ((v.lo >> (8 * i)) & 0xfu) << (4 * i);
        r |= ((v.hi >> (8 * i)) & 0xfu) << (4 * (i + 4));
    }
    return r;
}

__device__ __forceinline__ Vec vec_unpack(uint32_t p)
{
    Vec v{0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v.lo |= ((p >> (4 * i)) & 0xfu) << (8 * i);
        v.hi |= ((p >> (4 * (i + 4))) & 0xfu) << (8 * i);
    }
    return v;
}

// ---------------------------------------------------------------- atomics (agent scope)

__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_acquire(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- look-back status words
//
// Decoupled look-back (single-pass prefix scan with a per-tile status that is
// either the tile's own aggregate or its inclusive prefix). A status word is
// [63:34] call epoch, [33:32] flag, [31:0] payload. Every call clears its
// status arrays (clear_status) before its first tile starts: a workspace that
// served another call, another entry point or another input size can hold any
// bit pattern where the statuses now lie, small integers that happen to match
// the epoch field included. The epoch is a second guard.

constexpr uint32_t kFlagAgg = 1;
constexpr uint32_t kFlagIncl = 2;
constexpr uint32_t kEpochMask = 0x3fffffffu;

__device__ __forceinline__ uint64_t status_word(uint32_t epoch, uint32_t flag, uint32_t payload)
{
    return ((uint64_t)(epoch & kEpochMask) << 34) | ((uint64_t)flag << 32) | payload;
}
__device__ __forceinline__ uint32_t status_flag(uint64_t w, uint32_t epoch)
{
    return (uint32_t)(w >> 34) == (epoch & kEpochMask) ? (uint32_t)(w >> 32) & 3u : 0u;
}
__device__ __forceinline__ uint32_t status_payload(uint64_t w) { return (uint32_t)w; }

// Zero n 16-byte words, spread over the launch's grid (each workgroup a
// stride of the array).
__device__ __forceinline__ void clear_status(uint4* p, uint64_t n)
{
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) p[i] = make_uint4(0, 0, 0, 0);
}

// self-validating status word: call epoch in the high half, value in the low half
__device__ __forceinline__ uint64_t ew(uint32_t epoch, uint32_t v) { return ((uint64_t)epoch << 32) | v; }
__device__ __forceinline__ bool ew_ok(uint64_t w, uint32_t epoch) { return (uint32_t)(w >> 32) == epoch; }

// ---------------------------------------------------------------- wave shuffles

__device__ __forceinline__ uint32_t shfl_up(uint32_t v, int d) { return (uint32_t)__shfl_up((int)v, d, kWave); }
__device__ __forceinline__ uint32_t shfl_down(uint32_t v, int d) { return (uint32_t)__shfl_down((int)v, d, kWave); }
__device__ __forceinline__ uint32_t shfl(uint32_t v, int src) { return (uint32_t)__shfl((int)v, src, kWave); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Smallest of the active lanes' values v (0xffffffff: the lane has none), in
// every lane.
__device__ __forceinline__ uint32_t wave_min_defined(uint32_t v)
{
    uint64_t m = __ballot(v != 0xffffffffu);
    uint32_t best = 0xffffffffu;
    while (m) {
        best = min(best, (uint32_t)__builtin_amdgcn_readlane((int)v, __builtin_ctzll(m)));
        m &= m - 1;
    }
    return best;
}

// Lowers *dst, a position that only ever decreases, to the smallest of the
// wave's values v (0xffffffff: none): at most one atomic per wave, and none when
// *dst already holds a smaller position (a stale read is only ever larger).
__device__ __forceinline__ void wave_lower_min(uint32_t* dst, uint32_t v)
{
    const uint32_t best = wave_min_defined(v);
    if (best == 0xffffffffu) return;
    if (lane_id() == __builtin_ctzll(__ballot(1)) &&
        __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > best)
        atomicMin(dst, best);
}

// ---------------------------------------------------------------- wave-level output staging


// a 64-bit value the whole wave holds, in scalar registers (a store to
// base + uniform + lane then takes a scalar base and a 32-bit lane offset)
__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// One store of v to base[lane] with base wave-uniform: the base goes through
// readfirstlane into scalar registers and stays a global-address-space pointer,
// so the compiler emits global_store_dword with a scalar base and the lane's
// 32-bit offset (and handles the VALU-to-SGPR hazard itself). Indexing the
// kernel-argument pointer directly instead lets the compiler hoist base + lane
// into per-lane 64-bit addresses and add the uniform part before every store.
typedef __attribute__((address_space(1))) uint32_t global_u32;

__device__ __forceinline__ void store_u32(uint32_t* base, uint32_t lane, uint32_t v)
{
    global_u32* const g = (global_u32*)uniform64((uint64_t)(uintptr_t)base);
    g[lane] = v;
}

// Output slots for `count` items written from global index `first` on: those
// below the capacity. Computed in 64 bits once per window of items, so that the
// per-round test (item offset in the window < slots) involves no wrap-around.
__device__ __forceinline__ uint32_t slots_from(uint64_t cap, uint64_t first, uint32_t count)
{
    if (first >= cap) return 0u;
    const uint64_t left = cap - first;
    return left < (uint64_t)count ? (uint32_t)left : count;
}

// Lists a lane's terminators that fall in the window [w0, w1) of wave-local
// field indices into the wave's LDS list (entry = position << 1 | record bit,
// positions from rel0 on). The lane's fields are [first, first + mine); tw / rw:
// its terminator / record bitmaps as 32-bit words (bit j of word q = byte
// 32 q + j). When all of them fall in the window (the usual case) the loop
// runs without index checks.
template <int NWORDS, typename Entry>
__device__ __forceinline__ void list_terminators(Entry* list, const uint32_t (&tw)[NWORDS],
                                                 const uint32_t (&rw)[NWORDS], uint32_t rel0, uint32_t first,
                                                 uint32_t mine, uint32_t w0, uint32_t w1)
{
    if (!(mine && first < w1 && first + mine > w0)) return;
    if (first >= w0 && first + mine <= w1) {
        Entry* dst = list + (first - w0);
#pragma unroll
        for (int q = 0; q < NWORDS; ++q) {
            uint32_t bits = tw[q];
            const uint32_t base2 = (rel0 + 32u * q) << 1;
            while (bits) {
                const uint32_t j = (uint32_t)__builtin_ctz(bits);
                *dst++ = (Entry)(base2 + (j << 1) + ((rw[q] >> j) & 1u));
                bits &= bits - 1u;
            }
        }
        return;
    }
    uint32_t li = first;
#pragma unroll
    for (int q = 0; q < NWORDS; ++q) {
        uint32_t bits = tw[q];
        while (bits && li < w1) {
            const uint32_t j = (uint32_t)__builtin_ctz(bits);
            if (li >= w0) list[li - w0] = (Entry)(((rel0 + 32u * q + j) << 1) | ((rw[q] >> j) & 1u));
            ++li;
            bits &= bits - 1u;
        }
    }
}

}  // namespace ppr
