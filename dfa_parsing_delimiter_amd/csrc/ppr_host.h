// Host/device structures shared by the library's entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "ppr.h"

namespace ppr {

// Start of every workspace (256 bytes reserved): the scalar results the last
// tile writes and the running call's tile counter. The counter, which every
// workgroup increments once, sits on a 128-byte line of its own: on the line of
// the scalars that every tile also reads (the record counts), the two streams of
// requests to one address queue behind each other (measured: 5% of the
// single-pass parse at 31-byte chunks).
struct WsHeader {
    uint32_t end_state;
    uint32_t fault;     // set when a look-back wait gave up (never expected)
    uint64_t n_fields;  // n_tokens for the lexer
    uint64_t n_records;
    int64_t error_pos;  // written by the host from err_min and the end state
    uint32_t err_min;   // first INVALID byte (atomic minimum over tiles), 0xffffffff: none
    uint32_t last_rec;  // the input's last byte is a record delimiter (multi-kernel parse)
    uint32_t path;      // which kernels ran (PPR_PATH_*)
    uint32_t cols_min;  // fewest fields of a record (atomic minimum), 0xffffffff: no record yet
    uint32_t cols_max;  // most fields of a record (atomic maximum)
    uint32_t bad_records;  // records whose number of fields is not the expected one (atomic sum)
    uint32_t first_bad;    // the first of them (atomic minimum), 0xffffffff: none
    uint32_t tail_start;   // the unterminated tail: start of its field (1 + last terminator, 0: none)
    uint32_t tail_col;     // and that field's column
    alignas(128) uint32_t tile_counter;
};
static_assert(offsetof(WsHeader, tile_counter) == 128 && sizeof(WsHeader) <= 256, "WsHeader layout");

// Records stage event i of the call on the stream, if the caller asked for it.
inline void stage_event(const ppr_parse_opts_t* o, uint32_t i, hipStream_t s)
{
    if (o && o->stage_events && i < o->n_stage_events && o->stage_events[i])
        (void)hipEventRecord((hipEvent_t)o->stage_events[i], s);
}

// Upper bound on look-back polls per tile; beyond it the kernel records a fault
// and finishes instead of waiting forever.
constexpr uint32_t kSpinLimit = 1u << 22;
// Largest input of one call: every byte position a kernel forms, up to the end
// of the last (padded) tile, then fits 32 bits.
constexpr uint64_t kMaxInput = 0xffff0000ull;

// Count-carry status of one tile (second look-back). Every word is a relaxed
// 64-bit atomic holding the call epoch (high half) and one 32-bit value, so a
// word is valid on its own and no release/acquire ordering between words is
// needed (on gfx950 an agent-scope release writes back the L2 and an acquire
// invalidates it). agg: the tile's own carry, incl: its inclusive prefix.
struct StatB {
    uint64_t agg[3];
    uint64_t incl[4];
    uint64_t pad;
};
static_assert(sizeof(StatB) == 64, "StatB layout");

struct WsLayout {
    uint64_t tiles, off_a, off_b, total;
};

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Workgroups of 256 threads for a kernel that clears `bytes` of look-back
// statuses (clear_status): about one 16-byte word per thread, at most 1024.
inline uint32_t clear_grid(uint64_t bytes)
{
    const uint64_t g = (bytes + 16 * 256 - 1) / (16 * 256);
    return (uint32_t)(g < 1 ? 1 : g > 1024 ? 1024 : g);
}

// Call epochs tag look-back statuses so stale ones from earlier calls read as
// unpublished. 0 never occurs (a zero-filled workspace holds no valid status).
inline uint32_t next_epoch()
{
    static std::atomic<uint32_t> ctr{0};
    for (;;) {
        uint32_t e = (ctr.fetch_add(1, std::memory_order_relaxed) + 1u) & 0x3fffffffu;
        if (e) return e;
    }
}

}  // namespace ppr
