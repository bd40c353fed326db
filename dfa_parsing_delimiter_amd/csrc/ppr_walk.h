// The walk of a decoupled look-back over a tile's predecessors, with no device
// code of its own, so that its termination can be checked on the host.
//
// ParPaRaw (Sec. 3) takes every chunk's start state and offsets from exclusive
// scans; the single-pass kernels here find a tile's exclusive prefix by
// combining the published statuses of its predecessors, nearest first, until
// one of them is an inclusive prefix. A round looks at `span` predecessors at
// once (tiles base - span + 1 .. base; those below tile 0 do not exist).
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define PPR_HD __host__ __device__
#else
#define PPR_HD
#endif

namespace ppr {

// The walk is over after a round that found an inclusive prefix, or after the
// round that reached tile 0: then nothing before the tile is left to combine,
// whatever the statuses said (a status given up on after the spin limit counts
// as an empty aggregate, so without this rule a walk that never meets an
// inclusive prefix would step below tile 0 for ever).
PPR_HD inline bool walk_done(bool found_inclusive, int64_t base, int64_t span)
{
    return found_inclusive || base < span;
}

// Combination of all tiles before `tile` (tile > 0). round(base, found) returns
// the combination of the statuses it used from the round at `base` (earlier
// tiles first) and sets found if one of them was an inclusive prefix; comb(a, b)
// combines a earlier with b later.
template <typename T, typename Round, typename Comb>
PPR_HD T walk_predecessors(uint32_t tile, const T& ident, int64_t span, Round&& round, const Comb& comb)
{
    T acc = ident;
    for (int64_t base = (int64_t)tile - 1;; base -= span) {
        bool found = false;
        const T part = round(base, found);
        acc = comb(part, acc);
        if (walk_done(found, base, span)) return acc;
    }
}

}  // namespace ppr
