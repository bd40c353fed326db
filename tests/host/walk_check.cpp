// Host check of the look-back walk's termination (ppr_walk.h): a stub round
// that never meets an inclusive prefix (as after the spin limit, when every
// missing status counts as an empty aggregate) must still end the walk once
// tile 0 has been covered, having covered every predecessor exactly once.
#include <cstdio>
#include <cstdlib>

#include "ppr_walk.h"

struct Span {
    long long lo, hi, rounds;  // tiles covered [lo, hi], rounds taken
};

static int check(unsigned tile, long long span, long long found_at)
{
    long long rounds = 0;
    auto round = [&](long long base, bool& found) {
        ++rounds;
        if (rounds > 1000000) {
            std::printf("tile %u span %lld: walk does not end\n", tile, span);
            std::exit(1);
        }
        const long long lo = base - span + 1 < 0 ? 0 : base - span + 1;
        found = found_at >= lo && found_at <= base;
        // a round's combination: the tiles it covers (from the inclusive prefix on, if any)
        return Span{found ? found_at : lo, base, 1};
    };
    auto comb = [](const Span& a, const Span& b) {
        if (a.hi < 0) return b;
        if (b.hi < 0) return a;
        if (a.hi + 1 != b.lo) {
            std::printf("gap between %lld and %lld\n", a.hi, b.lo);
            std::exit(1);
        }
        return Span{a.lo, b.hi, a.rounds + b.rounds};
    };
    const Span r = ppr::walk_predecessors(tile, Span{0, -1, 0}, span, round, comb);
    const long long want_lo = found_at >= 0 && found_at < (long long)tile ? found_at : 0;
    if (r.lo != want_lo || r.hi != (long long)tile - 1) {
        std::printf("tile %u span %lld found_at %lld: covered [%lld, %lld]\n", tile, span, found_at, r.lo, r.hi);
        return 1;
    }
    const long long max_rounds = ((long long)tile - 1 - want_lo) / span + 1;
    if (rounds > max_rounds) {
        std::printf("tile %u: %lld rounds, expected at most %lld\n", tile, rounds, max_rounds);
        return 1;
    }
    return 0;
}

int main()
{
    int bad = 0;
    const long long spans[] = {64, 512, 1024};
    const unsigned tiles[] = {1, 2, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 4096, 100000};
    for (long long span : spans)
        for (unsigned tile : tiles) {
            bad += check(tile, span, -1);  // never an inclusive prefix
            bad += check(tile, span, 0);   // only tile 0's
            bad += check(tile, span, (long long)tile / 2);
            bad += check(tile, span, (long long)tile - 1);
        }
    std::printf(bad ? "FAIL\n" : "walk ok\n");
    return bad ? 1 : 0;
}
