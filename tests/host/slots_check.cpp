// Host check of the table-driven kernels' symbol classification
// (ppr_slots.h): for class maps with up to 8 special bytes anywhere in 0..255,
// every byte value at every position of a 4-byte word must get its own class
// code (its special's code, or the catch-all code). v_perm_b32 is emulated from
// its instruction-set definition: selectors 0-7 pick a byte of {hi, lo}, 8-11
// the sign of byte 1, 3, 5 or 7 spread over the byte, 12 gives 0x00 and 13-255
// give 0xff. A deliberately bad table (a slot function blind to the difference
// 12 ^ key) must fail, so the check can see the case the slot choice rules out.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "ppr_slots.h"

static uint32_t vperm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    const uint64_t v = ((uint64_t)hi << 32) | lo;
    uint32_t r = 0;
    for (int k = 0; k < 4; ++k) {
        const uint32_t s = (sel >> (8 * k)) & 0xffu;
        uint32_t b;
        if (s < 8) b = (uint32_t)(v >> (8 * s)) & 0xffu;
        else if (s < 12) b = ((v >> (16 * (s - 8) + 15)) & 1u) ? 0xffu : 0x00u;  // bits 15, 31, 47, 63
        else if (s == 12) b = 0x00u;
        else b = 0xffu;
        r |= b << (8 * k);
    }
    return r;
}

struct Perm {
    uint32_t operator()(uint32_t hi, uint32_t lo, uint32_t sel) const { return vperm(hi, lo, sel); }
};

// misclassified byte values of the class map (code[b] per byte) with tables t
static int misclassified(const ppr::SlotTables& t, const int* code, uint32_t cb, std::mt19937& rng)
{
    const uint32_t cm = (1u << cb) - 1u, cm4 = cm * 0x04040404u;
    int bad = 0;
    for (int b = 0; b < 256; ++b)
        for (int k = 0; k < 4; ++k) {
            const uint32_t other = rng();
            const uint32_t w = (other & ~(0xffu << (8 * k))) | ((uint32_t)b << (8 * k));
            const uint32_t got = (ppr::slot_codes4(w, t, cm4, Perm{}) >> (8 * k + 2)) & cm;
            if (got != (uint32_t)code[b]) ++bad;
        }
    return bad;
}

int main()
{
    std::mt19937 rng(12345);
    // the vperm emulation itself, on the cases the classification leans on
    if (vperm(0x87654321u, 0x0fedcba9u, 0x0d0c0b08u) != 0xff00ffffu ||
        vperm(0x00000000u, 0x00ff00ffu, 0x0a090807u) != 0x00000000u ||
        vperm(0x11223344u, 0x55667788u, 0x07000403u) != 0x11884455u) {
        std::printf("vperm emulation wrong\n");
        return 1;
    }
    int tables = 0, skipped = 0;
    const int fixed[][5] = {{',', '\n', '"', -1, -1}, {'\t', '\n', '"', '#', -1}, {'|', '\r', '\n', '\'', '\\'}};
    for (int trial = 0; trial < 3000; ++trial) {
        uint8_t specials[8], scode[8];
        int ns = 0;
        const uint32_t cb = 2 + (uint32_t)(trial % 3);
        const uint32_t catch_code = (1u << cb) - 1u;
        if (trial < 9) {
            for (int i = 0; i < 5 && fixed[trial % 3][i] >= 0; ++i) specials[ns++] = (uint8_t)fixed[trial % 3][i];
        } else {
            ns = 1 + (int)(rng() % 8);
            for (int i = 0; i < ns; ++i) {
                uint8_t b;
                bool dup;
                do {
                    b = (uint8_t)rng();
                    dup = false;
                    for (int j = 0; j < i; ++j) dup |= specials[j] == b;
                } while (dup);
                specials[i] = b;
            }
        }
        for (int i = 0; i < ns; ++i) scode[i] = (uint8_t)(rng() % catch_code);
        ppr::SlotTables t;
        if (!ppr::build_slot_tables(specials, scode, ns, catch_code, t)) {
            if (trial < 9) {  // the delimiter-separated tables of the workloads must have one
                std::printf("trial %d: no slot function for a fixed table\n", trial);
                return 1;
            }
            ++skipped;
            continue;
        }
        int code[256];
        for (int b = 0; b < 256; ++b) code[b] = (int)catch_code;
        for (int i = 0; i < ns; ++i) code[specials[i]] = scode[i];
        const int bad = misclassified(t, code, cb, rng);
        if (bad) {
            std::printf("trial %d (%d specials): %d misclassified byte positions\n", trial, ns, bad);
            return 1;
        }
        ++tables;
    }
    // a slot function that reads bits 4-6 only, with key 0: a byte differing
    // from a special by 12 shares its slot and must be taken for it
    {
        ppr::SlotTables t;
        const uint8_t sp[1] = {0x2c}, sc[1] = {0};
        if (!ppr::build_slot_tables(sp, sc, 1, 3u, t)) return 1;
        t.sh1 = 4;
        t.m1 = 0x07070707u;
        t.sh2 = 0;
        t.m2 = 0;
        uint8_t exp[8];
        for (int sl = 0; sl < 8; ++sl) exp[sl] = (uint8_t)(sl == ((0x2c >> 4) & 7) ? 0x2c : (sl == 0 ? 0x70 : 0x00));
        t.exp_lo = exp[0] | exp[1] << 8 | exp[2] << 16 | (uint32_t)exp[3] << 24;
        t.exp_hi = exp[4] | exp[5] << 8 | exp[6] << 16 | (uint32_t)exp[7] << 24;
        t.cls_lo = t.cls_hi = 0x0c0c0c0cu;
        t.cls_lo = (t.cls_lo & ~(0xffu << 16)) | (0u << 16);  // slot 2 (0x2c >> 4) holds the special, code 0
        t.hit_lo = 0xffffff00u;
        t.hit_hi = 0xffffffffu;
        int code[256];
        for (int b = 0; b < 256; ++b) code[b] = 3;
        code[0x2c] = 0;
        if (misclassified(t, code, 2, rng) == 0) {
            std::printf("the bad table passed: the check cannot see selector 12\n");
            return 1;
        }
    }
    std::printf("slots ok: %d tables checked, %d without a slot function\n", tables, skipped);
    return tables > 2000 ? 0 : 1;
}
