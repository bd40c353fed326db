// Symbol classification of the table-driven CSV kernels: the slot tables
// (built on the host) and the classification of four bytes (run by the
// kernels), with no device code of their own, so that a host build can check
// every byte value against the class map.
//
// ParPaRaw (Sec. 3, symbol matching) compares each byte with the symbols of
// the DFA by SWAR. Here each byte maps to a 3-bit slot from two bit fields,
// ((b >> sh1) & m1) | ((b >> sh2) & m2); the slots of the special bytes (every
// byte not of the catch-all class) differ, and one byte permute (v_perm)
// fetches the slot's special byte, another its code. A third permute, of the
// difference, decides whether the byte is that special byte exactly.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define PPR_SLOTS_HD __host__ __device__
#else
#define PPR_SLOTS_HD
#endif

namespace ppr {

struct SlotTables {
    uint32_t sh1, m1, sh2, m2;  // slot = ((byte >> sh1) & m1) | ((byte >> sh2) & m2); m1, m2 per byte
    uint32_t exp_lo, exp_hi;    // per slot: its special byte (or a filler) XORed with the key
    uint32_t cls_lo, cls_hi;    // per slot: 4 x the code of its special byte (the catch-all code for a filler)
    uint32_t hit_lo, hit_hi;    // byte select table: 0x00 at the key, 0xff elsewhere
};

// Symbol codes, times 4, of the four bytes of w (code << 2 in each byte).
// PERM(hi, lo, sel) is v_perm_b32: byte k of the result is byte sel.k of the
// 8-byte value {hi, lo} for selectors 0-7, the sign of byte 1, 3, 5 or 7 of
// it (as 0x00 / 0xff) for 8-11, 0x00 for 12 and 0xff for 13-255. The
// difference b ^ (x ^ key) of a byte b and its slot's special byte x selects
// the hit table's 0x00 exactly when b = x (selector key) or when the
// difference is 12, which the host's choice of slot function and key rules
// out; every other selector yields 0xff, the catch-all.
template <typename Perm>
PPR_SLOTS_HD inline uint32_t slot_codes4(uint32_t w, const SlotTables& t, uint32_t cm4, const Perm& perm)
{
    const uint32_t h = ((w >> t.sh1) & t.m1) | ((w >> t.sh2) & t.m2);
    const uint32_t miss = perm(t.hit_hi, t.hit_lo, w ^ perm(t.exp_hi, t.exp_lo, h));
    return (miss & cm4) | perm(t.cls_hi, t.cls_lo, h);
}

// Builds the slot tables for ns special bytes with codes code[i] (below the
// catch-all code) and the catch-all code (all ones). The slot function is the
// first two-field one (single fields first) that gives the specials distinct
// slots and that reads a bit of 12 ^ key for some key in {0, 2, 4, 6}: a byte
// that differs from its slot's special byte by exactly 12 ^ key then lies in
// another slot, so the permute's constant 0x00 for selector 12 never passes a
// byte as special. Fillers of empty slots are bytes of other slots that no
// byte of the slot equals or differs from by that. Returns false when no slot
// function separates the specials (more than 8 of them, or an unlucky set).
inline bool build_slot_tables(const uint8_t* specials, const uint8_t* code, int ns, uint32_t catch_code,
                              SlotTables& t)
{
    if (ns > 8) return false;
    int best_sh1 = -1, best_sh2 = 0;
    uint32_t best_m1 = 0, best_key = 0;
    for (int m1 = 7; m1 >= 1 && best_sh1 < 0; --m1) {
        const uint32_t m2 = 7u & ~(uint32_t)m1;
        for (int sh1 = 0; sh1 <= 5 && best_sh1 < 0; ++sh1) {
            for (int sh2 = 0; sh2 <= 7 && best_sh1 < 0; ++sh2) {
                if (m2 == 0 && sh2 != 0) continue;
                if ((m2 & 4u) && sh2 > 5) continue;
                if ((m2 & 2u) && sh2 > 6) continue;
                auto slot = [&](uint32_t b) { return ((b >> sh1) & (uint32_t)m1) | ((b >> sh2) & m2); };
                uint32_t used = 0;
                bool ok = true;
                for (int i = 0; i < ns && ok; ++i) {
                    if (used & (1u << slot(specials[i]))) ok = false;
                    used |= 1u << slot(specials[i]);
                }
                // the slot function is linear over XOR: it changes under a difference d iff slot(d) != 0
                int key = -1;
                for (uint32_t k = 0; k <= 6 && ok && key < 0; k += 2)
                    if (slot(12u ^ k) != 0u) key = (int)k;
                if (ok && key >= 0) {
                    best_sh1 = sh1;
                    best_sh2 = sh2;
                    best_m1 = (uint32_t)m1;
                    best_key = (uint32_t)key;
                }
            }
        }
    }
    if (best_sh1 < 0) return false;
    const uint32_t best_m2 = 7u & ~best_m1;
    auto slot_of = [&](uint32_t b) { return ((b >> best_sh1) & best_m1) | ((b >> best_sh2) & best_m2); };
    const uint32_t delta = 12u ^ best_key;
    uint8_t exp[8], cls[8];
    for (int sl = 0; sl < 8; ++sl) {
        int filler = -1;
        for (int b = 0; b < 256 && filler < 0; ++b)
            if (slot_of((uint32_t)b) != (uint32_t)sl && slot_of((uint32_t)b ^ delta) != (uint32_t)sl) filler = b;
        if (filler < 0) return false;
        exp[sl] = (uint8_t)filler;
        cls[sl] = (uint8_t)(catch_code << 2);
    }
    for (int i = 0; i < ns; ++i) {
        const uint32_t sl = slot_of(specials[i]);
        exp[sl] = specials[i];
        cls[sl] = (uint8_t)(code[i] << 2);
    }
    for (int sl = 0; sl < 8; ++sl) exp[sl] = (uint8_t)(exp[sl] ^ best_key);
    auto word = [](const uint8_t* b) {
        return (uint32_t)b[0] | (uint32_t)b[1] << 8 | (uint32_t)b[2] << 16 | (uint32_t)b[3] << 24;
    };
    t.sh1 = (uint32_t)best_sh1;
    t.sh2 = (uint32_t)best_sh2;
    t.m1 = best_m1 * 0x01010101u;
    t.m2 = best_m2 * 0x01010101u;
    t.exp_lo = word(exp);
    t.exp_hi = word(exp + 4);
    t.cls_lo = word(cls);
    t.cls_hi = word(cls + 4);
    t.hit_lo = best_key < 4 ? ~(0xffu << (8 * best_key)) : 0xffffffffu;
    t.hit_hi = best_key >= 4 ? ~(0xffu << (8 * (best_key - 4))) : 0xffffffffu;
    return true;
}

}  // namespace ppr
