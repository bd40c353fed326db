// Lexer table builder (host).
//
// "Lexing on the GPU: the scan is the easy part", section "A lexer is a prefix
// scan": precompute every reachable composition of partially applied
// transition functions, number them, and store composition as a k x k table of
// 16-bit identifiers; lexer.fut keeps a produces-a-token flag in bit 15.
//
// Elements: a byte c acts on the lexer state q as q -> delta[q][c] when defined
// and otherwise restarts, q -> delta[q0][c], with the flag "a token ended before
// c" set in the restarting case. An element is (f, p): the state map f and the
// map p from start states to that flag for its last byte. For non-empty a and
// b (a earlier), a.b = (f_b o f_a, p_b o f_a); the empty string's element is the
// identity on both sides. An entry's flag bit is p(q0) of the result.
//
// Construction: breadth-first closure from the identity under right
// multiplication by the distinct byte elements (every reachable element is a
// product of byte elements). For each element b != identity remember the BFS
// parent b' and byte element g with b = b'.g; then merge[a][b] =
// right[merge[a][b']][g], filled in BFS order, so the whole k x k table costs
// one lookup per entry instead of a composition of |Q|-entry maps.
#include <stdint.h>
#include <string.h>

#include <string>
#include <unordered_map>
#include <vector>

#include "ppr.h"

namespace {

struct Closure {
    uint32_t Q = 0;
    std::vector<std::string> elems;  // key: tag byte + f[Q] + p[Q]; identity = "\0"
    std::unordered_map<std::string, uint32_t> ids;
    std::vector<uint32_t> parent, gen;  // BFS parent and byte-element index
    std::vector<uint32_t> right;        // right[x * m + g] = id(x . g)
    std::vector<std::string> gens;      // distinct byte elements
    std::vector<uint32_t> byte_gen;     // byte -> generator index
};

std::string product(const std::string& a, const std::string& b, uint32_t Q)
{
    if (b.size() == 1) return a;  // b is the identity
    if (a.size() == 1) return b;
    std::string r(1 + 2 * Q, '\1');
    const uint8_t* fa = (const uint8_t*)a.data() + 1;
    const uint8_t* fb = (const uint8_t*)b.data() + 1;
    const uint8_t* pb = fb + Q;
    for (uint32_t q = 0; q < Q; ++q) {
        r[1 + q] = (char)fb[fa[q]];
        r[1 + Q + q] = (char)pb[fa[q]];
    }
    return r;
}

int closure(const int16_t* delta, uint32_t Q, uint32_t q0, uint32_t max_k, Closure& C)
{
    C.Q = Q;
    for (int c = 0; c < 256; ++c) {
        std::string e(1 + 2 * Q, '\1');
        for (uint32_t q = 0; q < Q; ++q) {
            const int16_t d = delta[q * 256 + c];
            e[1 + q] = (char)(uint8_t)(d >= 0 ? d : delta[q0 * 256 + c]);
            e[1 + Q + q] = (char)(d >= 0 ? 0 : 1);
        }
        uint32_t g = 0;
        while (g < C.gens.size() && C.gens[g] != e) ++g;
        if (g == C.gens.size()) C.gens.push_back(e);
        C.byte_gen.push_back(g);
    }
    const uint32_t m = (uint32_t)C.gens.size();
    C.elems.push_back(std::string(1, '\0'));
    C.ids.emplace(C.elems[0], 0u);
    C.parent.push_back(0);
    C.gen.push_back(0);
    for (size_t i = 0; i < C.elems.size(); ++i) {
        for (uint32_t g = 0; g < m; ++g) {
            std::string y = product(C.elems[i], C.gens[g], Q);
            auto it = C.ids.find(y);
            uint32_t id;
            if (it == C.ids.end()) {
                if (C.elems.size() >= max_k) return PPR_ECAPACITY;
                id = (uint32_t)C.elems.size();
                C.ids.emplace(y, id);
                C.elems.push_back(std::move(y));
                C.parent.push_back((uint32_t)i);
                C.gen.push_back(g);
            } else {
                id = it->second;
            }
            C.right.push_back(id);
        }
    }
    return PPR_OK;
}

}  // namespace

extern "C" int ppr_lex_build_tables(const int16_t* delta, const uint16_t* kind, uint32_t n_states, uint32_t q0,
                                    uint32_t max_k, uint32_t* k_out, uint16_t* initial_state, uint16_t* merge_table,
                                    uint16_t* final_states, uint16_t* identity_out)
{
    if (!delta || !kind || !k_out || n_states == 0 || n_states > 255 || q0 >= n_states) return PPR_EINVAL;
    if (max_k == 0 || max_k > 0x8000u) return PPR_EINVAL;
    for (uint32_t q = 0; q < n_states; ++q)
        for (int c = 0; c < 256; ++c) {
            const int16_t d = delta[q * 256 + c];
            if (d >= (int16_t)n_states || d < -1) return PPR_EINVAL;
            if (q == q0 && d < 0) return PPR_EINVAL;
        }
    Closure C;
    int rc = closure(delta, n_states, q0, max_k, C);
    if (rc != PPR_OK) {
        *k_out = max_k + 1;
        return rc;
    }
    const uint32_t k = (uint32_t)C.elems.size(), m = (uint32_t)C.gens.size(), Q = n_states;
    *k_out = k;
    if (!merge_table) return PPR_OK;
    if (!initial_state || !final_states) return PPR_EINVAL;
    std::vector<uint16_t> flag(k), id(k * (size_t)k);
    for (uint32_t x = 0; x < k; ++x) {
        const std::string& e = C.elems[x];
        flag[x] = (e.size() > 1 && e[1 + Q + q0]) ? 0x8000u : 0u;
        const uint32_t f0 = e.size() > 1 ? (uint8_t)e[1 + q0] : q0;
        final_states[x] = kind[f0];
    }
    for (uint32_t a = 0; a < k; ++a) {
        uint16_t* row = &id[(size_t)a * k];
        row[0] = (uint16_t)a;
        for (uint32_t b = 1; b < k; ++b) row[b] = (uint16_t)C.right[(size_t)row[C.parent[b]] * m + C.gen[b]];
    }
    for (size_t i = 0; i < (size_t)k * k; ++i) merge_table[i] = (uint16_t)(id[i] | flag[id[i]]);
    for (int c = 0; c < 256; ++c) {
        const uint32_t x = C.right[(size_t)0 * m + C.byte_gen[c]];
        initial_state[c] = (uint16_t)(x | flag[x]);
    }
    if (identity_out) *identity_out = 0;
    return PPR_OK;
}

extern "C" const char* ppr_version(void) { return "ppr 0.1 (gfx950)"; }
