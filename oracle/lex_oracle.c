/*
 * CPU oracles for the lexer: the restart lexer and the table-driven fold.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header or table with the GPU path.
 *
 * Source: "Lexing on the GPU: the scan is the easy part".
 *
 * oracle_lex_restart follows the section "A lexer is a prefix scan": a lexer
 * is a loop over bytes with one state variable, q_{i+1} = delta(q_i, a_i). A
 * token ends where the DFA has no continuation; the next token starts at that
 * byte from the start state q0. The start state's row is total (a byte that
 * starts no token leads to the dead state E, whose token kind is ERROR), so
 * the first byte never ends a token. Every token is reported, whitespace and
 * comments included; the kind of a token is the kind accepted in the state its
 * last byte leaves the DFA in (ERROR if that state accepts nothing). The last
 * token ends at n, accepted or not (section "Does it produce the same
 * tokens?": a trailing token in a non-accepting state comes out as an error).
 *
 * oracle_lex_fold follows the same page's description of the precomputed
 * tables (section "A lexer is a prefix scan") and of the harness in "Does it
 * produce the same tokens?": the state after each prefix is the previous
 * prefix's identifier merged with the identifier of the next byte, one table
 * load per byte; a set flag bit on the merged identifier marks that a token
 * ended just before this byte, and the ended token's kind is read from the
 * final-state table at the previous prefix. Bytes index the tables unsigned.
 * The flag bit is masked off both operands before the lookup.
 */
#include <stdint.h>

static void put(uint32_t* kind, uint32_t* start, uint32_t* len, uint64_t cap, uint64_t* nt, uint32_t k, uint64_t s,
                uint64_t l)
{
    if (*nt < cap) {
        kind[*nt] = k;
        start[*nt] = (uint32_t)s;
        len[*nt] = (uint32_t)l;
    }
    (*nt)++;
}

/* delta: row-major [n_states][256], -1 = no continuation; kind_of: [n_states] */
int oracle_lex_restart(const uint8_t* bytes, uint64_t n, uint32_t q0, const int16_t* delta, const uint16_t* kind_of,
                       uint32_t* kind, uint32_t* start, uint32_t* len, uint64_t cap, uint64_t* n_tokens)
{
    uint64_t nt = 0, tok_start = 0;
    uint32_t q = q0;
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t b = bytes[i];
        int32_t d = delta[(uint64_t)q * 256 + b];
        if (d >= 0) {
            q = (uint32_t)d;
        } else {
            put(kind, start, len, cap, &nt, kind_of[q], tok_start, i - tok_start);
            tok_start = i;
            q = (uint32_t)delta[(uint64_t)q0 * 256 + b];
        }
    }
    if (n > 0) put(kind, start, len, cap, &nt, kind_of[q], tok_start, n - tok_start);
    *n_tokens = nt;
    return nt > cap ? -2 : 0;
}

/* init: [256]; merge: row-major [k][k], row = earlier operand; final_: [k] */
int oracle_lex_fold(const uint8_t* bytes, uint64_t n, const uint16_t* init, const uint16_t* merge,
                    const uint16_t* final_, uint32_t k, uint16_t flag_mask, uint32_t* kind, uint32_t* start,
                    uint32_t* len, uint64_t cap, uint64_t* n_tokens)
{
    uint64_t nt = 0, tok_start = 0;
    if (n == 0) {
        *n_tokens = 0;
        return 0;
    }
    uint16_t id_mask = (uint16_t)~flag_mask;
    uint16_t prev = (uint16_t)(init[bytes[0]] & id_mask); /* a flag on the first byte ends no token */
    for (uint64_t i = 1; i < n; ++i) {
        uint16_t x = init[bytes[i]] & id_mask;
        uint16_t m = merge[(uint64_t)prev * k + x];
        if (m & flag_mask) {
            put(kind, start, len, cap, &nt, final_[prev], tok_start, i - tok_start);
            tok_start = i;
        }
        prev = m & id_mask;
    }
    put(kind, start, len, cap, &nt, final_[prev], tok_start, n - tok_start);
    *n_tokens = nt;
    return nt > cap ? -2 : 0;
}
