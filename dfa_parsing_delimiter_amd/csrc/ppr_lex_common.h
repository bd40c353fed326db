// Types shared by the lexer's host code and its streaming kernels.
//
// Method: "Lexing on the GPU: the scan is the easy part", section "A lexer is a
// prefix scan": bytes map to identifiers of transition functions, identifiers
// compose through a k x k merge table, and the state after every prefix is an
// inclusive scan under that composition; a flag on a merged identifier marks a
// token boundary, and the final-state table gives the kind of the token that
// ends there (section "Does it produce the same tokens?").
#pragma once

#include <algorithm>

#include "ppr.h"
#include "ppr_device.h"
#include "ppr_host.h"

namespace ppr {

// streaming lexer geometry: 512 threads x 40-byte chunks per tile
constexpr int kLexFastBlock = 512;
constexpr int kLexFastWaves = kLexFastBlock / kWave;
constexpr int kLexFastChunk = 40;
constexpr int kLexFastTile = kLexFastBlock * kLexFastChunk;
constexpr uint32_t kLexMaxRanges = 1024;
// LDS budgets of the streaming kernels' tables (two workgroups per CU)
constexpr uint32_t kLexRowLds = 80u << 10;     // fold rows (2-byte entries)
constexpr uint32_t kLexStepLds = 16u << 10;    // minimal automaton (4-byte entries)
constexpr uint32_t kLexStateLds = 8u << 10;    // state of each identifier (2-byte entries)

struct LexFastParams {
    const uint8_t* in;
    uint32_t n, num_tiles, num_ranges;
    uint32_t k, m, identity, id_mask;
    uint32_t row0;    // the identity's fold row, times m
    uint32_t n_rows;  // fold rows
    uint32_t nq;      // minimal automaton states
    const uint16_t* merge;       // k x k: identifier of the product (flag bit masked with id_mask)
    const uint16_t* final_;      // k: token kind
    const uint16_t* next_row;    // n_rows x m: the row reached by one more byte of column j, times m
    const uint16_t* row_id;      // n_rows x m: the identifier reached
    const uint16_t* state_of;    // k: minimal automaton state of an identifier
    const uint32_t* step;        // nq x m: successor state | flag << 16
    const uint16_t* state_kind;  // nq: kind of the token ending in a state
    uint16_t* chunk_id;          // per chunk: identifier of its tile's bytes before it
    uint32_t* tile_id;           // per tile: identifier of its bytes
    uint32_t* range_id;          // per range: identifier of its tiles' bytes
    uint2* range_tok;            // per range: boundaries in it, 1 + position of its last one (0: none)
    uint32_t* kind;
    uint32_t* start;
    uint32_t* len;
    uint64_t cap;
    WsHeader* hdr;
    uint8_t col[256];  // column of each byte
};

struct LexFastLayout {
    uint64_t tiles, ranges, chunk_id, tile_id, range_id, range_tok, total;
};

inline LexFastLayout lex_fast_layout(uint64_t n)
{
    LexFastLayout L;
    L.tiles = (n + kLexFastTile - 1) / kLexFastTile;
    L.ranges = std::min<uint64_t>(L.tiles, kLexMaxRanges);
    L.chunk_id = 256;
    L.tile_id = align_up(L.chunk_id + L.tiles * kLexFastBlock * 2u, 256);
    L.range_id = align_up(L.tile_id + L.tiles * 4u, 256);
    L.range_tok = align_up(L.range_id + kLexMaxRanges * 4u, 256);
    L.total = align_up(L.range_tok + kLexMaxRanges * 8u, 256);
    return L;
}

// Enqueue the streaming lexer kernels.
int launch_lex_fast(const LexFastParams& p, const ppr_parse_opts_t* opts, hipStream_t s);

}  // namespace ppr
