/*
 * ppr.h — data-parallel DFA parsing of delimiter-separated bytes and
 * table-driven lexing on one AMD Instinct MI355X (gfx950).
 *
 * Method sources:
 *   [P] "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated Raw Data":
 *       Sec. 3 (parsing context: one DFA instance per state per chunk, the
 *       state-transition vector, its composite and the exclusive scan seeded with
 *       the identity vector, Fig. 2; tagging: record and field delimiter bitmaps;
 *       offsets: record counts and relative/absolute column offsets, Fig. 4) and
 *       "validating format" (invalid transitions, non-accepting end state).
 *   [L] "Lexing on the GPU: the scan is the easy part": "A lexer is a prefix
 *       scan" (composition of partially applied transition functions as a scan,
 *       every reachable composition numbered, composition as a k x k table of
 *       16-bit identifiers, a produces-a-token flag bit masked off both operands)
 *       and "Does it produce the same tokens?" (the final-state table gives the
 *       kind of the token ending at a flagged position; bytes index unsigned).
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device pointers (hipMalloc or torch CUDA memory) of
 *     the current HIP device; all other pointers are host pointers.
 *   - The caller owns every buffer. The library allocates nothing on the device
 *     in these calls; the workspace is caller-provided.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on
 *     it; calls sharing one workspace must be ordered on one stream.
 *   - Return value: PPR_OK or a negative PPR_E* code. A malformed input is data,
 *     not an error: it is reported through error_pos with PPR_OK.
 *   - Blocking calls (ppr_parse, ppr_lex) return after the scalar results have
 *     been copied back; the *_async forms leave them in the workspace for
 *     ppr_*_results to read.
 */
#ifndef PPR_H
#define PPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these entry points are exported. */
#define PPR_API __attribute__((visibility("default")))

#define PPR_MAX_STATES 8
#define PPR_MAX_CLASSES 16

/* Per-byte tags, the Mealy output of reading a symbol class in a state [P Sec. 3, tagging]. */
enum ppr_tag { PPR_TAG_VALUE = 0, PPR_TAG_FIELD = 1, PPR_TAG_RECORD = 2, PPR_TAG_INVALID = 3 };

enum ppr_status {
    PPR_OK = 0,
    PPR_EINVAL = -1,     /* bad table, bad option, NULL pointer */
    PPR_ECAPACITY = -2,  /* output arrays too small; the counts are still reported */
    PPR_ETOOBIG = -3,    /* n too large for one call */
    PPR_EHIP = -4,       /* a HIP runtime call failed */
    PPR_EWORKSPACE = -5  /* workspace too small or misaligned */
};

/*
 * DFA over symbol classes [P Sec. 3, Fig. 3; symbol groups, Table 1].
 *   n_states in [1, 8], n_classes in [1, 16]; states and classes are indices.
 *   next[s][c]: state after reading a byte of class c in state s (< n_states).
 *   tag[s][c]:  ppr_tag of that byte.
 *   start_state: state before the first byte.
 *   accept_mask: bit s set if s is an accepting end state.
 * Entries for s >= n_states or c >= n_classes are ignored.
 */
typedef struct ppr_dfa {
    uint32_t n_states;
    uint32_t n_classes;
    uint32_t start_state;
    uint32_t accept_mask;
    uint8_t next[PPR_MAX_STATES][PPR_MAX_CLASSES];
    uint8_t tag[PPR_MAX_STATES][PPR_MAX_CLASSES];
} ppr_dfa_t;

/*
 * Per-field output [P Sec. 3, offsets and tagging, Fig. 4], one entry per field
 * in input order. A field ends at each FIELD or RECORD byte; if the input is
 * non-empty and its last byte is not tagged RECORD, the unterminated rest is one
 * more field (and record).
 *   record_idx[i]    records completed before field i,
 *   column_ids[i]    FIELD bytes since the last RECORD byte (or the start),
 *   field_offsets[i] first byte of the raw span (byte after the previous terminator, or 0),
 *   field_lengths[i] bytes from the offset up to (not including) the terminator, or to n.
 * Device arrays of cap_fields entries each. Entries beyond cap_fields are not
 * written; n_fields reports the full count.
 */
typedef struct ppr_parse_out {
    uint32_t* record_idx;
    uint32_t* column_ids;
    uint32_t* field_offsets;
    uint32_t* field_lengths;
    uint64_t cap_fields;
    uint64_t n_fields;  /* out */
    uint64_t n_records; /* out */
    int64_t error_pos;  /* out: first INVALID byte; else n if the end state is not accepting; else -1 */
    uint32_t end_state; /* out: DFA state after the last byte */
    uint32_t path;      /* out: the kernels that ran, a PPR_PATH_* value */
    /* out: the fewest and the most fields of any record (0 and 0 without records).
     * [ParPaRaw, "Inferring or validating number of columns"]: the
     * largest is the inferred number of columns; the records all conform to one
     * number of columns exactly when the two are equal. */
    uint32_t min_columns;
    uint32_t max_columns;
    /* out, with opts->expected_columns > 0 (else 0 and -1): the records whose
     * number of fields is not expected_columns, how many and the index of the
     * first (-1: none). [ParPaRaw, "Inferring or validating number of columns",
     * and the specialisations passage: rejecting records that have an
     * inconsistent number of field delimiters.] Their fields are still written;
     * a caller that rejects them drops the fields of those records. */
    uint64_t bad_records;
    int64_t first_bad_record;
    /* out: the unterminated tail of the input (after its last terminator, 0
     * if none): where it starts and the column of its field. With
     * PPR_PARSE_PARTIAL, the next call continues from there. */
    uint32_t tail_start;
    uint32_t tail_column;
} ppr_parse_out_t;

/*
 * Which kernels a parse runs (chosen at the call, reported in ppr_parse_out_t.path).
 * The first two need chunk_bytes 64, a 16-byte aligned input and a class map with
 * one catch-all class and at most 8 other bytes that a 3-bit hash of two bit
 * fields separates ("table-driven" below):
 *   PPR_PATH_FUSED       table-driven, 2 kernels (step tables, one persistent
 *                        single-pass kernel with decoupled look-back scans over
 *                        32 KiB tiles): the input is read once;
 *   PPR_PATH_STREAMING   table-driven, 4 kernels (codes, range vectors,
 *                        carries, emit), no waiting between workgroups;
 *   PPR_PATH_SINGLE_PASS any table and chunk size: 2 kernels (reset, one
 *                        single-pass kernel with decoupled look-back scans).
 * The lexer has two (reported in ppr_tokens_out_t.path):
 *   PPR_PATH_STREAMING   4 kernels (chunk identifiers through the fold rows,
 *                        range identifiers, boundary counts, tokens), no waiting
 *                        between workgroups; needs chunk_bytes 40, an 8-byte
 *                        aligned input and prepared fold rows (n_rows > 0);
 *                        the automatic choice above 8 MiB;
 *   PPR_PATH_SINGLE_PASS any chunk size: 2 kernels (reset, one single-pass
 *                        kernel with decoupled look-back scans).
 */
enum { PPR_PATH_STREAMING = 1, PPR_PATH_SINGLE_PASS = 2, PPR_PATH_FUSED = 3 };

/*
 * Launch options (opts may be NULL: all defaults).
 *   chunk_bytes:    bytes each thread simulates, 1..64; 0 = 64 (parse) or 40 (lexer).
 *   stage_events:   optional array of n_stage_events hipEvent_t (caller-created):
 *                   event 0 is recorded on the stream before the first kernel of the
 *                   call and event i after its i-th kernel, as far as the array
 *                   reaches (streaming parse and lexer: 3 events, after the
 *                   first two kernels and after each of the last two; fused and
 *                   single-pass parse and lexer: 2). For per-kernel timing;
 *                   NULL: none.
 *   path:           0 = automatic (where the table and input allow the
 *                   table-driven paths: the fused kernel up to 8 MiB, the
 *                   streaming kernels above; else the single-pass path); PPR_PATH_FUSED or
 *                   PPR_PATH_STREAMING ask for that path and fall back to the
 *                   single-pass path where it does not apply; PPR_PATH_SINGLE_PASS
 *                   forces the generic kernel. Any other value: PPR_EINVAL. The
 *                   lexer treats PPR_PATH_FUSED as PPR_PATH_STREAMING; its
 *                   automatic choice is the streaming kernels above 8 MiB
 *                   (where they apply), the single-pass kernel otherwise.
 */
typedef struct ppr_parse_opts {
    uint32_t chunk_bytes;
    uint32_t n_stage_events;
    void* const* stage_events;
    uint32_t path;
    uint32_t expected_columns; /* 0: none; else records are checked against it (ppr_parse_out_t.bad_records) */
    /* Resuming a parse across calls (input cut into partitions, ParPaRaw's
     * streaming passage; ppr_parse_stream is built on it):
     *   PPR_PARSE_CONTINUE: the bytes continue an earlier call's input: start in
     *     DFA state start_state, inside a record whose open field has column
     *     start_column (the earlier call's end_state and tail_column);
     *   PPR_PARSE_PARTIAL: more input follows: the unterminated tail (after the
     *     last terminator) is not emitted as a field, no record is closed at the
     *     end, and a non-accepting end state is not an error (error_pos is only
     *     an INVALID byte); tail_start / tail_column describe the open field.
     * Offsets, record indices and columns are those of this call's bytes: a
     * field continued from an earlier call starts at offset 0 here. */
    uint32_t flags;
    uint32_t start_state;
    uint32_t start_column;
} ppr_parse_opts_t;

enum { PPR_PARSE_CONTINUE = 1, PPR_PARSE_PARTIAL = 2 };

/*
 * Workspace bytes ppr_parse needs for n input bytes (opts may be NULL).
 * The workspace must be 256-byte aligned; it needs no initialisation (every
 * call clears what it reads before writing it, so one workspace may serve
 * calls of any size and any entry point in turn); 0 on invalid arguments.
 */
PPR_API size_t ppr_parse_workspace_bytes(uint64_t n, const ppr_parse_opts_t* opts);

/*
 * Parse n bytes at d_bytes with the DFA and the 256-entry class map (host
 * pointers, validated and copied at the call). n must be at most
 * 2^32 - 2^16 (PPR_ETOOBIG otherwise: every byte position then fits 32 bits,
 * up to the end of the last tile). d_bytes needs no particular alignment.
 * Blocking: returns with out->n_fields, n_records, error_pos, end_state set.
 * Returns PPR_ECAPACITY (with the counts set) if n_fields > cap_fields.
 */
PPR_API int ppr_parse(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
              ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream);

/* Enqueue the same work without waiting; ppr_parse_results completes it. */
PPR_API int ppr_parse_async(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                    const ppr_parse_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts,
                    void* stream);

/* Wait on `stream` and copy the scalars of the last ppr_parse_async on d_ws into out.
 * The copy goes through a 256-byte pinned host buffer that belongs to the
 * calling thread. It is allocated (hipHostMalloc) on the thread's first blocking
 * call (ppr_parse, ppr_parse_results, ppr_lex, ppr_lex_results) and kept until
 * the process ends. If that allocation fails, the copy goes into the stack
 * instead. ppr_parse_noalloc never uses it. */
PPR_API int ppr_parse_results(const void* d_ws, uint64_t n, ppr_parse_out_t* out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the parse of
 * ppr_parse, blocking, with no workspace argument. Its workspace is a fixed
 * array of PPR_NOALLOC_SCRATCH_BYTES in the library's own device memory (one
 * per GPU, held until the process ends); the call allocates nothing. The
 * caller still provides the input and the output arrays.
 *   - The streaming kernels are never used (their workspace grows with n):
 *     table-driven inputs run the fused kernel, others the generic kernel;
 *     opts->path PPR_PATH_STREAMING is read as PPR_PATH_FUSED.
 *   - PPR_ETOOBIG if the call's look-back statuses do not fit the scratch: never
 *     for table-driven inputs up to 2^32 - 2^16 bytes; with the generic kernel,
 *     above about 233,000 tiles of 1024 chunks of chunk_bytes.
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap in
 *     time on one GPU (other streams, other host threads) race and must not be
 *     made. Each call clears what it needs at zero (its header and look-back
 *     statuses) with kernels on `stream`; the scratch keeps the last call's contents.
 * Otherwise as ppr_parse (arguments, results, PPR_ECAPACITY).
 */
#define PPR_NOALLOC_SCRATCH_BYTES (16u << 20)
PPR_API int ppr_parse_noalloc(const uint8_t* d_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                              ppr_parse_out_t* out, const ppr_parse_opts_t* opts, void* stream);

/*
 * Host streaming [ParPaRaw, the end-to-end streaming passage, Fig. 7]: parse
 * n bytes of HOST memory, any size, by cutting them into partitions of
 * partition_bytes and running, on three HIP streams, the transfer of one
 * partition to the device, the parse of the one before and the return of
 * the one before that, with two device buffers used in turn. A partition
 * continues the previous one's parse (PPR_PARSE_CONTINUE with its end state
 * and open column, PPR_PARSE_PARTIAL on all but the last), so no incomplete
 * record has to be copied over and parsed again and records may span any
 * number of partitions. The results are those of one parse over the whole
 * input, with 64-bit record indices, offsets and lengths.
 *   out: host arrays of cap_fields entries each (pinned memory lets the
 *        returns overlap the parse); n_fields etc. as for ppr_parse.
 *   opts: chunk_bytes, path and expected_columns as for ppr_parse (flags,
 *        start_state, start_column must be 0; stage events are ignored).
 * Unlike ppr_parse, this driver allocates (and frees before it returns) its
 * device buffers (2 x (partition + workspace + outputs)) and streams.
 * PPR_ECAPACITY with the counts set if n_fields > cap_fields; PPR_EINVAL for
 * partition_bytes of 0 or above 2^32 - 2^16.
 */
typedef struct ppr_stream_out {
    uint64_t* record_idx;
    uint32_t* column_ids;
    uint64_t* field_offsets;
    uint64_t* field_lengths;
    uint64_t cap_fields;
    uint64_t n_fields;      /* out */
    uint64_t n_records;     /* out */
    int64_t error_pos;      /* out */
    uint32_t end_state;     /* out */
    uint32_t min_columns;   /* out */
    uint32_t max_columns;   /* out */
    uint32_t partitions;    /* out: partitions parsed */
    uint64_t bad_records;   /* out */
    int64_t first_bad_record; /* out */
} ppr_stream_out_t;

PPR_API int ppr_parse_stream(const uint8_t* h_bytes, uint64_t n, const ppr_dfa_t* dfa, const uint8_t class_map[256],
                             ppr_stream_out_t* out, uint64_t partition_bytes, const ppr_parse_opts_t* opts);

/*
 * Columnar partition [P Sec. 3: symbols partitioned by column with a stable
 * sort on their column tags, each column's concatenated symbol string (CSS),
 * and an index of each field's record, offset and number of symbols, Fig. 5;
 * the specialisations passage: inline-terminated and vector-delimited CSS,
 * Fig. 6]. Input: the bytes a parse read and its per-field arrays (device,
 * n_fields entries each; column ids below n_columns, at most 4096; a parse's
 * max_columns is the right n_columns). Output, all device memory the caller
 * provides:
 *   rec, css_off, length [n_fields]: one entry per field, grouped by column
 *     (column 0's fields, in input order, then column 1's, ...): the field's
 *     record, the offset of its first byte in css, its length;
 *   col_first_field, col_first_byte [n_columns + 1]: where each column's
 *     entries and bytes start (the last element: n_fields and css_bytes);
 *   css [css_cap]: the fields' raw spans (quotes included) in that order.
 *     mode PPR_CSS_INDEXED: nothing between fields; PPR_CSS_INLINE: each field
 *     followed by the byte `terminator` (e.g. 0x1E or 0x1F); PPR_CSS_VECTOR:
 *     each field followed by a 0 byte, and aux[css_cap] holds 1 at those slots
 *     and 0 elsewhere (so a field may hold any byte).
 * Blocking; returns css_bytes. PPR_ECAPACITY (css_bytes set, nothing written
 * at or beyond css_cap) if css_bytes > css_cap; PPR_EINVAL if a column id is
 * not below n_columns (detected on the device: the outputs are then
 * undefined); PPR_ETOOBIG if a CSS offset could exceed 32 bits. The workspace
 * (ppr_columns_workspace_bytes, 256-byte aligned) needs no initialisation.
 * opts may be NULL; only its stage_events are read: events recorded before
 * the first and after each of the six kernels (reset, histogram, scan of the
 * counts, scan of the bytes, partition, bounds; recorded in place of those
 * skipped when n_fields is 0).
 */
enum { PPR_CSS_INDEXED = 0, PPR_CSS_INLINE = 1, PPR_CSS_VECTOR = 2 };

typedef struct ppr_columns_out {
    uint8_t* css;
    uint8_t* aux;
    uint64_t css_cap;
    uint32_t* rec;
    uint32_t* css_off;
    uint32_t* length;
    uint32_t* col_first_field;
    uint32_t* col_first_byte;
    uint64_t css_bytes; /* out */
} ppr_columns_out_t;

PPR_API size_t ppr_columns_workspace_bytes(uint64_t n_fields, uint32_t n_columns);

PPR_API int ppr_columns(const uint8_t* d_bytes, uint64_t n, const uint32_t* d_rec, const uint32_t* d_col,
                        const uint32_t* d_off, const uint32_t* d_len, uint64_t n_fields, uint32_t n_columns,
                        uint32_t mode, uint32_t terminator, ppr_columns_out_t* out, void* d_ws, size_t ws_bytes,
                        const ppr_parse_opts_t* opts, void* stream);

/* ------------------------------------------------------------------ lexer */

/*
 * Lexer tables [L, "A lexer is a prefix scan"]. Device pointers.
 *   initial_state[256]: element identifier of each byte (flag bit allowed).
 *   merge_table[k*k]:   row a, column b = identifier of "a then b" with the flag
 *                       bit set when its last byte ends a token; a is the earlier
 *                       operand. Flag bits are masked off both operands first.
 *   final_states[k]:    token kind of the token ending at a prefix whose
 *                       identifier is x.
 *   identity:           identifier of the empty string (neutral on both sides).
 *   flag_mask:          the flag bit (0x8000); identifiers are < k <= flag_mask.
 */
typedef struct ppr_lex_tables {
    const uint16_t* initial_state;
    const uint16_t* merge_table;
    const uint16_t* final_states;
    uint32_t k;
    uint16_t identity;
    uint16_t flag_mask;
} ppr_lex_tables_t;

/*
 * Prepared form of the tables for the kernels, filled by ppr_lex_prepare:
 * bytes with the same initial identifier share a column, and d_fold holds,
 * for every identifier x and column j, merge_table[x][column j's identifier]
 * (k * m entries, device memory the caller provides). After those entries the
 * same buffer holds the minimal automaton of that fold (identifiers that give
 * the same flags and token kinds on every continuation share a state; found by
 * partition refinement): the state of each identifier, and per state and
 * column its successor state and flag, and its token kind. Lexing from a known
 * prefix (the second pass over a chunk) steps through this small automaton.
 * Then the fold rows of the streaming lexer kernels: identifiers whose rows of
 * the fold name the same identifiers share a row; per row and column, the row
 * reached (times m) and the identifier reached. The first pass over a chunk
 * walks these rows in LDS.
 */
typedef struct ppr_lex_prepared {
    uint16_t* d_fold;      /* caller-provided device buffer of ppr_lex_fold_bytes(k) bytes */
    uint32_t k;
    uint32_t m;            /* out: number of columns */
    uint16_t identity;
    uint16_t flag_mask;
    uint8_t column_of[256]; /* out: column of each byte */
    uint32_t n_states;     /* out: states of the minimal automaton (0: it does not fit the buffer; not used) */
    uint32_t n_rows;       /* out: fold rows (0: the streaming kernels are not used: their tables do not fit
                              their LDS budgets, a token kind exceeds 255, or m exceeds 64) */
    uint32_t row0;         /* out: the identity's row, times m */
} ppr_lex_prepared_t;

/* Device bytes the prepared fold table needs (k * 256 * 2 at most). */
PPR_API size_t ppr_lex_fold_bytes(uint32_t k);

/* Build the prepared tables (reads initial_state back; blocking). */
PPR_API int ppr_lex_prepare(const ppr_lex_tables_t* tables, ppr_lex_prepared_t* prep, void* stream);

/*
 * Token output, one entry per token in input order: kind = final_states of the
 * prefix ending at the token's last byte, start, length. Every byte belongs to
 * exactly one token; a token ends before each byte whose merged identifier has
 * the flag bit (position 0 excepted) and at n.
 */
typedef struct ppr_tokens_out {
    uint32_t* kind;
    uint32_t* start;
    uint32_t* length;
    uint64_t cap_tokens;
    uint64_t n_tokens; /* out */
    uint32_t path;     /* out: the kernels that ran (PPR_PATH_STREAMING or PPR_PATH_SINGLE_PASS) */
} ppr_tokens_out_t;

/* Workspace bytes ppr_lex needs for n input bytes (opts may be NULL): 256-byte
 * aligned, no initialisation needed; 0 on invalid arguments. */
PPR_API size_t ppr_lex_workspace_bytes(uint64_t n, const ppr_parse_opts_t* opts);

/* Lex n bytes (n <= 2^32 - 2^16, else PPR_ETOOBIG). Blocking. PPR_ECAPACITY if n_tokens > cap_tokens. */
PPR_API int ppr_lex(const uint8_t* d_bytes, uint64_t n, const ppr_lex_tables_t* tables, const ppr_lex_prepared_t* prep,
            ppr_tokens_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts, void* stream);

PPR_API int ppr_lex_async(const uint8_t* d_bytes, uint64_t n, const ppr_lex_tables_t* tables, const ppr_lex_prepared_t* prep,
                  const ppr_tokens_out_t* out, void* d_ws, size_t ws_bytes, const ppr_parse_opts_t* opts,
                  void* stream);

PPR_API int ppr_lex_results(const void* d_ws, uint64_t n, ppr_tokens_out_t* out, void* stream);

/*
 * Build lexer tables from a token DFA [L, "A lexer is a prefix scan"]: the element
 * of byte c maps state q to delta[q][c] when defined and otherwise restarts from
 * q0 (delta[q0][c]), flagging that a token ended; elements compose left to
 * right; the empty string is the identity. Host memory throughout.
 *   delta: [n_states][256], -1 = undefined; delta[q0][*] must all be defined.
 *   kind:  [n_states] token kind accepted in each state.
 * First call with merge_table == NULL to get k (in *k_out); then call again with
 * initial_state[256], merge_table[k*k], final_states[k] allocated.
 * PPR_ECAPACITY if the closure exceeds max_k (then *k_out = max_k + 1).
 */
PPR_API int ppr_lex_build_tables(const int16_t* delta, const uint16_t* kind, uint32_t n_states, uint32_t q0,
                         uint32_t max_k, uint32_t* k_out, uint16_t* initial_state, uint16_t* merge_table,
                         uint16_t* final_states, uint16_t* identity_out);

/* Library version string. */
PPR_API const char* ppr_version(void);

/* ------------------------------------------------------------ diagnostics */

/*
 * Bandwidth probe (not part of the method): enqueues one kernel on `stream`
 * that streams `bytes` (a multiple of 16 KiB) of device memory, so that the
 * caller can time the device's own read / write / copy rate with events and
 * compare the kernels' traffic with it.
 *   mode 0: read d_src; d_dst receives one 32-bit word per thread
 *           (grid * 256 * 4 bytes), so the loads are not optimised away;
 *   mode 1: write d_dst (d_src unused, may be NULL);
 *   mode 2: copy d_src to d_dst (`bytes` each).
 *   pattern 0: wave-contiguous 16-byte words (one instruction covers 1 KiB);
 *   pattern 1: 64 contiguous bytes per lane (the CSV codes kernel's layout);
 *   pattern 2: wave-contiguous 4-byte words (one instruction covers 256 bytes:
 *              the shape of the field and token stores).
 *   grid: workgroups of 256 threads (a grid-stride loop covers the buffer).
 * Pointers must be 16-byte aligned. PPR_EINVAL on bad arguments.
 */
PPR_API int ppr_bandwidth_probe(uint32_t mode, uint32_t pattern, const void* d_src, void* d_dst, uint64_t bytes,
                                uint32_t grid, void* stream);

/*
 * Numeric type inference and conversion [P "Type inference" (each field's
 * minimal numerical type, a reduction over the column's fields), "Default
 * values for empty strings", and Sec. 3 (fields converted to their column's
 * type, threads alone on short fields and collaborating on long ones)].
 *
 * A field is a span (off, len) of `bytes` (device): a parse's fields in the
 * input, or a CSS index's entries in the CSS. Its text is the raw span (quotes
 * included: a quoted number is TEXT). Types, ordered:
 *   EMPTY (no symbols) < INT8 < INT16 < INT32 < INT64 < FLOAT64 < TEXT.
 * INT: optional sign and decimal digits, typed by the smallest signed width
 * holding the value (beyond int64: FLOAT64). FLOAT64: optional sign, digits
 * with a point (a digit on at least one side) or without, then an optional
 * exponent (e/E, optional sign, digits), with a point or an exponent present.
 * Anything else is TEXT. A column's type is the largest of its fields'.
 *
 * Columns: col[j] per field (device, may be NULL); else col_first[n_columns +
 * 1] (device: fields grouped by column, as ppr_columns' col_first_field); else
 * a single column. 1 <= n_columns <= 4096. A column id >= n_columns counts in
 * no column (its field converts to PPR_NUM_NOT_CONVERTED). A span past
 * n_bytes is TEXT (never for a parse's own fields).
 */
enum { PPR_NUM_EMPTY = 0, PPR_NUM_INT8 = 1, PPR_NUM_INT16 = 2, PPR_NUM_INT32 = 3, PPR_NUM_INT64 = 4,
       PPR_NUM_FLOAT64 = 5, PPR_NUM_TEXT = 6 };
/* per-field conversion status */
enum { PPR_NUM_OK = 0, PPR_NUM_DEFAULTED = 1, PPR_NUM_MISMATCH = 2, PPR_NUM_INEXACT = 3, PPR_NUM_NOT_CONVERTED = 4 };

typedef struct ppr_fields {
    const uint8_t* bytes;
    uint64_t n_bytes;
    const uint32_t* off;
    const uint32_t* len;
    const uint32_t* col;
    const uint32_t* col_first;
    uint64_t n_fields;
    uint32_t n_columns;
} ppr_fields_t;

/* Workspace bytes of ppr_infer_types / ppr_convert (256-byte aligned, no
 * initialisation needed); 0 if n_columns is 0 or above 4096. */
PPR_API size_t ppr_numbers_workspace_bytes(uint32_t n_columns);

/*
 * Blocking. column_type (host, n_columns): each column's type. d_field_type
 * (device, n_fields bytes, may be NULL): each field's type.
 */
PPR_API int ppr_infer_types(const ppr_fields_t* f, uint8_t* d_field_type, uint32_t* column_type, void* d_ws,
                            size_t ws_bytes, void* stream);

/*
 * Blocking. Converts every field to its column's type (column_type: host,
 * n_columns, PPR_NUM_* values, e.g. from ppr_infer_types). d_values (device,
 * n_fields x 8 bytes): int64 for EMPTY and INT columns, the double's bits for
 * FLOAT64 columns, 0 for TEXT columns. d_status (device, n_fields bytes):
 *   PPR_NUM_OK            converted;
 *   PPR_NUM_DEFAULTED     empty field: int_default or float_default;
 *   PPR_NUM_MISMATCH      the field's own type is above the column's: the default;
 *   PPR_NUM_INEXACT       a FLOAT64 column's number outside the exactly converted
 *                         class: NaN. The class: with w the mantissa's digits
 *                         without leading and trailing zeros and |value| =
 *                         w * 10^e, w <= 2^53 and |e| <= 22, or e > 22 and
 *                         w * 10^(e - 22) <= 2^53 (one IEEE operation on exact
 *                         doubles rounds correctly, to nearest even), or w = 0;
 *   PPR_NUM_NOT_CONVERTED a TEXT column (or a column id >= n_columns): 0.
 * counts (host, may be NULL): fields with status 1, 2, 3 and 4.
 */
PPR_API int ppr_convert(const ppr_fields_t* f, const uint32_t* column_type, int64_t int_default, double float_default,
                        uint64_t* d_values, uint8_t* d_status, uint64_t counts[4], void* d_ws, size_t ws_bytes,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PPR_H */
