/*
 * CPU oracle: delimiter-separated parsing by one sequential DFA run.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header or table with the GPU path.
 *
 * What it computes is the plain definition that ParPaRaw's data-parallel
 * method reaches: "ParPaRaw: Massively Parallel Parsing of Delimiter-Separated
 * Raw Data", Sec. 3 (a sequential approach sets the DFA's start state and reads
 * the input from beginning to end, always knowing the current state; the
 * tagging step marks record delimiters and field delimiters; the offsets step
 * gives every symbol its record and column) and the "validating format"
 * capability (an invalid transition or a non-accepting end state is reported).
 *
 * Per byte i, with c = class_map[byte], the table gives the tag of reading c in
 * state s and the next state. A FIELD or RECORD tag ends the current field,
 * whose raw span runs from the byte after the previous terminator (or 0) up to
 * i; FIELD moves to the next column, RECORD to the next record and column 0.
 * After the last byte, if the input is non-empty and its last byte was not a
 * record delimiter, the unterminated final field (and its record) is emitted.
 * error_pos is the first byte tagged INVALID, else n if the end state is not
 * accepting, else -1.
 */
#include <stdint.h>

enum { TAG_VALUE = 0, TAG_FIELD = 1, TAG_RECORD = 2, TAG_INVALID = 3 };

/* next/tag: row-major [n_states][n_classes] */
int oracle_csv_parse(const uint8_t* bytes, uint64_t n, uint32_t n_states, uint32_t n_classes,
                     uint32_t start_state, uint32_t accept_mask, const uint8_t* next, const uint8_t* tag,
                     const uint8_t* class_map, uint32_t* rec_out, uint32_t* col_out, uint32_t* off_out,
                     uint32_t* len_out, uint64_t cap, uint64_t* n_fields, uint64_t* n_records, int64_t* error_pos,
                     uint32_t* end_state)
{
    (void)n_states;
    uint32_t s = start_state;
    uint64_t field_start = 0, rec = 0, col = 0, nf = 0;
    int64_t err = -1;
    uint32_t last_tag = TAG_VALUE;
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t c = class_map[bytes[i]];
        uint32_t t = tag[s * n_classes + c];
        uint32_t s_next = next[s * n_classes + c];
        if (t == TAG_INVALID && err < 0) err = (int64_t)i;
        if (t == TAG_FIELD || t == TAG_RECORD) {
            if (nf < cap) {
                rec_out[nf] = (uint32_t)rec;
                col_out[nf] = (uint32_t)col;
                off_out[nf] = (uint32_t)field_start;
                len_out[nf] = (uint32_t)(i - field_start);
            }
            nf++;
            field_start = i + 1;
            if (t == TAG_FIELD) {
                col++;
            } else {
                rec++;
                col = 0;
            }
        }
        last_tag = t;
        s = s_next;
    }
    if (n > 0 && last_tag != TAG_RECORD) {
        if (nf < cap) {
            rec_out[nf] = (uint32_t)rec;
            col_out[nf] = (uint32_t)col;
            off_out[nf] = (uint32_t)field_start;
            len_out[nf] = (uint32_t)(n - field_start);
        }
        nf++;
        rec++;
    }
    if (err < 0 && !((accept_mask >> s) & 1u)) err = (int64_t)n;
    *n_fields = nf;
    *n_records = rec;
    *error_pos = err;
    *end_state = s;
    return nf > cap ? -2 : 0;
}

/*
 * Convenience for exhaustive tests: parses `count` independent inputs stored
 * back to back (input j is bytes[starts[j] .. starts[j+1])), each from the start
 * state, by calling oracle_csv_parse once per input. Field arrays are written
 * back to back; field_base[j] is where input j's fields begin.
 */
int oracle_csv_parse_many(const uint8_t* bytes, const uint64_t* starts, uint64_t count, uint32_t n_states,
                          uint32_t n_classes, uint32_t start_state, uint32_t accept_mask, const uint8_t* next,
                          const uint8_t* tag, const uint8_t* class_map, uint32_t* rec_out, uint32_t* col_out,
                          uint32_t* off_out, uint32_t* len_out, uint64_t cap, uint64_t* field_base,
                          uint64_t* n_records, int64_t* error_pos, uint32_t* end_state)
{
    uint64_t base = 0;
    for (uint64_t j = 0; j < count; ++j) {
        uint64_t nf = 0;
        field_base[j] = base;
        int rc = oracle_csv_parse(bytes + starts[j], starts[j + 1] - starts[j], n_states, n_classes, start_state,
                                  accept_mask, next, tag, class_map, rec_out + base, col_out + base,
                                  off_out + base, len_out + base, cap - base, &nf, &n_records[j], &error_pos[j],
                                  &end_state[j]);
        if (rc != 0) return rc;
        base += nf;
    }
    field_base[count] = base;
    return 0;
}
