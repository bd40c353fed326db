"""DFA tables for the delimiter-separated workloads (pure data, no parsing code).

ParPaRaw (Sec. 3, parsing context, Fig. 3) drives parsing with a DFA whose
states are the parsing contexts and which includes an invalid state (INV) for
malformed input, e.g. a quote read inside an unquoted field. The printed figure
and its transition table (Table 1) did not survive extraction, so the two tables
below are this project's own. Each cell is (next state, tag); the tag is the
Mealy output of reading that symbol in that state:

  VALUE   the byte belongs to a field's raw span (quotes included),
  FIELD   the byte ends a field (field delimiter),
  RECORD  the byte ends a field and its record (record delimiter),
  INVALID the byte makes the input malformed.

Both tables are inputs to the parser: the oracle and the GPU path read them as
data and never special-case them.
"""

VALUE, FIELD, RECORD, INVALID = 0, 1, 2, 3
TAG_NAMES = ("VALUE", "FIELD", "RECORD", "INVALID")


def _class_map(specials, n_other):
    cm = bytearray([n_other] * 256)
    for byte, cls in specials.items():
        cm[byte] = cls
    return bytes(cm)


def _table(name, states, classes, rows, start, invalid, accepting, class_map):
    S, C = len(states), len(classes)
    nxt = [[0] * C for _ in range(S)]
    tag = [[0] * C for _ in range(S)]
    for s, row in enumerate(rows):
        assert len(row) == C
        for c, (ns, t) in enumerate(row):
            nxt[s][c] = states.index(ns)
            tag[s][c] = t
    return {
        "name": name,
        "n_states": S,
        "n_classes": C,
        "state_names": tuple(states),
        "class_names": tuple(classes),
        "next": nxt,
        "tag": tag,
        "start": states.index(start),
        "invalid": states.index(invalid),
        "accept_mask": sum(1 << states.index(a) for a in accepting),
        "class_map": class_map,
    }


def csv_t5(fdelim=b",", rdelim=b"\n", quote=b'"'):
    """Five-state RFC 4180 style table: EOR (at a field start), FLD (inside an
    unquoted field), ENC (inside quotes), ESC (a quote read inside quotes: either
    the closing quote or the first half of a doubled quote), INV (absorbing).
    Classes: field delimiter, record delimiter, quote, every other byte."""
    V, F, R, I = VALUE, FIELD, RECORD, INVALID
    states = ("EOR", "FLD", "ENC", "ESC", "INV")
    classes = ("FDELIM", "RDELIM", "QUOTE", "OTHER")
    rows = [
        # FDELIM        RDELIM          QUOTE           OTHER
        [("EOR", F), ("EOR", R), ("ENC", V), ("FLD", V)],  # EOR
        [("EOR", F), ("EOR", R), ("INV", I), ("FLD", V)],  # FLD
        [("ENC", V), ("ENC", V), ("ESC", V), ("ENC", V)],  # ENC
        [("EOR", F), ("EOR", R), ("ENC", V), ("INV", I)],  # ESC
        [("INV", I), ("INV", I), ("INV", I), ("INV", I)],  # INV
    ]
    cm = _class_map({fdelim[0]: 0, rdelim[0]: 1, quote[0]: 2}, 3)
    return _table("T5", states, classes, rows, "EOR", "INV", ("EOR", "FLD", "ESC"), cm)


def tsv_t6(fdelim=b"\t", rdelim=b"\n", quote=b'"', comment=b"#"):
    """Six-state tab-separated table with comment lines: a record whose first
    byte is the comment byte runs, uninterpreted, to the next record delimiter
    (state CMT). EOR is the record start, FLD is after a field delimiter or
    inside an unquoted field (a quote there opens an enclosure), ENC/ESC/INV as
    in the five-state table. Classes: TAB, newline, quote, '#', every other byte."""
    V, F, R, I = VALUE, FIELD, RECORD, INVALID
    states = ("EOR", "FLD", "ENC", "ESC", "INV", "CMT")
    classes = ("FDELIM", "RDELIM", "QUOTE", "COMMENT", "OTHER")
    rows = [
        # FDELIM        RDELIM          QUOTE           COMMENT         OTHER
        [("FLD", F), ("EOR", R), ("ENC", V), ("CMT", V), ("FLD", V)],  # EOR
        [("FLD", F), ("EOR", R), ("ENC", V), ("FLD", V), ("FLD", V)],  # FLD
        [("ENC", V), ("ENC", V), ("ESC", V), ("ENC", V), ("ENC", V)],  # ENC
        [("FLD", F), ("EOR", R), ("ENC", V), ("INV", I), ("INV", I)],  # ESC
        [("INV", I), ("INV", I), ("INV", I), ("INV", I), ("INV", I)],  # INV
        [("CMT", V), ("EOR", R), ("CMT", V), ("CMT", V), ("CMT", V)],  # CMT
    ]
    cm = _class_map({fdelim[0]: 0, rdelim[0]: 1, quote[0]: 2, comment[0]: 3}, 4)
    return _table("T6", states, classes, rows, "EOR", "INV", ("EOR", "FLD", "ESC", "CMT"), cm)


TABLES = {"T5": csv_t5, "T6": tsv_t6}
