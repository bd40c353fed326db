"""Columnar partition of parsed fields (test infrastructure; part of the oracle).

ParPaRaw, Sec. 3 (partitioning and the CSS index, Fig. 5): the symbols are
partitioned by the column they belong to with a stable sort on their column
tags, so that each column's symbols lie together in input order: the column's
concatenated symbol string (CSS). An index into each CSS gives every field's
record, offset and number of symbols (run-length encoding of the record tags,
then an exclusive sum). The specialisations passage (Fig. 6) gives two
variants that replace the record tags: an inline-terminated CSS, where each
field is followed by a terminator byte (ASCII 0x1E or 0x1F), and a
vector-delimited CSS, where an auxiliary boolean vector marks the field ends.

Readings (the pages leave these open):
* A field's symbols are its raw span as the parse reports it (field_offsets /
  field_lengths: quotes included; unquoting belongs to type conversion).
* Each field keeps its place even when empty: the index has one entry per
  field. In both variants a field takes its length plus one slot: the
  inline-terminated CSS writes the terminator there; the vector-delimited CSS
  writes 0 there and sets aux = 1 at that slot (aux = 0 elsewhere), so empty
  fields and terminator bytes inside fields stay unambiguous.
* Columns run from 0 to the largest column id; a column no record reaches is
  an empty CSS.

The plain definition, written out: a stable sort of the field indices by
column (numpy's stable argsort, the one library step), then each field's
bytes copied in that order with a running offset.
"""
from __future__ import annotations

import numpy as np

MODE_INDEXED, MODE_INLINE, MODE_VECTOR = 0, 1, 2


def partition(data, rec, col, off, length, mode: int = MODE_INDEXED, terminator: int = 0x1F) -> dict:
    """Per-column CSS and its index from one parse's per-field arrays.

    Returns order (field index of each partitioned entry), col_first_field /
    col_first_byte (C + 1 bounds of each column's entries and bytes), rec /
    css_off / length per entry, css (uint8), aux (uint8, vector mode only)."""
    b = np.frombuffer(bytes(data), dtype=np.uint8) if not isinstance(data, np.ndarray) else data
    col = np.asarray(col, dtype=np.int64)
    nf = col.size
    n_cols = int(col.max()) + 1 if nf else 0
    order = np.argsort(col, kind="stable")
    slot = 0 if mode == MODE_INDEXED else 1
    lens = np.asarray(length, dtype=np.int64)[order]
    offs = np.asarray(off, dtype=np.int64)[order]
    css_off = np.zeros(nf, dtype=np.int64)
    pos = 0
    css = bytearray()
    aux = bytearray()
    for j in range(nf):
        css_off[j] = pos
        css += b[offs[j]:offs[j] + lens[j]].tobytes()
        aux += bytes(int(lens[j]))
        if slot:
            css.append(terminator if mode == MODE_INLINE else 0)
            aux.append(1)
        pos += int(lens[j]) + slot
    counts = np.bincount(col, minlength=n_cols) if nf else np.zeros(0, np.int64)
    col_first_field = np.zeros(n_cols + 1, dtype=np.int64)
    np.cumsum(counts, out=col_first_field[1:])
    col_first_byte = np.array([css_off[f] if f < nf else pos for f in col_first_field], dtype=np.int64)
    out = dict(order=order, n_columns=n_cols, col_first_field=col_first_field, col_first_byte=col_first_byte,
               rec=np.asarray(rec, dtype=np.int64)[order], css_off=css_off, length=lens,
               css=np.frombuffer(bytes(css), dtype=np.uint8), css_bytes=pos)
    if mode == MODE_VECTOR:
        out["aux"] = np.frombuffer(bytes(aux), dtype=np.uint8)
    return out
