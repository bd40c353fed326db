"""Numeric type inference and conversion of fields (test infrastructure; part
of the oracle).

ParPaRaw, "Type inference" (capabilities section): threads find the minimal
numerical type each field's value needs, and a reduction over those types
gives the column's type (numerical types only). ParPaRaw, Sec. 3 (after the
partition, a field's symbol string is converted to its column's type, e.g.
int or float) and "Default values for empty strings" (an empty field takes the
column's default value).

Readings (the pages leave these open):
* A field's text is its raw span as the parse reports it (quotes included):
  nothing is trimmed or unquoted, so a quoted number is TEXT.
* Types, ordered: EMPTY (no symbols) < INT8 < INT16 < INT32 < INT64 < FLOAT64
  < TEXT. INT: an optional sign and one or more decimal digits; its type is the
  smallest signed two's-complement width that holds the value, and a value
  beyond int64 is FLOAT64. FLOAT64: an optional sign, then digits with a
  decimal point (at least one digit on either side of it) or digits alone,
  then an optional exponent (e or E, an optional sign, one or more digits),
  with a point or an exponent present. Anything else is TEXT (spaces, inf,
  nan, hexadecimal, digit separators). A column's type is the largest of its
  fields' types; EMPTY if it has no field or only empty ones.
* Conversion to a column's type. A field whose own type is EMPTY takes the
  default value (status EMPTY); one whose type is above the column's takes the
  default value (status MISMATCH). INT8..INT64 and EMPTY columns: the value as
  int64. FLOAT64 columns: the nearest double (ties to even), computed only in
  Clinger's exact class; outside it the value is NaN (status INEXACT). TEXT
  columns: value 0 (status TEXT).
* The exact class. Let D be the mantissa's digits (integer and fraction parts)
  without leading and trailing zeros, w = int(D) (0 without digits) and e10 the
  power of ten with |value| = w * 10^e10. Exact iff w == 0, or w <= 2^53 and
  -22 <= e10 <= 22, or w <= 2^53, e10 > 22 and w * 10^(e10 - 22) <= 2^53. In
  it, w and 10^|e10| (or w * 10^(e10 - 22) and 10^22) are exact doubles, and
  one IEEE multiplication or division of them rounds correctly.

The plain definitions, written out: regular expressions for the grammar,
Python's int() and float() (both exact / correctly rounded) for the values,
a maximum over each column for the reduction.
"""
from __future__ import annotations

import re

import numpy as np

EMPTY, INT8, INT16, INT32, INT64, FLOAT64, TEXT = range(7)
TYPE_NAMES = ("EMPTY", "INT8", "INT16", "INT32", "INT64", "FLOAT64", "TEXT")
ST_OK, ST_EMPTY, ST_MISMATCH, ST_INEXACT, ST_TEXT = range(5)

_INT = re.compile(rb"[+-]?[0-9]+")
_FLOAT = re.compile(rb"[+-]?([0-9]+\.[0-9]*|\.[0-9]+|[0-9]+)([eE][+-]?[0-9]+)?")
_WIDTHS = ((INT8, 8), (INT16, 16), (INT32, 32), (INT64, 64))


def field_type(s: bytes) -> int:
    """the minimal type of one field's text"""
    if len(s) == 0:
        return EMPTY
    if _INT.fullmatch(s):
        v = int(s)
        for t, bits in _WIDTHS:
            if -(1 << (bits - 1)) <= v < (1 << (bits - 1)):
                return t
        return FLOAT64
    if _FLOAT.fullmatch(s):
        return FLOAT64
    return TEXT


def decompose(s: bytes):
    """(negative, w, e10) of a numeric text: |value| = w * 10^e10, w without trailing zeros"""
    m = re.fullmatch(rb"([+-]?)([0-9]*)\.?([0-9]*)(?:[eE]([+-]?[0-9]+))?", s)
    sign, ip, fp, ex = m.group(1), m.group(2), m.group(3), m.group(4)
    digits = (ip + fp).lstrip(b"0")
    stripped = digits.rstrip(b"0")
    e10 = (int(ex) if ex else 0) - len(fp) + (len(digits) - len(stripped))
    return sign == b"-", int(stripped) if stripped else 0, e10


def exact_class(s: bytes) -> bool:
    _, w, e10 = decompose(s)
    if w == 0:
        return True
    if w > 1 << 53:
        return False
    if -22 <= e10 <= 22:
        return True
    return e10 > 22 and w * 10 ** (e10 - 22) <= 1 << 53


def _texts(data, off, length):
    b = bytes(data) if not isinstance(data, np.ndarray) else data.tobytes()
    return [b[int(o):int(o) + int(n)] for o, n in zip(off, length)]


def infer(data, off, length, col, n_columns: int):
    """(type of every field, type of every column)"""
    texts = _texts(data, off, length)
    ft = np.array([field_type(s) for s in texts], dtype=np.uint8)
    ct = np.zeros(n_columns, dtype=np.uint8)
    for c, t in zip(np.asarray(col, dtype=np.int64), ft):
        ct[c] = max(ct[c], t)
    return ft, ct


def convert(data, off, length, col, column_types, int_default: int = 0, float_default: float = 0.0):
    """(values as int64 bit patterns, status) of every field in its column's type"""
    texts = _texts(data, off, length)
    values = np.zeros(len(texts), dtype=np.int64)
    status = np.zeros(len(texts), dtype=np.uint8)
    for j, (s, c) in enumerate(zip(texts, np.asarray(col, dtype=np.int64))):
        ct, t = int(column_types[c]), field_type(s)
        as_float = ct == FLOAT64
        if ct == TEXT:
            values[j], status[j] = 0, ST_TEXT
        elif t == EMPTY:
            values[j] = np.float64(float_default).view(np.int64) if as_float else int_default
            status[j] = ST_EMPTY
        elif t > ct:
            values[j] = np.float64(float_default).view(np.int64) if as_float else int_default
            status[j] = ST_MISMATCH
        elif not as_float:
            values[j] = int(s)
        elif exact_class(s):
            values[j] = np.float64(float(s)).view(np.int64)
        else:
            values[j], status[j] = np.float64(np.nan).view(np.int64), ST_INEXACT
    return values, status
