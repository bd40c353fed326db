"""Seeded field texts for numeric type inference and conversion: integers of
every width and at their bounds, integers beyond int64, decimals and
exponents inside and outside the exactly converted class, zero-padded and
long digit strings (longer than the 32 bytes a thread reads alone), text with
a long numeric prefix, plain text and empty fields. No delimiter, quote or
newline occurs in them, so a CSV row of them parses into exactly these
fields."""
from __future__ import annotations

import numpy as np

_BOUNDS = [-(1 << 63), -(1 << 31) - 1, -(1 << 31), -32769, -32768, -129, -128, -1, 0, 1, 127, 128, 32767, 32768,
           (1 << 31) - 1, 1 << 31, (1 << 63) - 1, 1 << 63]


def numeric_text(r: np.random.Generator) -> bytes:
    k = int(r.integers(0, 14))
    sign = r.choice(["", "-", "+"], p=[0.6, 0.3, 0.1])
    digits = lambda n: "".join(r.choice(list("0123456789"), int(n)))  # noqa: E731
    if k == 0:
        return b""
    if k == 1:
        return str(int(r.choice(_BOUNDS)) + int(r.integers(-1, 2))).encode()
    if k == 2:
        return (sign + str(int(r.integers(0, 1 << 62)) >> int(r.integers(0, 62)))).encode()
    if k == 3:
        return (sign + digits(r.integers(19, 26))).encode()  # around and beyond int64
    if k == 4:
        return (sign + digits(r.integers(1, 8)) + "." + digits(r.integers(0, 8))).encode()
    if k == 5:
        return (sign + "." + digits(r.integers(1, 12))).encode()
    if k == 6:
        return (sign + digits(r.integers(1, 17)) + r.choice(["e", "E"]) + r.choice(["", "-", "+"]) +
                str(int(r.integers(0, 40)))).encode()
    if k == 7:  # many significant digits: outside the exact class
        return (sign + digits(r.integers(15, 30)) + "." + digits(r.integers(0, 10))).encode()
    if k == 8:  # zero-padded: a long numeric text with a small value
        return (sign + "0" * int(r.integers(20, 120)) + digits(r.integers(1, 6)) +
                ("." + digits(r.integers(0, 6)) if r.random() < 0.5 else "")).encode()
    if k == 9:  # a long numeric prefix, then text
        return (digits(r.integers(30, 90)) + r.choice(["x", "e", ".", "-", "e+", ".5."])).encode()
    if k == 10:  # trailing zeros and large exponents
        return (digits(r.integers(1, 4)) + "0" * int(r.integers(0, 20)) + "e" + str(int(r.integers(-40, 400)))).encode()
    if k == 11:
        odd = [b"abc", b"1.2.3", b"--1", b"1e", b".", b"+", b"e5", b"1x", b"inf", b"nan", b"0x1F", b"1_000", b"1.e5",
               b"-.5", b"5.", b"0e0", b"-0", b"-0.0", b"00"]
        return odd[int(r.integers(0, len(odd)))]
    if k == 12:  # long plain text
        return r.choice(np.frombuffer(b"abcdefghij ", np.uint8), int(r.integers(1, 200))).tobytes()
    return digits(r.integers(1, 10)).encode()


def numeric_csv(seed: int, n_rows: int, n_cols: int) -> bytes:
    """rows of n_cols fields from numeric_text, some columns all-integer or all-empty for variety"""
    r = np.random.default_rng(seed)
    rows = []
    for _ in range(n_rows):
        f = []
        for c in range(n_cols):
            if c == 0:
                f.append(str(int(r.integers(-100, 100))).encode())  # an INT8 column
            elif c == 1:
                f.append(b"" if r.random() < 0.9 else str(int(r.integers(0, 1 << 40))).encode())
            elif c == 2:
                f.append(b"")  # an EMPTY column
            else:
                f.append(numeric_text(r))
        rows.append(b",".join(f))
    return b"\n".join(rows) + b"\n"
