"""Pins of the numbers oracle (oracle/numbers.py) against things other than
itself: hand-worked type tables at every width boundary, Python's fractions
module (exact rational values of decimal texts), the exact class checked by
doing the one IEEE operation it promises, and hand-worked conversions.

ParPaRaw, "Type inference" and "Default values for empty strings"
(capabilities section); Sec. 3 (conversion to the column's type).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import numbers as N

HAND_TYPES = [
    (b"", N.EMPTY), (b"0", N.INT8), (b"-0", N.INT8), (b"+7", N.INT8), (b"127", N.INT8), (b"128", N.INT16),
    (b"-128", N.INT8), (b"-129", N.INT16), (b"32767", N.INT16), (b"32768", N.INT32), (b"-32768", N.INT16),
    (b"2147483647", N.INT32), (b"2147483648", N.INT64), (b"-2147483648", N.INT32), (b"-2147483649", N.INT64),
    (b"9223372036854775807", N.INT64), (b"9223372036854775808", N.FLOAT64), (b"-9223372036854775808", N.INT64),
    (b"-9223372036854775809", N.FLOAT64), (b"000000000000000000000000000127", N.INT8),
    (b"1.", N.FLOAT64), (b".5", N.FLOAT64), (b"1.5", N.FLOAT64), (b"1e5", N.FLOAT64), (b"1E+05", N.FLOAT64),
    (b"-.5e-3", N.FLOAT64), (b"0.0", N.FLOAT64),
    (b"+", N.TEXT), (b"-", N.TEXT), (b".", N.TEXT), (b"e5", N.TEXT), (b"1e", N.TEXT), (b"1e+", N.TEXT),
    (b"1.e5", N.FLOAT64), (b".e5", N.TEXT), (b"+-1", N.TEXT), (b"1-", N.TEXT), (b"0x10", N.TEXT), (b"inf", N.TEXT),
    (b"nan", N.TEXT), (b" 1", N.TEXT), (b"1 ", N.TEXT), (b'"1"', N.TEXT), (b"1_000", N.TEXT), (b"1.2.3", N.TEXT),
    (b"1e5.0", N.TEXT), ("١".encode(), N.TEXT), (b"abc", N.TEXT),
]


@pytest.mark.parametrize("text,want", HAND_TYPES)
def test_hand_worked_types(text, want):
    assert N.field_type(text) == want, (text, N.TYPE_NAMES[N.field_type(text)], N.TYPE_NAMES[want])


def test_width_boundaries():
    """every signed width's two ends and one step beyond them"""
    for t, bits in ((N.INT8, 8), (N.INT16, 16), (N.INT32, 32), (N.INT64, 64)):
        lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        assert N.field_type(str(lo).encode()) <= t and N.field_type(str(hi).encode()) <= t
        assert N.field_type(str(lo - 1).encode()) == t + 1 and N.field_type(str(hi + 1).encode()) == t + 1


def _random_numeric(rng, n):
    out = []
    for _ in range(n):
        ip = "".join(rng.choice(list("0123456789"), int(rng.integers(0, 25))))
        fp = "".join(rng.choice(list("0123456789"), int(rng.integers(0, 25))))
        if not ip and not fp:
            ip = "0"
        s = rng.choice(["", "+", "-"]) + ip
        if fp or rng.random() < 0.2:
            s += "." + fp
        if rng.random() < 0.5:
            s += rng.choice(["e", "E"]) + rng.choice(["", "+", "-"]) + str(int(rng.integers(0, 40)))
        if rng.random() < 0.3:  # short mantissas with zeros: exact-class candidates near the exponent bounds
            s = rng.choice(["", "-"]) + str(int(rng.integers(1, 10 ** int(rng.integers(1, 17))))) + \
                "0" * int(rng.integers(0, 6)) + "e" + str(int(rng.integers(-30, 31)))
        out.append(s.encode())
    return out


def test_decompose_against_fractions():
    """|value| = w * 10^e10 exactly (fractions parses the decimal text on its own), w without trailing zeros"""
    rng = np.random.default_rng(1)
    for s in _random_numeric(rng, 4000):
        assert N.field_type(s) in (N.INT8, N.INT16, N.INT32, N.INT64, N.FLOAT64), s
        neg, w, e10 = N.decompose(s)
        v = Fraction(s.decode())
        assert abs(v) == w * Fraction(10) ** e10, s
        assert w == 0 or w % 10 != 0, s
        if w:
            assert (v < 0) == neg, s


def test_exact_class_one_rounding():
    """in the exact class, one IEEE multiplication or division of exact doubles gives the correctly rounded
    value (float of the exact fraction); just outside it (e10 = +-23 with 10^23 inexact) it does not always"""
    rng = np.random.default_rng(2)
    n_exact = 0
    sweep = [("%de%d" % (w, e)).encode() for e in range(-26, 27) for w in range(1, 400)]
    for s in _random_numeric(rng, 6000) + sweep:
        neg, w, e10 = N.decompose(s)
        want = float(Fraction(s.decode()))
        if want == 0.0 and s.startswith(b"-"):
            want = -0.0  # (a fraction has no signed zero; the text's sign decides)
        if not N.exact_class(s):
            continue
        n_exact += 1
        if w == 0:
            got = 0.0
        elif -22 <= e10 <= 22:
            got = float(w) * float(10 ** e10) if e10 >= 0 else float(w) / float(10 ** -e10)
        else:
            got = float(w * 10 ** (e10 - 22)) * 1e22
        got = -got if neg else got
        assert np.float64(got).view(np.int64) == np.float64(want).view(np.int64), s
    assert n_exact > 1000
    # 10^23 is not a double: w * 10^23 by one multiplication with float(10**23) misses for some w
    misses = sum(float(w) * float(10 ** 23) != float(Fraction(w) * 10 ** 23) for w in range(1, 3000))
    assert misses > 0


def test_infer_reduction():
    data = b"12|-300|1.5|x||70000|"
    texts = [b"12", b"-300", b"1.5", b"x", b"", b"70000", b""]
    off, pos = [], 0
    for t in texts:
        off.append(pos)
        pos += len(t) + 1
    data = b"|".join(texts)
    cols = [0, 0, 1, 2, 3, 4, 5]
    ft, ct = N.infer(data, off, [len(t) for t in texts], cols, 7)
    assert list(ft) == [N.INT8, N.INT16, N.FLOAT64, N.TEXT, N.EMPTY, N.INT32, N.EMPTY]
    assert list(ct) == [N.INT16, N.FLOAT64, N.TEXT, N.EMPTY, N.INT32, N.EMPTY, N.EMPTY]


def test_convert_hand_worked():
    texts = [b"12", b"", b"1.5", b"-7", b"x", b"0.1", b"", b"12345678901234567890", b"1e400", b"-0.0", b"3"]
    cols = [0, 0, 0, 1, 1, 1, 1, 1, 1, 1, 2]
    off, pos = [], 0
    for t in texts:
        off.append(pos)
        pos += len(t) + 1
    data = b",".join(texts)
    types = np.array([N.INT16, N.FLOAT64, N.TEXT], dtype=np.uint8)
    v, st = N.convert(data, off, [len(t) for t in texts], cols, types, int_default=-1, float_default=2.5)
    f = v.view(np.float64)
    assert (v[0], st[0]) == (12, N.ST_OK)
    assert (v[1], st[1]) == (-1, N.ST_EMPTY)
    assert (v[2], st[2]) == (-1, N.ST_MISMATCH)  # a FLOAT64 field in an INT16 column
    assert (f[3], st[3]) == (-7.0, N.ST_OK)
    assert (f[4], st[4]) == (2.5, N.ST_MISMATCH)  # TEXT in a FLOAT64 column
    assert (f[5], st[5]) == (0.1, N.ST_OK)
    assert (f[6], st[6]) == (2.5, N.ST_EMPTY)
    assert np.isnan(f[7]) and st[7] == N.ST_INEXACT  # w > 2^53
    assert np.isnan(f[8]) and st[8] == N.ST_INEXACT  # e10 = 400
    assert st[9] == N.ST_OK and f[9] == 0.0 and np.signbit(f[9])
    assert (v[10], st[10]) == (0, N.ST_TEXT)
