"""The seeded input generators: published PRNG values, determinism, shapes."""
import numpy as np
import pytest

import workloads as W


def test_splitmix64_known_value():
    # splitmix64 seeded with 0: the widely reproduced first output (e.g. the first
    # nextLong() of java.util.SplittableRandom(0), which uses the same mixer)
    out = np.zeros(1, dtype=np.uint64)
    W.lib().wl_splitmix64_stream(0, out.ctypes.data, 1)
    assert int(out[0]) == 0xE220A8397B1DCDAF


def test_xoshiro_matches_definition_on_small_state():
    """xoshiro256** step written out with Python integers (published algorithm)"""
    M = (1 << 64) - 1

    def rotl(x, k):
        return ((x << k) | (x >> (64 - k))) & M

    s = [1, 2, 3, 4]
    want = []
    for _ in range(8):
        want.append((rotl((s[1] * 5) & M, 7) * 9) & M)
        t = (s[1] << 17) & M
        s[2] ^= s[0]
        s[3] ^= s[1]
        s[1] ^= s[2]
        s[0] ^= s[3]
        s[2] ^= t
        s[3] = rotl(s[3], 45)
    st = np.array([1, 2, 3, 4], dtype=np.uint64)
    out = np.zeros(8, dtype=np.uint64)
    W.lib().wl_xoshiro_stream(st.ctypes.data, out.ctypes.data, 8)
    assert [int(x) for x in out] == want
    # the first output from state (1,2,3,4) is rotl(2*5, 7)*9 = 11520
    assert want[0] == 11520


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_deterministic_and_exact_size(cfg):
    n = 1 << 16
    a = W.generate(cfg, n=n)
    b = W.generate(cfg, n=n)
    c = W.generate(cfg, n=n, seed=W.seed_of(cfg) + 1000)
    assert a.size == n and a.dtype == np.uint8
    assert W.sha256(a) == W.sha256(b)
    assert W.sha256(a) != W.sha256(c)


def test_configs_shape():
    assert [W.CONFIGS[i]["n"] for i in (1, 2, 3, 4, 5)] == [1 << 20, 256 << 20, 1 << 30, 1 << 30, 512 << 20]
    assert W.CONFIGS[3]["chunk_bytes"] == 31
    b, truth = W.generate(3, n=1 << 20, truth=True)
    # geometric lengths with mean 40 plus quotes: about 42-46 bytes per field
    assert 38 < (1 << 20) / truth["n_fields"] < 50
    assert np.all(truth["col"] < 12)
    b, truth = W.generate(4, n=1 << 20, truth=True)
    assert np.max(truth["col"]) == 511


def test_token_pair_table_is_consistent():
    te = W.token_entries()
    assert te["n"] == 40 + 2
    assert te["pair"].shape == (42, 42)
    d = W.lexer_dfa()
    assert d["n_states"] <= 64
    # whitespace never follows whitespace directly
    ws = [i for i in range(te["n"]) if te["entries"][i].kind == te["pad_kind"]]
    for a in ws:
        for b in ws:
            assert te["pair"][a, b] == 255
