"""GPU parity with blocking calls from several host threads at once.

A blocking call reads the workspace header back into a pinned buffer that
belongs to the calling host thread. Two threads here each enqueue parses on
their own stream with their own workspace and read the results back, several
times over, while the other thread does the same. The foreign calls release
the interpreter lock, so the read-backs really overlap. Every result must equal
the oracle's.
"""
import threading

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def test_blocking_calls_from_two_threads():
    import torch
    assert torch.cuda.is_available()
    import dfa_parsing_delimiter_amd as ppr
    t5 = W.table("T5")
    inputs = [W.generate(3, n=24 << 20), W.generate(2, n=8 << 20)]  # quote-heavy, numeric
    refs = [oracle.csv_parse(x, t5) for x in inputs]
    devs = [torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in inputs]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()  # default priority
            x, r = inputs[i], refs[i]
            P = ppr.Parser(t5, max_n=x.size, capacity=r["n_fields"])
            for rep in range(6):
                with torch.cuda.stream(s):
                    for a in P.out_arrays:
                        a.fill_(-1)
                P.launch(devs[i], s)
                o = P.results(x.size, s)
                assert int(o.n_fields) == r["n_fields"], (i, rep, int(o.n_fields), r["n_fields"])
                assert int(o.n_records) == r["n_records"], (i, rep)
                assert int(o.error_pos) == r["error_pos"], (i, rep)
                k = r["n_fields"]
                for a, key in zip(P.out_arrays, ("rec", "col", "off", "len")):
                    got = a[:k].cpu().numpy().view(np.uint32)
                    assert np.array_equal(got, r[key]), (i, rep, key)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
