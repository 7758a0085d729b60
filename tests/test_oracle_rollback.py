"""Pins of the oracle's KV rollback bookkeeping (no GPU): the worked example
of the KV page, and properties any correct rollback has."""
import numpy as np

from conftest import read_golden

import oracle


def test_rollback_worked_example():
    g = read_golden("kv_rollback_example.txt")
    K, A, bs = int(g["drafts"]), int(g["accepted"]), int(g["block_size"])
    nct, _, _ = oracle.rollback([A], [K], num_computed_tokens=[int(g["num_computed_before"])])
    assert K - A == int(g["expect_rejected"])
    assert nct[0] == int(g["expect_num_computed_after"])
    assert divmod(nct[0], bs) == (int(g["expect_block"]), int(g["expect_offset"]))


def test_rollback_properties():
    rng = np.random.default_rng(5)
    n = 400
    gam = rng.integers(0, 9, n)
    A = np.array([rng.integers(-1, g + 1) for g in gam])
    nct = rng.integers(-3, 3000, n)
    nop = rng.integers(0, 9, n)
    slots = [list(rng.integers(0, 10 ** 6, g)) for g in gam]
    c, p, s = oracle.rollback(A, gam, nct, nop, slots)
    for i in range(n):
        if A[i] < 0:  # faulted verify: untouched
            assert (c[i], p[i], s[i]) == (nct[i], nop[i], slots[i])
            continue
        r = gam[i] - A[i]
        assert c[i] == (nct[i] - r if nct[i] > 0 else nct[i])
        assert p[i] == (nop[i] - r if nop[i] > 0 else nop[i])
        assert s[i][: A[i]] == slots[i][: A[i]]          # accepted drafts keep their slots
        assert all(x == -1 for x in s[i][A[i]:])          # rejected ones are padding
    # everything accepted changes nothing; nothing accepted takes back every draft
    c, p, s = oracle.rollback(gam, gam, nct, nop, slots)
    assert list(c) == list(nct) and list(p) == list(nop) and s == slots
    c, _, s = oracle.rollback(np.zeros(n, int), gam, np.full(n, 100), None, slots)
    assert list(c) == list(100 - gam) and all(all(x == -1 for x in r) for r in s)
