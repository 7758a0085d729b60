"""Pins of the oracle's banned tokens (no GPU).

zwjcode.cn page, section 06: p and q go through identical transforms, banned
tokens among them.  A banned token has logit -inf in every target row of its
request and probability 0 in every draft row, so p' and q' are renormalised over
the allowed tokens; the tests below check that against numpy and against the
method's closed-form law, and check the faults of malformed lists."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from test_oracle_pins import closed_form_law, enumerate_law, run as pins_run


def _csr(lists):
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    ids = np.concatenate([np.asarray(x, np.int32) for x in lists] + [np.zeros(0, np.int32)])
    return off, ids


def _run(b, banned):
    return oracle.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                      b["top_k"], b["top_p"], b["u_accept"], b["u_sample"], banned=banned)


def _lists(rng, N, V, n):
    return [np.sort(rng.choice(V, size=n, replace=False)) for _ in range(N)]


def test_renormalised_over_allowed_tokens():
    rng = np.random.default_rng(1)
    b = W.generate(W.config(1, N=30, gmax=3, V=40))
    lists = _lists(rng, 30, 40, 6)
    r = _run(b, _csr(lists))
    l = b["target_logits"].astype(np.float64)
    q = b["draft_probs"].astype(np.float64)
    for i in range(30):
        allowed = np.ones(40, bool)
        allowed[lists[i]] = False
        for j in range(3):
            y = b["draft_ids"][i, j]
            if np.isnan(r["p_y"][i, j]):
                continue  # after the first rejection
            p = np.where(allowed, np.exp(l[i, j] - l[i, j][allowed].max()), 0.0)
            qq = np.where(allowed, q[i, j], 0.0)
            assert r["p_y"][i, j] == pytest.approx(p[y] / p.sum(), rel=1e-12, abs=1e-15)
            assert r["q_y"][i, j] == pytest.approx(qq[y] / qq.sum(), rel=1e-12, abs=1e-15)


def test_banned_tokens_are_never_committed():
    rng = np.random.default_rng(2)
    for cfg in (W.config(1, N=200, gmax=4, V=30), W.config(4, N=200, gmax=4, V=30, greedy_count=50),
                W.config(3, N=200, gmax=4, V=30, top_k=8, top_p=0.9, draft_top_k=0)):
        b = W.generate(cfg)
        lists = _lists(rng, 200, 30, 10)
        # every other request bans its first draft token
        for i in range(0, 200, 2):
            lists[i] = np.unique(np.concatenate([lists[i], b["draft_ids"][i, :1]]))
        r = _run(b, _csr(lists))
        for i in range(200):
            A = r["num_accepted"][i]
            toks = r["tokens"][i, : A + 1]
            assert not np.isin(toks, lists[i]).any()
            if i % 2 == 0:
                assert A == 0


def test_banning_outside_both_top_k_sets_changes_nothing():
    b = W.generate(W.config(3, N=40, gmax=3, V=60, top_k=5, top_p=1.0))
    lists = []
    for i in range(40):
        p_low = np.argsort(W.bf16_bits_to_f32(b["target_logits"][i]), axis=1)[:, :20]
        q_low = np.argsort(b["draft_probs"][i], axis=1)[:, :20]
        common = set(p_low[0])
        for row in list(p_low[1:]) + list(q_low):
            common &= set(row)
        lists.append(np.array(sorted(common), np.int32))
    assert sum(len(x) for x in lists) > 0
    r0, r1 = _run(b, None), _run(b, _csr(lists))
    np.testing.assert_array_equal(r0["tokens"], r1["tokens"])
    np.testing.assert_array_equal(r0["num_accepted"], r1["num_accepted"])


def test_malformed_lists_fault():
    b = W.generate(W.config(1, N=5, gmax=2, V=16))
    b["temperature"][4] = -1.0  # a parameter fault as well
    lists = [[3, 1], [16], [-1, 2], list(range(16)), [5, 5]]
    off, ids = _csr([np.array(x) for x in lists])
    r = _run(b, (off, ids))
    bad = np.array([True, True, True, False, True])
    assert (r["fault"][bad] & oracle.FAULT_BAN_LIST).all()
    assert r["fault"][4] == oracle.FAULT_BAN_LIST | oracle.FAULT_TEMPERATURE
    # a valid list that bans every token leaves no finite logit: a target-row fault
    assert r["fault"][3] == oracle.FAULT_TARGET_ROW
    assert (r["num_accepted"] == -1).all() and (r["tokens"] == -1).all()
    long_list = np.arange(oracle.BAN_MAX + 1) % 16  # too long (and not ascending)
    r = _run(W.generate(W.config(1, N=1, gmax=2, V=16)), (np.array([0, len(long_list)]), long_list))
    assert r["fault"][0] == oracle.FAULT_BAN_LIST


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_enumerated_law_with_bans(seed):
    # the law on a tiny vocabulary with one token banned equals the closed form
    # on the renormalised allowed distributions (the token gets zero mass)
    import oracle as oracle_mod
    rng = np.random.default_rng(30 + seed)
    V, gam = 4, 2
    logits = (rng.standard_normal((gam + 1, V)) * 1.5).astype(np.float32)
    q = softmax(rng.standard_normal((gam, V)) * 1.5, axis=1).astype(np.float32)
    ban = int(rng.integers(V))
    lm, qm = logits.copy(), q.copy()
    lm[:, ban] = -np.inf
    qm[:, ban] = 0.0
    qm = (qm / qm.sum(axis=1, keepdims=True)).astype(np.float32)
    got, P, Qd = enumerate_law(oracle_mod, lm, qm, 1.0, 0, 1.0, gam, V)
    want = closed_form_law(P, Qd, gam, None)
    assert set(got) == set(want)
    for key in want:
        assert ban not in key
        assert got[key] == pytest.approx(want[key], abs=1e-9)
    # and the wrapper's masking gives the same outputs as the masked inputs
    b = dict(draft_ids=np.array([[x for x in range(V) if x != ban][:gam]], np.int32), draft_probs=q[None],
             target_logits=logits[None], dtype="f32", temperature=np.ones(1, np.float32),
             top_k=np.zeros(1, np.int32), top_p=np.ones(1, np.float32),
             u_accept=np.full((1, gam), 0.3, np.float32), u_sample=np.full(1, 0.6, np.float32))
    r1 = _run(b, (np.array([0, 1]), np.array([ban])))
    r2 = pins_run(oracle_mod, dict(b, target_logits=lm[None], draft_probs=q.copy()[None] * (np.arange(V) != ban)))
    np.testing.assert_array_equal(r1["tokens"], r2["tokens"])
