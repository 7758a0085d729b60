"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values printed in
the pages (tests/golden), closed forms derived from the acceptance/residual
identity, exhaustive enumeration on tiny vocabularies, library routines
(numpy sort / cumsum / searchsorted, scipy softmax) and reductions between
modes.  No GPU is needed.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

from conftest import floats, ints, read_golden

LN = np.log


def batch1(ids, q, logits, T=1.0, k=0, p=1.0, ua=None, us=0.5, dtype="f32"):
    ids = np.asarray(ids, np.int32)[None]
    g = ids.shape[1]
    return dict(draft_ids=ids, draft_probs=None if q is None else np.asarray(q, np.float32)[None],
                target_logits=np.asarray(logits, np.float32 if dtype == "f32" else np.uint16)[None],
                dtype=dtype, temperature=np.array([T], np.float32), top_k=np.array([k], np.int32),
                top_p=np.array([p], np.float32),
                u_accept=np.asarray(ua if ua is not None else np.zeros(g), np.float32)[None],
                u_sample=np.array([us], np.float32))


def run(oracle_mod, b, threads=1):
    return oracle_mod.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                          b["top_k"], b["top_p"], b["u_accept"], b["u_sample"], threads=threads)


# --------------------------------------------------------------------------------------------
# values printed in the pages
# --------------------------------------------------------------------------------------------

def test_worked_example_two_token(oracle_mod):
    g = read_golden("worked_example_two_token.txt")
    q = floats(g["draft_probs"])
    p = floats(g["target_probs"])
    ids = ints(g["draft_ids"])
    logits = LN(np.array(p))
    for us in np.linspace(0, 1, 21, endpoint=False):
        b = batch1(ids, q, logits, ua=[float(g["u_accept"])], us=us)
        r = run(oracle_mod, b)
        assert list(r["tokens"][0]) == ints(g["expect_tokens"])
        assert r["num_accepted"][0] == int(g["expect_num_accepted"])
        alpha = r["p_y"][0, 0] / r["q_y"][0, 0]
        assert alpha == pytest.approx(float(g["expect_alpha"]), abs=1e-6)
        assert r["resid_mass"][0] == pytest.approx(sum(floats(g["expect_residual"])[0]), abs=1e-6)
    # accepted branch (u < alpha): the bonus row (0.3, 0.7) is drawn by inverse CDF
    for us, tok in [(0.1, 0), (0.29, 0), (0.31, 1), (0.9, 1)]:
        r = run(oracle_mod, batch1(ids, q, logits, ua=[0.49], us=us))
        assert list(r["tokens"][0]) == [1, tok] and r["num_accepted"][0] == 1


def test_exercise_three_token(oracle_mod):
    g = read_golden("exercise_three_token.txt")
    q = floats(g["draft_probs"])
    p = floats(g["target_probs"])
    logits = LN(np.array(p))
    alpha = float(g["expect_alpha"])
    res = np.array(floats(g["expect_residual_normalised"])[0])
    b = batch1(ints(g["draft_ids"]), q, logits, ua=[alpha - 1e-3])
    r = run(oracle_mod, b)
    assert r["p_y"][0, 0] / r["q_y"][0, 0] == pytest.approx(alpha, abs=1e-6)
    assert r["num_accepted"][0] == 1
    cdf = np.cumsum(res)
    for us in np.linspace(0, 1, 31, endpoint=False):
        r = run(oracle_mod, batch1(ints(g["draft_ids"]), q, logits, ua=[alpha + 1e-3], us=us))
        assert r["num_accepted"][0] == 0
        assert r["resid_mass"][0] == pytest.approx(sum(floats(g["expect_residual"])[0]), abs=1e-6)
        expect = int(np.searchsorted(cdf, us, side="right"))
        if abs(us - 2 / 3) > 1e-6:
            assert r["tokens"][0, 0] == expect, us


def _greedy_logits(argmax, V, rng):
    rows = []
    for a in argmax:
        l = rng.standard_normal(V).astype(np.float32)
        l[a] = l.max() + 1.0
        rows.append(l)
    return np.array(rows, np.float32)


def test_greedy_example(oracle_mod):
    g = read_golden("greedy_example.txt")
    V = int(g["V"])
    logits = _greedy_logits(ints(g["target_argmax"]), V, np.random.default_rng(0))
    for ua in (0.0, 0.999):
        r = run(oracle_mod, batch1(ints(g["draft_ids"]), None, logits, T=0.0, ua=[ua] * 4))
        assert list(r["tokens"][0]) == ints(g["expect_tokens"])
        assert r["num_accepted"][0] == int(g["expect_num_accepted"])
        # greedy ignores q entirely
        q = np.full((4, V), 1.0 / V, np.float32)
        r2 = run(oracle_mod, batch1(ints(g["draft_ids"]), q, logits, T=0.0, ua=[ua] * 4))
        assert list(r2["tokens"][0]) == ints(g["expect_tokens"])
    r = run(oracle_mod, batch1(ints(g["all_match_draft_ids"]), None, logits, T=0.0))
    assert list(r["tokens"][0]) == ints(g["all_match_expect_tokens"])
    assert r["num_accepted"][0] == int(g["all_match_expect_num_accepted"])


def test_accept_is_strict(oracle_mod):
    # equal logits give p' = (1/2, 1/2) exactly; without draft probabilities q'(y) = 1,
    # so u = 1/2 sits exactly on the acceptance boundary u < p'(y) / q'(y)
    l = np.zeros((2, 2), np.float32)
    r = run(oracle_mod, batch1([1], None, l, ua=[0.5], us=0.0))
    assert r["num_accepted"][0] == 0 and list(r["tokens"][0]) == [0, -1]
    r = run(oracle_mod, batch1([1], None, l, ua=[np.nextafter(np.float32(0.5), np.float32(0))], us=0.0))
    assert r["num_accepted"][0] == 1 and list(r["tokens"][0]) == [1, 0]


def test_greedy_ties_lowest_id(oracle_mod):
    V = 8
    l = np.zeros((2, V), np.float32)
    l[0, [2, 5, 6]] = 3.0
    l[1, [1, 7]] = 2.0
    r = run(oracle_mod, batch1([2], None, l, T=0.0))
    assert list(r["tokens"][0]) == [2, 1]
    r = run(oracle_mod, batch1([5], None, l, T=0.0))
    assert list(r["tokens"][0]) == [2, -1] and r["num_accepted"][0] == 0


def test_exercise_reject_third(oracle_mod):
    g = read_golden("exercise_reject_third.txt")
    gam, rej = int(g["gamma"]), int(g["reject_at"])
    V = 5
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((gam + 1, V)).astype(np.float32)
    q = softmax(rng.standard_normal((gam, V)), axis=1).astype(np.float32)
    ids = [int(np.argmax(q[j])) for j in range(gam)]
    b = batch1(ids, q, logits)
    ratios = run(oracle_mod, b)["p_y"][0] / run(oracle_mod, b)["q_y"][0]
    ua = [0.0] * gam
    ua[rej] = min(0.999, (min(1.0, ratios[rej]) + 1.0) / 2)
    assert ratios[rej] < 0.999, "fixture must allow a rejection at the chosen position"
    r = run(oracle_mod, batch1(ids, q, logits, ua=ua))
    toks = list(r["tokens"][0])
    assert r["num_accepted"][0] == int(g["expect_num_accepted"])
    assert sum(t >= 0 for t in toks) == int(g["expect_committed"])
    assert toks[:rej] == ids[:rej] and toks.count(-1) == int(g["expect_placeholders"])


# --------------------------------------------------------------------------------------------
# transforms against numpy / scipy
# --------------------------------------------------------------------------------------------

def np_filters(order, mass, k, top_p):
    """Sort-based top-k (ties kept) then top-p over whole tie groups."""
    V = order.shape[0]
    keep = np.ones(V, bool)
    if 1 <= k < V:
        kth = np.sort(order)[::-1][k - 1]
        keep = order >= kth
    if top_p < 1.0:
        vals = order[keep]
        ms = mass[keep]
        zk = ms.sum()
        uniq = np.unique(vals)[::-1]
        group_mass = np.array([ms[vals == v].sum() for v in uniq])
        cum = np.cumsum(group_mass)
        t = int(np.argmax(cum >= top_p * zk)) if (cum >= top_p * zk).any() else len(uniq) - 1
        keep = keep & (order >= uniq[t])
    return keep


def np_target(l, T, k, p):
    s = l.astype(np.float64) / T
    e = np.exp(s - s.max())
    keep = np_filters(s, e, k, p)
    w = np.where(keep, e, 0.0)
    return w / w.sum()


def np_draft(q, T, k, p):
    r = q.astype(np.float64) ** (1.0 / T)
    keep = np_filters(r, r, k, p)
    w = np.where(keep, r, 0.0)
    return w / w.sum()


@pytest.mark.parametrize("seed", range(6))
def test_target_transform_matches_numpy(oracle_mod, seed):
    import workloads as W
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 3000))
    l = (rng.standard_normal(V) * 3).astype(np.float32)
    if seed % 2:  # tie-heavy rows: coarse values
        l = np.round(l * 2) / 2
    bits = W.f32_to_bf16_bits(l)
    for T, k, p in [(1.0, 0, 1.0), (0.7, 0, 1.0), (1.3, 10, 1.0), (1.0, 0, 0.8), (0.9, 50, 0.9),
                    (1.0, 1, 1.0), (2.0, V, 0.5), (1.0, V - 1, 0.999)]:
        got, f, _ = oracle_mod.target_probs(l, "f32", T, k, p)
        assert f == 0
        np.testing.assert_allclose(got, np_target(l, T, k, p), rtol=1e-12, atol=1e-15)
        got, f, _ = oracle_mod.target_probs(bits, "bf16", T, k, p)
        np.testing.assert_allclose(got, np_target(W.bf16_bits_to_f32(bits), T, k, p), rtol=1e-12, atol=1e-15)


def test_plain_softmax_when_filters_off(oracle_mod):
    rng = np.random.default_rng(7)
    l = (rng.standard_normal(1000) * 4).astype(np.float32)
    for T in (0.25, 1.0, 3.0):
        for k, p in ((0, 1.0), (1000, 1.0), (-3, 1.5), (5000, 1.0)):
            got, f, _ = oracle_mod.target_probs(l, "f32", T, k, p)
            np.testing.assert_allclose(got, softmax(l.astype(np.float64) / T), rtol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_draft_transform_matches_numpy(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(2, 3000))
    q = softmax(rng.standard_normal(V) * 2).astype(np.float32)
    if seed % 2:
        q = (np.round(q * 2000) / 2000).astype(np.float32)  # ties and exact zeros
        q[0] = max(q[0], 1e-3)
    for T, k, p in [(1.0, 0, 1.0), (0.6, 0, 1.0), (1.2, 7, 1.0), (1.0, 0, 0.85), (0.8, 40, 0.9), (1.0, 1, 1.0)]:
        got, f, _ = oracle_mod.draft_probs(q, T, k, p)
        assert f == 0
        np.testing.assert_allclose(got, np_draft(q, T, k, p), rtol=1e-12, atol=1e-15)


def np_draft_logdomain(q, T, k, p):
    """q' from the logs: exp(log(q) / T - max), the route that stays in range at any T."""
    q64 = q.astype(np.float64)
    with np.errstate(divide="ignore"):
        s = np.log(q64) / T
    e = np.exp(s - s.max())
    keep = np_filters(e, e, k, p)
    w = np.where(keep, e, 0.0)
    return w / w.sum()


@pytest.mark.parametrize("seed", range(4))
def test_draft_transform_low_temperature(oracle_mod, seed):
    # q^(1/T) / sum at T = 0.05 and 0.02 equals the log-domain form, and q' is unchanged when every q is
    # scaled by the same power of two (exact in fp32): the normalisation removes any common factor
    rng = np.random.default_rng(200 + seed)
    V = int(rng.integers(50, 4000))
    q = softmax(rng.standard_normal(V) * 1.5).astype(np.float32)
    for T, k, p in [(0.05, 0, 1.0), (0.05, 0, 0.9), (0.02, 65, 1.0), (0.05, 5, 0.95)]:
        got, f, _ = oracle_mod.draft_probs(q, T, k, p)
        assert f == 0
        np.testing.assert_allclose(got, np_draft_logdomain(q, T, k, p), rtol=1e-9, atol=1e-300)
        scaled, f2, _ = oracle_mod.draft_probs((q * np.float32(2.0 ** -5)).astype(np.float32), T, k, p)
        assert f2 == 0
        np.testing.assert_allclose(scaled, got, rtol=1e-12, atol=1e-300)


def test_top_k_keeps_ties(oracle_mod):
    l = np.array([5, 4, 4, 4, 3, 2, 4, 1], np.float32)
    got, _, _ = oracle_mod.target_probs(l, "f32", 1.0, 2, 1.0)
    kept = got > 0
    assert list(np.nonzero(kept)[0]) == [0, 1, 2, 3, 6]
    e = np.exp(l[kept].astype(np.float64) - 5)
    np.testing.assert_allclose(got[kept], e / e.sum(), rtol=1e-14)


def test_top_p_cut_is_smallest_tie_group_prefix(oracle_mod):
    # probabilities 0.4, 0.2, 0.2, 0.1, 0.1 (as logits): top_p 0.5 needs 0.4 + both 0.2s (tie group)
    p = np.array([0.1, 0.2, 0.4, 0.2, 0.1])
    got, _, m = oracle_mod.target_probs(np.log(p).astype(np.float32), "f32", 1.0, 0, 0.5)
    assert list(np.nonzero(got > 0)[0]) == [1, 2, 3]
    np.testing.assert_allclose(got[[1, 2, 3]], [0.25, 0.5, 0.25], rtol=1e-6)
    got, _, _ = oracle_mod.target_probs(np.log(p).astype(np.float32), "f32", 1.0, 0, 0.4)
    assert list(np.nonzero(got > 0)[0]) == [2]


def test_inverse_cdf_matches_searchsorted(oracle_mod):
    rng = np.random.default_rng(11)
    V = 257
    l = (rng.standard_normal(V) * 2).astype(np.float32)
    pp = softmax(l.astype(np.float64))
    cdf = np.cumsum(pp)
    us = np.sort(rng.integers(0, 1 << 24, 400) * 2.0 ** -24).astype(np.float32)
    b = dict(draft_ids=np.zeros((400, 0), np.int32), draft_probs=None,
             target_logits=np.repeat(l[None, None], 400, axis=0), dtype="f32",
             temperature=np.ones(400, np.float32), top_k=np.zeros(400, np.int32), top_p=np.ones(400, np.float32),
             u_accept=np.zeros((400, 0), np.float32), u_sample=us)
    r = run(oracle_mod, b)
    expect = np.searchsorted(cdf, us.astype(np.float64) * cdf[-1], side="right")
    ok = r["margin"] >= 1e-9
    assert ok.sum() > 390
    np.testing.assert_array_equal(r["tokens"][ok, 0], expect[ok])
    assert (r["num_accepted"] == 0).all() and (r["tokens"][:, 1:] == -1).all() if r["tokens"].shape[1] > 1 else True


# --------------------------------------------------------------------------------------------
# exact output law by enumeration against the closed form
# --------------------------------------------------------------------------------------------

def closed_form_law(P, Q, gam, ids_fixed=None):
    """Law of the committed token sequence.

    With draft probabilities: drafts y_j ~ q'_j independently; the acceptance
    branch contributes min(p', q') per accepted token, the rejection branch
    (p' - q')_+ for the replacement, the bonus row p'_gamma after gamma
    acceptances.  Without them (ids_fixed): accept y_j with probability
    p'_j(y_j), replacement ~ p'_A with y_A removed.
    """
    law = {}
    V = P.shape[1]
    if ids_fixed is None:
        def rec(prefix, prob):
            a = len(prefix)
            if a == gam:
                for z in range(V):
                    if P[gam, z] > 0:
                        key = tuple(prefix) + (z,)
                        law[key] = law.get(key, 0) + prob * P[gam, z]
                return
            mn = np.minimum(P[a], Q[a])
            for x in range(V):
                if mn[x] > 0:
                    rec(prefix + [x], prob * mn[x])
            res = np.maximum(P[a] - Q[a], 0)
            for z in range(V):
                if res[z] > 0:
                    key = tuple(prefix) + (z,)
                    law[key] = law.get(key, 0) + prob * res[z]
        rec([], 1.0)
    else:
        prob = 1.0
        for a in range(gam + 1):
            if prob == 0:
                break
            if a == gam:
                for z in range(V):
                    if P[gam, z] > 0:
                        key = tuple(ids_fixed[:a]) + (z,)
                        law[key] = law.get(key, 0) + prob * P[gam, z]
                break
            y = ids_fixed[a]
            for z in range(V):
                if z != y and P[a, z] > 0:
                    key = tuple(ids_fixed[:a]) + (z,)
                    law[key] = law.get(key, 0) + prob * P[a, z]
            prob *= P[a, y]
    return law


def law_cells(logits, q, T, k, p, gam, V, ids_fixed=None):
    """One request per cell of (y, u_accept, u_sample) space, placed at the
    cell's midpoint: returns the batch, the cells (ids, ua, us, measure,
    expected A) and the transformed rows P and Qd.  Cells are cut at the
    acceptance ratios and at the residual CDF boundaries, both computed here
    with numpy from the transformed rows."""
    P = np.array([np_target(logits[j], T, k, p) for j in range(gam + 1)])
    Qd = None if q is None else np.array([np_draft(q[j], T, k, p) for j in range(gam)])
    cases = []  # (ids, ua, us, measure, expected_A)
    ys = itertools.product(range(V), repeat=gam) if ids_fixed is None else [tuple(ids_fixed)]
    for y in ys:
        py = 1.0
        if ids_fixed is None:
            for j in range(gam):
                py *= Qd[j, y[j]]
        if py == 0:
            continue
        acc_prob = []
        for j in range(gam):
            qy = Qd[j, y[j]] if Qd is not None else 1.0
            acc_prob.append(1.0 if qy == 0 and P[j, y[j]] > 0 else (0.0 if qy == 0 else min(1.0, P[j, y[j]] / qy)))
        prefix = 1.0
        for a in range(gam + 1):
            if a < gam:
                rej = 1.0 - acc_prob[a]
                m_a = prefix * rej
            else:
                m_a = prefix
            if m_a > 0:
                ua = [acc_prob[j] / 2 for j in range(gam)]
                if a < gam:
                    ua[a] = (acc_prob[a] + 1.0) / 2
                if a < gam:
                    qa = Qd[a] if Qd is not None else np.eye(V)[y[a]]
                    w = np.maximum(P[a] - qa, 0)
                    if w.sum() == 0:
                        w = P[a].copy()
                else:
                    w = P[gam].copy()
                c = np.concatenate([[0.0], np.cumsum(w) / w.sum()])
                for z in range(V):
                    width = c[z + 1] - c[z]
                    if width > 1e-12:
                        cases.append((y, ua, (c[z] + c[z + 1]) / 2, py * m_a * width, a))
            if a < gam:
                prefix *= acc_prob[a]
                if prefix == 0:
                    break
    n = len(cases)
    b = dict(draft_ids=np.array([c[0] for c in cases], np.int32).reshape(n, gam),
             draft_probs=None if q is None else np.repeat(np.asarray(q, np.float32)[None], n, axis=0),
             target_logits=np.repeat(np.asarray(logits, np.float32)[None], n, axis=0), dtype="f32",
             temperature=np.full(n, T, np.float32), top_k=np.full(n, k, np.int32),
             top_p=np.full(n, p, np.float32), u_accept=np.array([c[1] for c in cases], np.float32).reshape(n, gam),
             u_sample=np.array([c[2] for c in cases], np.float32))
    return b, cases, P, Qd


def enumerate_law(oracle_mod, logits, q, T, k, p, gam, V, ids_fixed=None):
    """Run the oracle at the midpoint of every cell (law_cells) and add up the
    cell measures by output."""
    b, cases, P, Qd = law_cells(logits, q, T, k, p, gam, V, ids_fixed)
    n = len(cases)
    r = run(oracle_mod, b)
    law = {}
    for t in range(n):
        assert r["num_accepted"][t] == cases[t][4]
        toks = tuple(int(x) for x in r["tokens"][t] if x >= 0)
        law[toks] = law.get(toks, 0) + cases[t][3]
    return law, P, Qd


LAW_CASES = [
    # V, gamma, T, top_k, top_p, null_q, seed
    (2, 1, 1.0, 0, 1.0, False, 0),
    (3, 2, 1.0, 0, 1.0, False, 1),
    (4, 2, 0.7, 0, 1.0, False, 2),
    (4, 2, 1.0, 2, 1.0, False, 3),
    (4, 2, 1.0, 0, 0.7, False, 4),
    (4, 1, 1.3, 3, 0.8, False, 5),
    (3, 2, 1.0, 0, 1.0, True, 6),
    (4, 2, 0.8, 0, 0.9, True, 7),
    (4, 0, 1.0, 0, 1.0, False, 8),
]


@pytest.mark.parametrize("V,gam,T,k,p,null_q,seed", LAW_CASES)
def test_enumerated_law_equals_closed_form(oracle_mod, V, gam, T, k, p, null_q, seed):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((gam + 1, V)) * 1.5).astype(np.float32)
    q = None if null_q else softmax(rng.standard_normal((gam, V)) * 1.5, axis=1).astype(np.float32)
    ids_fixed = [int(x) for x in rng.integers(0, V, gam)] if null_q else None
    got, P, Qd = enumerate_law(oracle_mod, logits, q, T, k, p, gam, V, ids_fixed)
    want = closed_form_law(P, Qd, gam, ids_fixed)
    assert set(got) == set(want)
    for key in want:
        assert got[key] == pytest.approx(want[key], abs=1e-9), key
    assert sum(got.values()) == pytest.approx(1.0, abs=1e-9)
    if not null_q:
        # marginal of the first committed token is p'_0 (the acceptance/residual identity)
        first = np.zeros(V)
        for key, v in got.items():
            first[key[0]] += v
        np.testing.assert_allclose(first, P[0], atol=1e-9)


# --------------------------------------------------------------------------------------------
# reductions between modes
# --------------------------------------------------------------------------------------------

def _rand_batch(rng, N, gam, V, null_q=False):
    logits = (rng.standard_normal((N, gam + 1, V)) * 2).astype(np.float32)
    q = softmax(rng.standard_normal((N, gam, V)) * 2, axis=2).astype(np.float32)
    ids = rng.integers(0, V, (N, gam)).astype(np.int32)
    return dict(draft_ids=ids, draft_probs=None if null_q else q, target_logits=logits, dtype="f32",
                temperature=np.ones(N, np.float32), top_k=np.zeros(N, np.int32), top_p=np.ones(N, np.float32),
                u_accept=rng.random((N, gam)).astype(np.float32), u_sample=rng.random(N).astype(np.float32))


def test_top_k_one_is_greedy(oracle_mod):
    rng = np.random.default_rng(21)
    b = _rand_batch(rng, 200, 3, 16)
    am = b["target_logits"].argmax(axis=2)
    b["draft_ids"][:100] = am[:100, :3]          # many matches
    b["draft_ids"][100:150, 1:] = am[100:150, 1:3]
    g = dict(b, temperature=np.zeros(200, np.float32))
    s = dict(b, top_k=np.ones(200, np.int32), temperature=rng.uniform(0.3, 2, 200).astype(np.float32))
    rg, rs = run(oracle_mod, g), run(oracle_mod, s)
    np.testing.assert_array_equal(rg["tokens"], rs["tokens"])
    np.testing.assert_array_equal(rg["num_accepted"], rs["num_accepted"])
    assert (rg["num_accepted"] == 3).sum() >= 100


def test_one_hot_q_equals_null_q(oracle_mod):
    rng = np.random.default_rng(22)
    b = _rand_batch(rng, 300, 3, 12)
    onehot = np.zeros_like(b["draft_probs"])
    for i in range(300):
        for j in range(3):
            onehot[i, j, b["draft_ids"][i, j]] = 1.0
    for T, k, p in ((1.0, 0, 1.0), (0.7, 5, 0.9), (1.4, 0, 0.8)):
        bb = dict(b, temperature=np.full(300, T, np.float32), top_k=np.full(300, k, np.int32),
                  top_p=np.full(300, p, np.float32))
        r1 = run(oracle_mod, dict(bb, draft_probs=onehot))
        r2 = run(oracle_mod, dict(bb, draft_probs=None))
        np.testing.assert_array_equal(r1["tokens"], r2["tokens"])
        np.testing.assert_array_equal(r1["num_accepted"], r2["num_accepted"])


def test_q_equal_p_accepts_everything(oracle_mod):
    rng = np.random.default_rng(23)
    b = _rand_batch(rng, 300, 4, 50)
    b["draft_probs"] = softmax(b["target_logits"][:, :4].astype(np.float64), axis=2).astype(np.float32)
    r = run(oracle_mod, b)
    amb = r["margin"] < 1e-6
    assert (r["num_accepted"][~amb] == 4).all()
    assert amb.sum() <= 3


# --------------------------------------------------------------------------------------------
# padding, faults
# --------------------------------------------------------------------------------------------

def test_padding_rows_are_not_read(oracle_mod):
    rng = np.random.default_rng(31)
    b = _rand_batch(rng, 50, 4, 20)
    gam = rng.integers(0, 5, 50)
    ref = run(oracle_mod, b)  # reference before poisoning (uses full gamma)
    for i in range(50):
        b["draft_ids"][i, gam[i]:] = -1
        b["target_logits"][i, gam[i] + 1:] = np.nan
        b["draft_probs"][i, gam[i]:] = np.nan
    r = run(oracle_mod, b)
    assert (r["fault"] == 0).all()
    for i in range(50):
        assert r["num_accepted"][i] <= gam[i]
        assert (r["tokens"][i, r["num_accepted"][i] + 1:] == -1).all()
    del ref


def test_fault_reporting(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(32)
    base = _rand_batch(rng, 1, 2, 8)

    def fault_of(**mod):
        b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
        for k, f in mod.items():
            f(b)
        r = run(oracle_mod, b)
        if r["fault"][0]:
            assert r["num_accepted"][0] == -1 and (r["tokens"][0] == -1).all()
        return int(r["fault"][0])

    assert fault_of() == 0
    assert fault_of(a=lambda b: b["draft_ids"].__setitem__((0, 1), 8)) == O.FAULT_DRAFT_ID
    assert fault_of(a=lambda b: b["draft_ids"].__setitem__((0, 0), -1),
                    c=lambda b: b["draft_ids"].__setitem__((0, 1), 99)) == 0  # after padding: ignored
    for T in (-1.0, np.nan, np.inf, 1e-40):
        assert fault_of(a=lambda b, T=T: b["temperature"].__setitem__(0, T)) == O.FAULT_TEMPERATURE
    for p in (0.0, -0.5, np.nan):
        assert fault_of(a=lambda b, p=p: b["top_p"].__setitem__(0, p)) == O.FAULT_TOP_P
    assert fault_of(a=lambda b: b["top_p"].__setitem__(0, 0.0), t=lambda b: b["temperature"].__setitem__(0, 0.0)) == 0
    for v in (np.nan, np.inf):
        assert fault_of(a=lambda b, v=v: b["target_logits"].__setitem__((0, 2, 3), v)) == O.FAULT_TARGET_ROW
    assert fault_of(a=lambda b: b["target_logits"].__setitem__((0, 1), -np.inf)) == O.FAULT_TARGET_ROW
    assert fault_of(a=lambda b: b["target_logits"].__setitem__((0, 1, 0), -np.inf)) == 0
    for v in (np.nan, np.inf, -1e-3, -0.0):
        assert fault_of(a=lambda b, v=v: b["draft_probs"].__setitem__((0, 1, 5), v)) == O.FAULT_DRAFT_ROW
    assert fault_of(a=lambda b: b["draft_probs"].__setitem__((0, 0), 0.0)) == O.FAULT_DRAFT_MASS
    # greedy: q rows are never read
    assert fault_of(a=lambda b: b["draft_probs"].__setitem__((0, 1, 5), np.nan),
                    t=lambda b: b["temperature"].__setitem__(0, 0.0)) == 0
    assert fault_of(a=lambda b: b["target_logits"].__setitem__((0, 2, 3), np.nan),
                    t=lambda b: b["temperature"].__setitem__(0, 0.0)) == O.FAULT_TARGET_ROW


def test_empty_and_zero_gamma(oracle_mod):
    rng = np.random.default_rng(33)
    b = _rand_batch(rng, 0, 3, 10)
    r = run(oracle_mod, b)
    assert r["tokens"].shape == (0, 4)
    b = _rand_batch(rng, 5, 0, 10)
    r = run(oracle_mod, b)
    assert (r["num_accepted"] == 0).all() and (r["tokens"][:, 0] >= 0).all()


def test_threads_do_not_change_results(oracle_mod):
    rng = np.random.default_rng(34)
    b = _rand_batch(rng, 97, 3, 64)
    b["top_k"][:] = 10
    b["top_p"][:] = 0.8
    r1, r4 = run(oracle_mod, b, threads=1), run(oracle_mod, b, threads=4)
    for k in ("tokens", "num_accepted", "fault"):
        np.testing.assert_array_equal(r1[k], r4[k])
