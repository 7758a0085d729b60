"""Pins of the oracle's repetition penalties (no GPU).

zwjcode.cn page, section 06: p and q go through identical transforms at each
position, repetition penalties among them (the vLLM page's sampler applies
"penalty" logits processors to the target logits as well).  Each row j of a
request carries its own list: the context tokens position j continues, with
their counts in the generated output.  A listed token's logit l becomes
l / theta if l > 0, else l * theta, minus (frequency * count + presence) when
count > 0; its draft probability is multiplied by exp(-(frequency * count +
presence)), the same shift on the probability scale.  The tests pin the value
rule by hand-computed numbers, the direction of each term by monotonicity, the
draft-side rule by the closed form on the draft's own logits, the plumbing by
the method's law, and the faults."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as W
from test_oracle_pins import closed_form_law, enumerate_law, run as pins_run


def _run(b, pen):
    return oracle.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                      b["top_k"], b["top_p"], b["u_accept"], b["u_sample"], penalties=pen)


def _gammas(b):
    ids = b["draft_ids"]
    return np.where((ids < 0).any(axis=1), np.argmax(ids < 0, axis=1), ids.shape[1])


def _empty_lists(b):
    return [[(np.zeros(0, np.int64), np.zeros(0, np.int64)) for _ in range(g + 1)] for g in _gammas(b)]


# ------------------------------------------------------------------------------------------
# the value rule, by hand
# ------------------------------------------------------------------------------------------

def test_deltas_by_hand():
    d = oracle.penalty_deltas([0, 1, 3, 0], presence=0.5, frequency=0.25)
    np.testing.assert_array_equal(d, np.array([0.0, 0.75, 1.25, 0.0], np.float32))
    # a prompt-only token (count 0) gets no presence or frequency term
    assert oracle.penalty_deltas([0], presence=9.0, frequency=9.0)[0] == 0.0


def test_f32_logits_by_hand():
    l = np.array([2.0, -2.0, 0.0, -np.inf, 3e38], np.float32)
    d = np.array([0.5, 0.5, 0.0, 1.0, 0.0], np.float32)
    out = oracle.penalize_logits(l, "f32", 2.0, d)
    # 2 / 2 - 0.5; -2 * 2 - 0.5; 0 is not positive: 0 * 2; -inf stays -inf
    np.testing.assert_array_equal(out[:4], np.array([0.5, -4.5, 0.0, -np.inf], np.float32))
    # theta below 1 can push a large logit past the float32 range
    assert np.isposinf(oracle.penalize_logits(l[4:], "f32", 0.5, d[4:])[0])
    assert np.isnan(oracle.penalize_logits(np.array([np.nan], np.float32), "f32", 2.0, d[:1])[0])


def test_bf16_logits_by_hand():
    # 1.5 (bf16 0x3FC0) / 3 = 0.5; 0.5 - fl32(0.1) = fl32(0.4) = 0x3ECCCCCD, whose
    # low half 0xCCCD is above the halfway point 0x8000: rounds up to 0x3ECD
    # (0.400390625)
    out = oracle.penalize_logits(np.array([0x3FC0], np.uint16), "bf16", 3.0, np.array([0.1], np.float32))
    assert out[0] == 0x3ECD
    # -1.0 (0xBF80) * 1.25 = -1.25 (0xBFA0), exact; minus 0 stays
    assert oracle.penalize_logits(np.array([0xBF80], np.uint16), "bf16", 1.25, np.zeros(1, np.float32))[0] == 0xBFA0
    # a tie: 1 + 2^-8 (0x3F808000 in float32) is halfway between bf16 0x3F80 and
    # 0x3F81 and rounds to the even 0x3F80; 1 + 3 * 2^-8 rounds up to the even 0x3F82
    one = np.array([0x3F80], np.uint16)
    assert oracle.penalize_logits(one, "bf16", 1.0, np.array([-2.0 ** -8], np.float32))[0] == 0x3F80
    assert oracle.penalize_logits(one, "bf16", 1.0, np.array([-3 * 2.0 ** -8], np.float32))[0] == 0x3F82


# ------------------------------------------------------------------------------------------
# through the sampler
# ------------------------------------------------------------------------------------------

def test_each_term_lowers_the_listed_token():
    # theta > 1 shrinks a positive logit and stretches a negative one: both
    # lower the token's probability; presence and frequency lower it further
    l = np.array([[2.0, -1.0, 0.5, 0.0, 1.0, -2.0, 0.3, 0.1]] * 2, np.float32)
    p0 = softmax(l[0].astype(np.float64))

    def prob(tok, theta, pres, freq, cnt):
        # p'(tok) of row 0, read as p'(y) of a draft-free request drafting tok
        b = dict(draft_ids=np.array([[tok]], np.int32), draft_probs=None, target_logits=l[None], dtype="f32",
                 temperature=np.ones(1, np.float32), top_k=np.zeros(1, np.int32), top_p=np.ones(1, np.float32),
                 u_accept=np.zeros((1, 1), np.float32), u_sample=np.zeros(1, np.float32))
        none = (np.zeros(0, np.int64), np.zeros(0, np.int64))
        pen = dict(lists=[[(np.array([tok]), np.array([cnt])), none]], repetition=np.array([theta], np.float32),
                   presence=np.array([pres], np.float32), frequency=np.array([freq], np.float32))
        return _run(b, pen)["p_y"][0, 0]

    for tok in (0, 1):  # a positive and a negative logit
        assert prob(tok, 1.0, 0.0, 0.0, 0) == pytest.approx(p0[tok], rel=1e-12)
        p1 = prob(tok, 1.8, 0.0, 0.0, 0)
        p2 = prob(tok, 1.8, 0.7, 0.0, 1)
        p3 = prob(tok, 1.8, 0.7, 0.4, 3)
        assert p1 < 0.9 * p0[tok] and p2 < 0.9 * p1 and p3 < 0.9 * p2
        # theta < 1 raises the token instead
        assert prob(tok, 0.6, 0.0, 0.0, 0) > 1.1 * p0[tok]


def test_target_probabilities_follow_the_penalised_logits():
    rng = np.random.default_rng(3)
    b = W.generate(W.config(1, N=20, gmax=3, V=40))
    b["draft_probs"] = None  # draft-free requests: theta may differ from 1
    gam = _gammas(b)
    lists = []
    for i in range(20):
        rows = []
        for _ in range(gam[i] + 1):
            ids = np.sort(rng.choice(40, size=8, replace=False))
            rows.append((ids, rng.integers(0, 4, size=8)))
        lists.append(rows)
    theta = rng.uniform(0.7, 1.6, 20).astype(np.float32)
    pres = rng.uniform(-0.5, 1.0, 20).astype(np.float32)
    freq = rng.uniform(0.0, 0.6, 20).astype(np.float32)
    r = _run(b, dict(lists=lists, repetition=theta, presence=pres, frequency=freq))
    assert (r["fault"] == 0).all()
    for i in range(20):
        for j in range(gam[i]):
            if np.isnan(r["p_y"][i, j]):
                continue
            l = b["target_logits"][i, j].astype(np.float64)
            ids, cnt = lists[i][j]
            for x, c in zip(ids, cnt):
                l[x] = l[x] / theta[i] if l[x] > 0 else l[x] * theta[i]
                if c > 0:
                    l[x] -= float(freq[i]) * c + float(pres[i])
            p = softmax(l)
            assert r["p_y"][i, j] == pytest.approx(p[b["draft_ids"][i, j]], rel=2e-6, abs=1e-12)


def test_draft_probabilities_follow_the_drafts_penalised_logits():
    # q = softmax(lq): presence and frequency on q give softmax(lq - delta)
    rng = np.random.default_rng(4)
    V, G = 30, 3
    lq = rng.standard_normal((1, G, V)) * 1.5
    q = softmax(lq, axis=2).astype(np.float32)
    lt = (rng.standard_normal((1, G + 1, V)) * 1.5).astype(np.float32)
    ids = np.array([[3, 7, 11]], np.int32)
    b = dict(draft_ids=ids, draft_probs=q, target_logits=lt, dtype="f32", temperature=np.ones(1, np.float32),
             top_k=np.zeros(1, np.int32), top_p=np.ones(1, np.float32),
             u_accept=np.zeros((1, G), np.float32), u_sample=np.zeros(1, np.float32))
    lists = [[(np.array([3, 7, 20]), np.array([2, 1, 0])),      # row 0 penalises its own draft token 3
              (np.array([3, 7]), np.array([3, 1])),
              (np.array([3, 7, 11]), np.array([3, 2, 5])),
              (np.array([3]), np.array([1]))]]
    pen = dict(lists=lists, presence=np.array([0.4], np.float32), frequency=np.array([0.3], np.float32))
    r = _run(b, pen)
    for j in range(G):
        if np.isnan(r["q_y"][0, j]):
            continue
        d = np.zeros(V)
        for x, c in zip(*lists[0][j]):
            d[x] = 0.3 * c + 0.4 if c > 0 else 0.0
        want = softmax(np.log(q[0, j].astype(np.float64)) - d)[ids[0, j]]
        assert r["q_y"][0, j] == pytest.approx(want, rel=1e-6)
    assert not np.isnan(r["q_y"][0, 0])


def test_a_uniform_presence_shift_changes_no_probability():
    # softmax is shift-invariant: the same delta on every token of a row
    # changes nothing beyond float32 rounding of the shifted logits
    b = W.generate(W.config(2, N=12, V=64))
    b["target_logits"] = W.bf16_bits_to_f32(b["target_logits"]).astype(np.float32)
    b["dtype"] = "f32"
    gam = _gammas(b)
    lists = [[(np.arange(64), np.ones(64, np.int64)) for _ in range(g + 1)] for g in gam]
    r0 = _run(b, None)
    r1 = _run(b, dict(lists=lists, presence=np.full(12, 0.75, np.float32)))
    ok = ~np.isnan(r0["p_y"])
    np.testing.assert_allclose(r1["p_y"][ok], r0["p_y"][ok], rtol=1e-5)
    np.testing.assert_allclose(r1["q_y"][ok], r0["q_y"][ok], rtol=1e-5)


def test_each_row_uses_its_own_list():
    # a token that only the bonus row's list pushes down never comes out of the
    # bonus draw, while the draft rows are untouched
    b = W.generate(W.config(1, N=40, gmax=2, V=12))
    gam = _gammas(b)
    lists = _empty_lists(b)
    for i in range(40):
        lists[i][gam[i]] = (np.array([5]), np.array([1]))
    r0 = _run(b, None)
    r1 = _run(b, dict(lists=lists, presence=np.full(40, 1e4, np.float32)))
    np.testing.assert_array_equal(r0["p_y"], r1["p_y"])
    np.testing.assert_array_equal(r0["num_accepted"], r1["num_accepted"])
    for i in range(40):
        A = r1["num_accepted"][i]
        if A == gam[i]:
            assert r1["tokens"][i, A] != 5


@pytest.mark.parametrize("seed", [0, 1])
def test_enumerated_law_with_penalties(seed):
    # the sampler stays exact for the penalised rows: its law equals the closed
    # form on the penalised distributions, and the wrapper gives the same
    # outputs as a run on inputs penalised beforehand
    import oracle as oracle_mod
    rng = np.random.default_rng(40 + seed)
    V, gam = 4, 2
    logits = (rng.standard_normal((gam + 1, V)) * 1.5).astype(np.float32)
    q = softmax(rng.standard_normal((gam, V)) * 1.5, axis=1).astype(np.float32)
    lists = [(np.array([0, 2]), np.array([1, 0])), (np.array([1]), np.array([2])), (np.array([3]), np.array([1]))]
    pres, freq = np.float32(0.6), np.float32(0.35)
    lm, qm = logits.copy(), q.copy().astype(np.float64)
    for j, (ids, cnt) in enumerate(lists):
        d = oracle.penalty_deltas(cnt, pres, freq)
        lm[j, ids] = oracle.penalize_logits(lm[j, ids], "f32", 1.0, d)
        if j < gam:
            qm[j, ids] *= np.exp(-d.astype(np.float64))
    qm = qm.astype(np.float32)
    qn = (qm / qm.sum(axis=1, keepdims=True)).astype(np.float32)
    got, P, Qd = enumerate_law(oracle_mod, lm, qn, 1.0, 0, 1.0, gam, V)
    want = closed_form_law(P, Qd, gam, None)
    assert set(got) == set(want)
    for key in want:
        assert got[key] == pytest.approx(want[key], abs=1e-9)
    for ua, us in ((0.3, 0.6), (0.9, 0.1), (0.05, 0.95)):
        b = dict(draft_ids=np.array([[1, 3]], np.int32), draft_probs=q[None], target_logits=logits[None],
                 dtype="f32", temperature=np.ones(1, np.float32), top_k=np.zeros(1, np.int32),
                 top_p=np.ones(1, np.float32), u_accept=np.full((1, gam), ua, np.float32),
                 u_sample=np.full(1, us, np.float32))
        r1 = _run(b, dict(lists=[lists], presence=np.array([pres]), frequency=np.array([freq])))
        r2 = pins_run(oracle_mod, dict(b, target_logits=lm[None], draft_probs=qm[None]))
        np.testing.assert_array_equal(r1["tokens"], r2["tokens"])
        np.testing.assert_allclose(r1["p_y"], r2["p_y"], rtol=1e-12)


# ------------------------------------------------------------------------------------------
# faults
# ------------------------------------------------------------------------------------------

def test_faults():
    b = W.generate(W.config(1, N=9, gmax=2, V=16))
    b["draft_ids"][:, :] = np.abs(b["draft_ids"])  # every request has gamma = 2
    b["temperature"][8] = -1.0
    ok = (np.array([1, 4]), np.array([0, 2]))
    lists = [[ok, ok, ok] for _ in range(9)]
    lists[1][2] = (np.array([4, 1]), np.array([0, 0]))       # not ascending
    lists[2][0] = (np.array([16]), np.array([1]))            # outside [0, V)
    lists[3][1] = (np.array([2, 3]), np.array([1, -1]))      # negative count
    lists[4][0] = (np.arange(oracle.PEN_MAX + 1) % 16, np.zeros(oracle.PEN_MAX + 1, np.int64))  # too long
    theta = np.ones(9, np.float32)
    pres = np.zeros(9, np.float32)
    theta[5] = 1.5                # theta != 1 with draft rows at a nonzero temperature
    theta[6] = 0.0                # not positive
    pres[7] = np.inf              # not finite
    theta[8] = 2.0                # with a temperature fault as well
    r = _run(b, dict(lists=lists, repetition=theta, presence=pres))
    assert r["fault"][0] == 0
    for i in range(1, 8):
        assert r["fault"][i] == oracle.FAULT_PENALTY, i
    assert r["fault"][8] == oracle.FAULT_PENALTY | oracle.FAULT_TEMPERATURE
    assert (r["num_accepted"][1:] == -1).all() and (r["tokens"][1:] == -1).all()
    # theta != 1 is fine for a greedy request and for a draft-free one
    b["temperature"][:] = 1.0
    b["temperature"][5] = 0.0
    r = _run(b, dict(lists=[[ok, ok, ok] for _ in range(9)], repetition=np.where(np.arange(9) == 5, 1.5, 1.0)))
    assert (r["fault"] == 0).all()
    b["draft_probs"] = None
    r = _run(b, dict(lists=[[ok, ok, ok] for _ in range(9)], repetition=np.full(9, 1.5, np.float32)))
    assert (r["fault"] == 0).all()
