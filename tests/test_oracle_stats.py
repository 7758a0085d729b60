"""Frequency pins of the oracle over 10**6 rounds.

- The first committed token of a round is distributed as the transformed target
  row p'_0, whatever the draft distribution: acceptance contributes min(p', q'),
  the residual (p' - q')_+, and their sum is p' (zwjcode.cn, "Speculative
  Decoding 的提议、验证与接受", sections 04 and 05; section 07 asks for exactly
  this frequency check, section 18 for one over 100,000 draws).  For draft-free
  rounds the same holds for any fixed draft token.
- The expected advance per round is E[S] = E[A] + 1 (section 09); with draft
  tokens drawn from q' independently per position, P(A >= k) is the product of
  the per-position acceptance masses a_j = sum_x min(p'_j, q'_j)(x), so
  E[S] = 1 + sum_{k=1..gamma} prod_{j<k} a_j.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from test_oracle_pins import np_draft, np_target, run

DRAWS = 1_000_000


def _sample_rows(rng, probs, n):
    """n draws from each row of probs [gamma, V]: returns [n, gamma]."""
    c = np.cumsum(probs, axis=1)
    u = rng.random((n, probs.shape[0])) * c[:, -1]
    return np.stack([np.minimum(np.searchsorted(c[j], u[:, j], side="right"), probs.shape[1] - 1)
                     for j in range(probs.shape[0])], axis=1).astype(np.int32)


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue


CASES = [
    # V, gamma, T, top_k, top_p, null_q, seed
    (6, 2, 1.0, 0, 1.0, False, 0),
    (8, 3, 0.7, 5, 0.9, False, 1),
    (6, 2, 1.3, 0, 1.0, True, 2),
]


@pytest.mark.parametrize("V,gam,T,k,p,null_q,seed", CASES)
def test_first_token_marginal_and_expected_advance(oracle_mod, V, gam, T, k, p, null_q, seed):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((gam + 1, V)) * 1.5).astype(np.float32)
    q = softmax(rng.standard_normal((gam, V)) * 1.5, axis=1).astype(np.float32)
    P = np.array([np_target(logits[j], T, k, p) for j in range(gam + 1)])
    n = DRAWS
    if null_q:
        ids = np.broadcast_to(rng.integers(0, V, gam).astype(np.int32), (n, gam)).copy()
        Qd = None
    else:
        Qd = np.array([np_draft(q[j], T, k, p) for j in range(gam)])
        ids = _sample_rows(rng, Qd, n)
    b = dict(draft_ids=ids, draft_probs=None if null_q else np.broadcast_to(q, (n, gam, V)),
             target_logits=np.broadcast_to(logits, (n, gam + 1, V)), dtype="f32",
             temperature=np.full(n, T, np.float32), top_k=np.full(n, k, np.int32), top_p=np.full(n, p, np.float32),
             u_accept=(rng.integers(0, 1 << 24, (n, gam)) * 2.0 ** -24).astype(np.float32),
             u_sample=(rng.integers(0, 1 << 24, n) * 2.0 ** -24).astype(np.float32))
    r = run(oracle_mod, b, threads=8)
    assert (r["fault"] == 0).all()
    first = r["tokens"][:, 0]
    counts = np.bincount(first, minlength=V).astype(np.float64)
    assert counts[P[0] == 0].sum() == 0
    pv = _chi2_pvalue(counts, P[0])
    assert pv > 1e-3, (pv, counts / n, P[0])

    S = r["num_accepted"].astype(np.float64) + 1
    if null_q:
        acc = np.array([P[j, ids[0, j]] for j in range(gam)])
    else:
        acc = np.minimum(P[:gam], Qd).sum(axis=1)
    es = 1.0 + sum(np.prod(acc[:kk]) for kk in range(1, gam + 1))
    sigma = S.std() / np.sqrt(n)
    assert abs(S.mean() - es) < 4 * sigma + 1e-12, (S.mean(), es, sigma)
    # committed length is A + 1, padding after it
    lens = (r["tokens"] >= 0).sum(axis=1)
    np.testing.assert_array_equal(lens, r["num_accepted"] + 1)
