"""Exactness of the GPU sampler in law (SD page, sections 04 and 06: with drafts
drawn from q', the committed tokens follow p'; section 13: frequency tests on
an enumerable vocabulary covering rejection at the first position, rejection
in the middle, full acceptance and zero-probability tokens).

10^6 requests share one set of target and draft rows; each has its own drafts
(drawn from q' here, in numpy) and uniforms.  Two laws are checked by
chi-square: the first committed token must follow p'_0 whatever q' is, and the
pair (A, token at A) must follow its closed form
    P(A = j, z) = a_0 ... a_{j-1} (1 - a_j) r_j(z)   for j < gamma,
    P(A = gamma, z) = a_0 ... a_{gamma-1} p'_gamma(z),
with a_j = sum_x min(p'_j, q'_j)(x) and r_j = max(0, p'_j - q'_j) / (1 - a_j);
cells of probability zero must stay empty.  p' and q' are computed here with
numpy (softmax, and the top-k / top-p cut on values without ties),
independently of the oracle."""
import numpy as np
import pytest
from scipy.stats import chisquare

from parity import log

pytestmark = pytest.mark.gpu

DRAWS = 1_000_000


def _filtered(w, k, top_p):
    w = np.asarray(w, np.float64)
    if 0 < k < len(w):
        w = np.where(w >= np.sort(w)[-k], w, 0.0)
    w = w / w.sum()
    if top_p < 1.0:
        order = np.argsort(-w)
        c = np.cumsum(w[order])
        keep = order[: int(np.searchsorted(c, top_p * c[-1]) + 1)]
        m = np.zeros_like(w)
        m[keep] = w[keep]
        w = m / m.sum()
    return w


def _chi2(counts, expect, label):
    """Chi-square over the cells with nonzero expectation (cells expected below 5
    pooled); cells of zero expectation must be empty."""
    counts, expect = np.asarray(counts, np.float64), np.asarray(expect, np.float64)
    assert counts[expect == 0].sum() == 0, "%s: draws in cells of probability zero" % label
    live = expect > 0
    c, e = counts[live], expect[live]
    small = e < 5
    if small.any():
        c = np.append(c[~small], c[small].sum())
        e = np.append(e[~small], e[small].sum())
    res = chisquare(c, e * c.sum() / e.sum())
    log("[stats] %s: %d cells, chi-square p-value %.3g" % (label, len(c), res.pvalue))
    return res.pvalue


@pytest.mark.parametrize("k,top_p", [(0, 1.0), (4, 0.85)])
def test_law_of_committed_tokens(k, top_p):
    import torch
    import rejection_sampling_verify_13_amd as sv
    rng = np.random.default_rng(2024 + k)
    V, G, N = 7, 2, DRAWS
    l = rng.normal(0, 1.2, (G + 1, V)).astype(np.float32)
    q = np.stack([np.exp(rng.normal(0, 1.2, V)) for _ in range(G)])
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    p_f = [_filtered(np.exp(l[j].astype(np.float64) - l[j].max()), k, top_p) for j in range(G + 1)]
    q_f = [_filtered(q[j].astype(np.float64), k, top_p) for j in range(G)]
    ids = np.stack([rng.choice(V, size=N, p=q_f[j]) for j in range(G)], axis=1).astype(np.int32)
    u24 = lambda shape: (rng.integers(0, 1 << 24, size=shape) * 2.0 ** -24).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    log("[stats] law of the committed tokens, N=%d V=%d top_k=%d top_p=%.2f" % (N, V, k, top_p))
    t, n = sv.verify(d(ids), d(np.broadcast_to(q, (N, G, V))), d(np.broadcast_to(l, (N, G + 1, V))),
                     d(np.ones(N, np.float32)), d(np.full(N, k, np.int32)), d(np.full(N, top_p, np.float32)),
                     d(u24((N, G))), d(u24((N,))))
    torch.cuda.synchronize()
    tok = t.cpu().numpy()
    A = n.cpu().numpy().astype(np.int64)
    assert (A >= 0).all() and (A <= G).all()
    # the first committed token follows p'_0
    first = tok[:, 0]
    assert _chi2(np.bincount(first, minlength=V), N * p_f[0], "first token ~ p'_0") > 1e-4
    # the pair (A, token at A) follows the closed form
    a = [np.minimum(p_f[j], q_f[j]).sum() for j in range(G)]
    expect = np.zeros((G + 1, V))
    reach = 1.0
    for j in range(G):
        resid = np.maximum(p_f[j] - q_f[j], 0.0)
        expect[j] = reach * resid  # (1 - a_j) r_j = max(0, p'_j - q'_j)
        reach *= a[j]
    expect[G] = reach * p_f[G]
    z = tok[np.arange(N), A]
    counts = np.zeros((G + 1, V))
    np.add.at(counts, (A, z), 1)
    assert _chi2(counts.ravel(), N * expect.ravel(), "(A, token at A)") > 1e-4
    # every stopping position of non-negligible probability is reached (first,
    # middle, none rejected); with top-k 4 / top-p 0.85 full acceptance has
    # probability zero and its cells stay empty (checked above)
    assert all(counts[j].sum() > 1000 for j in range(G + 1) if expect[j].sum() > 0.01)
    # the mean advance E[A + 1] is the closed form 1 + a_0 + a_0 a_1
    adv = (A + 1).mean()
    exp_adv = 1 + a[0] + a[0] * a[1]
    assert abs(adv - exp_adv) < 5 * np.sqrt(1.0 / N), (adv, exp_adv)
