"""Exactness of the GPU sampler in law (SD page, sections 04 and 06: with drafts
drawn from q', the committed tokens follow p').  Many requests share one set of
target and draft rows; each has its own drafts (drawn from q' here, in numpy)
and uniforms.  The first committed token must then be distributed as p'_0,
whatever q' is.  p' and q' are computed here with numpy (softmax, and the
top-k / top-p cut on values without ties), independently of the oracle."""
import numpy as np
import pytest
from scipy.stats import chisquare

from parity import log

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("k,top_p", [(0, 1.0), (4, 0.85)])
def test_first_token_follows_target(k, top_p):
    import torch
    import rejection_sampling_verify_13_amd as sv
    rng = np.random.default_rng(2024 + k)
    V, G, N = 7, 2, 20000
    l = rng.normal(0, 1.2, (G + 1, V)).astype(np.float32)
    q = np.stack([np.exp(rng.normal(0, 1.2, V)) for _ in range(G)])
    q = (q / q.sum(axis=1, keepdims=True)).astype(np.float32)
    p_f = [_filtered(np.exp(l[j].astype(np.float64) - l[j].max()), k, top_p) for j in range(G + 1)]
    q_f = [_filtered(q[j].astype(np.float64), k, top_p) for j in range(G)]
    ids = np.stack([rng.choice(V, size=N, p=q_f[j]) for j in range(G)], axis=1).astype(np.int32)
    u24 = lambda shape: (rng.integers(0, 1 << 24, size=shape) * 2.0 ** -24).astype(np.float32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    log("[stats] first-token law, N=%d V=%d top_k=%d top_p=%.2f" % (N, V, k, top_p))
    t, n = sv.verify(d(ids), d(np.broadcast_to(q, (N, G, V))), d(np.broadcast_to(l, (N, G + 1, V))),
                     d(np.ones(N, np.float32)), d(np.full(N, k, np.int32)), d(np.full(N, top_p, np.float32)),
                     d(u24((N, G))), d(u24((N,))))
    torch.cuda.synchronize()
    first = t.cpu().numpy()[:, 0]
    counts = np.bincount(first, minlength=V)
    support = p_f[0] > 0
    assert counts[~support].sum() == 0, "tokens outside the kept set"
    res = chisquare(counts[support], N * p_f[0][support])
    log("[stats] counts %s expected %s p-value %.3g" % (counts.tolist(), np.round(N * p_f[0], 1).tolist(),
                                                       res.pvalue))
    assert res.pvalue > 1e-4
    # the mean advance E[A + 1] is the closed form 1 + a_0 + a_0 a_1 with a_j = sum_x min(p'_j, q'_j)
    a = [np.minimum(p_f[j], q_f[j]).sum() for j in range(G)]
    adv = (n.cpu().numpy() + 1).mean()
    expect = 1 + a[0] + a[0] * a[1]
    assert abs(adv - expect) < 5 * np.sqrt(1.0 / N), (adv, expect)
