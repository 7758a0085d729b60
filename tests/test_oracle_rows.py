"""Per-row outputs of the oracle (zwjcode.cn page, section 14: when top-p runs
do not reproduce, record the filtered support set and its probability sum).

Each row's kept-set size, kept mass fraction and top-p cut margin are checked
against independent numpy code: sort the tempered values, keep the top-k set
(ties kept), walk whole tie groups from the largest down to the first whose
cumulative mass reaches top_p of the top-k mass, and measure how far top_p
lies from the two cumulative fractions around that cut."""
import numpy as np
import pytest

import workloads as W


def np_row(values, mass, k, top_p):
    """(kept count, kept mass / total mass, top-p margin) of one row, from the definitions."""
    V = values.shape[0]
    keep = np.ones(V, bool)
    if 1 <= k < V:
        keep = values >= np.sort(values)[::-1][k - 1]
    zk = mass[keep].sum()
    margin = np.inf
    if top_p < 1.0:
        groups = np.unique(values[keep])[::-1]
        cum = np.cumsum([mass[keep & (values == g)].sum() for g in groups]) / zk
        hit = np.nonzero(cum >= top_p)[0]
        t = int(hit[0]) if len(hit) else len(groups) - 1
        if len(hit):
            before = cum[t - 1] if t > 0 else 0.0
            margin = min(top_p - before, cum[t] - top_p)
        keep = keep & (values >= groups[t])
    return int(keep.sum()), mass[keep].sum() / mass.sum(), margin


def check_batch(b, o):
    N, G = b["draft_ids"].shape
    V = b["target_logits"].shape[-1]
    tl = W.bf16_bits_to_f32(b["target_logits"]) if b["dtype"] == "bf16" else b["target_logits"]
    for i in range(N):
        g = int(b["gamma"][i])
        T = float(b["temperature"][i])
        k, p = int(b["top_k"][i]), float(b["top_p"][i])
        if T == 0:
            assert np.isnan(o["row_margin"][i]).all() and (o["kept_p"][i] == -1).all()
            continue
        for j in range(G + 1):
            if j > g:
                assert np.isnan(o["row_margin"][i, j]) and o["kept_p"][i, j] == -1
                continue
            s = tl[i, j].astype(np.float64) / np.float64(np.float32(T))
            e = np.exp(s - s.max())
            n, f, mg = np_row(s, e, k, p)
            assert o["kept_p"][i, j] == n
            assert o["frac_p"][i, j] == pytest.approx(f, rel=1e-12)
            expect = mg
            if j < g and b["draft_probs"] is not None:
                r = b["draft_probs"][i, j].astype(np.float64) ** (1.0 / np.float64(np.float32(T)))
                nq, fq, mq = np_row(r, r, k, p)
                assert o["kept_q"][i, j] == nq
                assert o["frac_q"][i, j] == pytest.approx(fq, rel=1e-12)
                expect = min(mg, mq)
            if np.isinf(expect):
                assert np.isinf(o["row_margin"][i, j])
            else:
                assert o["row_margin"][i, j] == pytest.approx(expect, rel=1e-9, abs=1e-15)


@pytest.mark.parametrize("spec", [
    W.config(3, N=10, V=3000),
    W.config(3, N=6, V=2500, top_k=0, top_p=0.75, temperature=0.6),
    W.config(2, N=6, V=2000, top_k=40, top_p=1.0),
    W.config(4, N=8, V=1500, greedy_count=3),
    W.config(5, N=12, V=1024, top_k=20, top_p=0.8),
], ids=["topk_topp", "topp_only_lowT", "topk_only", "greedy_mix", "ragged"])
def test_row_outputs_match_numpy(oracle_mod, spec):
    b = W.generate(spec)
    q = b["draft_probs"]
    if q is not None and not b["has_q"].all():
        q = None  # the ragged batch as draft-free requests: q rows are not read
        b = dict(b, draft_probs=None)
    o = oracle_mod.run(b["draft_ids"], q, b["target_logits"], b["dtype"], b["temperature"], b["top_k"],
                       b["top_p"], b["u_accept"], b["u_sample"])
    check_batch(b, o)


def test_tie_heavy_rows(oracle_mod):
    """Coarse logits: many values tie at both cuts; sizes count every tied token."""
    rng = np.random.default_rng(3)
    V, G, N = 400, 2, 5
    l = (np.round(rng.standard_normal((N, G + 1, V)) * 2) / 2).astype(np.float32)
    q = np.exp(np.round(rng.standard_normal((N, G, V)) * 2) / 2)
    q = (q / q.sum(axis=-1, keepdims=True)).astype(np.float32)
    b = dict(draft_ids=rng.integers(0, V, (N, G)).astype(np.int32), draft_probs=q, target_logits=l, dtype="f32",
             temperature=np.ones(N, np.float32), top_k=np.full(N, 7, np.int32), top_p=np.full(N, 0.6, np.float32),
             u_accept=np.full((N, G), 0.5, np.float32), u_sample=np.full(N, 0.5, np.float32),
             gamma=np.full(N, G))
    o = oracle_mod.run(b["draft_ids"], q, l, "f32", b["temperature"], b["top_k"], b["top_p"], b["u_accept"],
                       b["u_sample"])
    check_batch(b, o)
    assert (o["kept_p"] >= 1).all() and (o["kept_p"] <= V).all()


def test_request_margin_covers_decisive_rows(oracle_mod):
    """The request's margin is at most the top-p margin of every row up to its
    first rejection (those rows decide the outcome)."""
    b = W.generate(W.config(3, N=40, V=2000, top_p=0.7))
    o = oracle_mod.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                       b["top_k"], b["top_p"], b["u_accept"], b["u_sample"])
    for i in range(40):
        A = int(o["num_accepted"][i])
        assert o["margin"][i] <= np.min(o["row_margin"][i, :A + 1])


# ------------------------------------------------------------------------------------------
# ambiguity kinds and the draw window
# ------------------------------------------------------------------------------------------

def np_softmax_rows(l, T):
    s = l.astype(np.float64) / np.float64(np.float32(T))
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_draw_window_matches_numpy(oracle_mod):
    """Without filters: p' and q' from numpy; the window's ends are
    searchsorted(cumsum(w), (u -+ 1e-6) S, 'right') over the positive
    weights, and a request is flagged for its draw exactly when the window
    holds more than its own token or u S lies within 1e-6 S of a boundary."""
    b = W.generate(W.config(2, N=60, V=400, peak=None, noise_sigma=0.05, temperature=0.9))
    tl = W.bf16_bits_to_f32(b["target_logits"])
    o = oracle_mod.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                       b["top_k"], b["top_p"], b["u_accept"], b["u_sample"])
    T = float(b["temperature"][0])
    for i in range(60):
        A, g = int(o["num_accepted"][i]), int(b["gamma"][i])
        p = np_softmax_rows(tl[i, A], T)
        if A < g:
            q = b["draft_probs"][i, A].astype(np.float64) ** (1.0 / np.float64(np.float32(T)))
            w = np.maximum(p - q / q.sum(), 0.0)
            if w.sum() == 0:
                w = p
        else:
            w = p
        pos = np.flatnonzero(w > 0)
        c = np.cumsum(w[pos])
        S = c[-1]
        u = float(b["u_sample"][i])
        at = lambda x: pos[min(np.searchsorted(c, x * S, side="right"), len(pos) - 1)]
        assert o["z_lo"][i] == at(u - 1e-6) and o["z_hi"][i] == at(u + 1e-6)
        near = np.min(np.abs(u - c / S)) < 1e-6
        assert bool(o["amb_kind"][i] & oracle_mod.AMB_CDF) == near


def test_ambiguity_kinds_on_crafted_requests(oracle_mod):
    """u_sample 5e-7 above the boundary between tokens 0 and 1 (bonus p' =
    (0.5, 0.25, 0.25)): token 1, window [0, 1], flagged for the draw only.
    u_accept 5e-7 above p'/q' = 0.5: rejected, flagged for the accept test."""
    lp = np.log(np.array([0.5, 0.25, 0.25]))
    l = np.stack([lp, lp]).astype(np.float32)[None]
    q = np.array([[[0.25, 0.25, 0.5]]], np.float32)  # q'(y = 0) = 0.25: p'/q' = 2, always accepted
    u_hi = np.float32(0.5) + np.float32(5e-7)
    one = dict(draft_ids=np.array([[0]], np.int32), draft_probs=q, target_logits=l,
               temperature=np.ones(1, np.float32), top_k=np.zeros(1, np.int32), top_p=np.ones(1, np.float32))
    o = oracle_mod.run(one["draft_ids"], q, l, "f32", one["temperature"], one["top_k"], one["top_p"],
                       np.array([[0.3]], np.float32), np.array([u_hi], np.float32))
    assert o["num_accepted"][0] == 1 and o["tokens"][0, 1] == 1
    assert o["amb_kind"][0] == oracle_mod.AMB_CDF and (o["z_lo"][0], o["z_hi"][0]) == (0, 1)
    # far from every boundary: a one-token window, no flag
    o = oracle_mod.run(one["draft_ids"], q, l, "f32", one["temperature"], one["top_k"], one["top_p"],
                       np.array([[0.3]], np.float32), np.array([0.6], np.float32))
    assert o["amb_kind"][0] == 0 and o["z_lo"][0] == o["z_hi"][0] == o["tokens"][0, 1] == 1
    # accept ratio p'/q' = 0.5 (draft token 1: p' = 0.25, q' = 0.5)
    q2 = np.array([[[0.25, 0.5, 0.25]]], np.float32)
    o = oracle_mod.run(np.array([[1]], np.int32), q2, l, "f32", one["temperature"], one["top_k"], one["top_p"],
                       np.array([[u_hi]], np.float32), np.array([0.9], np.float32))
    assert o["num_accepted"][0] == 0
    assert o["amb_kind"][0] & oracle_mod.AMB_ACCEPT
    assert not o["amb_kind"][0] & oracle_mod.AMB_CDF
