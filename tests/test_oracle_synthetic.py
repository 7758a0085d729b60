"""Pins of the oracle's synthetic acceptance mode (no GPU).

vLLM page, section "关于 synthetic / block 验证模式": each position has a preset
acceptance rate and draft j is accepted iff u_j < rate_j, without the target
probabilities.  The token at the first rejection is drawn as in the standard
method, so it is pinned to the standard oracle (itself pinned elsewhere); the
acceptance rule is pinned by the closed-form law of A."""
import numpy as np

import oracle
import workloads as W

RATES = np.array([0.9, 0.8, 0.7, 0.55, 0.4], np.float32)


def _run(b, rates, ua=None):
    return oracle.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                      b["top_k"], b["top_p"], b["u_accept"] if ua is None else ua, b["u_sample"],
                      synthetic_rates=rates)


def test_synthetic_token_equals_standard_token_at_the_same_position():
    for cfg in (W.config(3, N=24, V=3000), W.config(4, N=24, gmax=5, V=2500, greedy_count=8),
                W.config(5, N=24, gmax=5, V=2000, q_mode="dense")):
        b = W.generate(cfg)
        std = oracle.run(b["draft_ids"], b["draft_probs"], b["target_logits"], b["dtype"], b["temperature"],
                         b["top_k"], b["top_p"], b["u_accept"], b["u_sample"])
        # u chosen so that the synthetic first rejection is the standard one
        ua = np.zeros_like(b["u_accept"])
        for i, A in enumerate(std["num_accepted"]):
            if 0 <= A < ua.shape[1]:
                ua[i, A] = np.float32(0.999)
        syn = _run(b, RATES, ua)
        ok = std["fault"] == 0
        np.testing.assert_array_equal(syn["num_accepted"][ok], std["num_accepted"][ok])
        np.testing.assert_array_equal(syn["tokens"][ok], std["tokens"][ok])
        assert np.isnan(syn["p_y"]).all() and np.isnan(syn["q_y"]).all()


def test_synthetic_acceptance_law():
    # A = j with probability rate_0 ... rate_{j-1} (1 - rate_j); A = gamma with prod(rates)
    b = W.generate(W.config(2, N=4000, gmax=5, V=64))
    res = _run(b, RATES)
    A = res["num_accepted"]
    expect = [np.prod(RATES[:j]) * (1 - RATES[j]) for j in range(5)] + [np.prod(RATES)]
    got = np.bincount(A, minlength=6) / len(A)
    sd = np.sqrt(np.array(expect) * (1 - np.array(expect)) / len(A))
    assert (np.abs(got - expect) < 5 * sd + 1e-9).all(), (got, expect)
    # and each request follows the rule exactly
    u = b["u_accept"]
    for i in range(50):
        j = next((t for t in range(5) if not u[i, t] < RATES[t]), 5)
        assert A[i] == j


def test_synthetic_reads_only_row_A():
    b = W.generate(W.config(3, N=1, V=500))
    ua = np.zeros_like(b["u_accept"])
    ua[0, 2] = 0.99  # A = 2
    tl = b["target_logits"].copy()
    tl[0, 4] = W.BF16_NAN  # a row after A: never read
    b2 = dict(b, target_logits=tl)
    r = _run(b2, RATES, ua)
    assert r["fault"][0] == 0 and r["num_accepted"][0] == 2
    tl[0, 2] = W.BF16_NAN  # row A itself
    r = _run(dict(b, target_logits=tl), RATES, ua)
    assert r["fault"][0] == oracle.FAULT_TARGET_ROW and r["num_accepted"][0] == -1
