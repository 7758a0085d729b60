"""GPU parity: the HIP path against the CPU oracle, request by request.

Reduced-size cases span several 2048-token workgroup steps and a ragged tail
(V not a multiple of the step; V not a multiple of 8 takes the scalar-load
path); full-size cases run the whole workload on the GPU exactly as the
benchmark does and compare every request with the oracle; stress cases put
many decisions near the margins (drafts close to the target over the whole
vocabulary, low temperatures).  Every case prints its name before it touches
the GPU.
"""
import numpy as np
import pytest

from conftest import floats, ints, read_golden
from parity import check_layout, compare, gpu_run, gpu_run_flat, log, oracle_run

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_13_amd  # noqa: F401  (raises if the library is missing)
    import oracle
    oracle.build(force=False)


def one_request(ids, q, logits, T=1.0, k=0, p=1.0, ua=None, us=0.5, dtype="f32"):
    ids = np.asarray(ids, np.int32).reshape(1, -1)
    g = ids.shape[1]
    return dict(draft_ids=ids, draft_probs=None if q is None else np.asarray(q, np.float32)[None],
                target_logits=np.asarray(logits, np.float32 if dtype == "f32" else np.uint16)[None], dtype=dtype,
                temperature=np.array([T], np.float32), top_k=np.array([k], np.int32), top_p=np.array([p], np.float32),
                u_accept=np.asarray(ua if ua is not None else np.zeros(g), np.float32).reshape(1, g),
                u_sample=np.array([us], np.float32))


def stack(reqs):
    out = {}
    for k in reqs[0]:
        v = reqs[0][k]
        out[k] = v if not isinstance(v, np.ndarray) else np.concatenate([r[k] for r in reqs], axis=0)
    return out


def parity(batch, label, rows=None):
    log("[parity] %s: N=%d gmax=%d V=%d dtype=%s" % (label, batch["draft_ids"].shape[0], batch["draft_ids"].shape[1],
                                                       batch["target_logits"].shape[-1], batch["dtype"]))
    g = gpu_run(batch)
    o = oracle_run(batch)
    res = compare(g, o, rows=rows, label=label)
    check_layout(batch, g)
    log("[parity] %s ok %s" % (label, res))
    return g, o, res


# ------------------------------------------------------------------------------------------
# the pages' examples on the GPU
# ------------------------------------------------------------------------------------------

def test_worked_example_on_gpu():
    g = read_golden("worked_example_two_token.txt")
    logits = np.log(np.array(floats(g["target_probs"])))
    reqs = [one_request(ints(g["draft_ids"]), floats(g["draft_probs"]), logits, ua=[float(g["u_accept"])], us=us)
            for us in np.linspace(0, 1, 16, endpoint=False)]
    b = stack(reqs)
    log("[parity] worked example")
    r = gpu_run(b)
    for t in range(len(reqs)):
        assert list(r["tokens"][t]) == ints(g["expect_tokens"])
        assert r["num_accepted"][t] == int(g["expect_num_accepted"])
        assert r["p_y"][t, 0] / r["q_y"][t, 0] == pytest.approx(float(g["expect_alpha"]), abs=1e-6)
        assert r["resid_mass"][t] == pytest.approx(0.4, abs=1e-6)
    compare(r, oracle_run(b), label="worked example")


def test_exercise_on_gpu():
    g = read_golden("exercise_three_token.txt")
    logits = np.log(np.array(floats(g["target_probs"])))
    us_list = [u for u in np.linspace(0, 1, 24, endpoint=False) if abs(u - 2 / 3) > 1e-3]
    b = stack([one_request(ints(g["draft_ids"]), floats(g["draft_probs"]), logits, ua=[0.41], us=u) for u in us_list])
    log("[parity] exercise")
    r = gpu_run(b)
    for t, u in enumerate(us_list):
        assert r["num_accepted"][t] == 0
        assert r["tokens"][t, 0] == (1 if u < 2 / 3 else 2)


def test_greedy_example_on_gpu():
    g = read_golden("greedy_example.txt")
    V = int(g["V"])
    rng = np.random.default_rng(0)
    rows = []
    for a in ints(g["target_argmax"]):
        l = rng.standard_normal(V).astype(np.float32)
        l[a] = l.max() + 1
        rows.append(l)
    logits = np.array(rows)
    b = stack([one_request(ints(g["draft_ids"]), None, logits, T=0.0),
               one_request(ints(g["all_match_draft_ids"]), None, logits, T=0.0)])
    log("[parity] greedy example")
    r = gpu_run(b)
    assert list(r["tokens"][0]) == ints(g["expect_tokens"]) and r["num_accepted"][0] == 2
    assert list(r["tokens"][1]) == ints(g["all_match_expect_tokens"]) and r["num_accepted"][1] == 4


# ------------------------------------------------------------------------------------------
# reduced-size workloads: every request compared
# ------------------------------------------------------------------------------------------

SMALL = {
    "cfg1": W.config(1),
    "cfg2_small": W.config(2, N=24, V=5000),
    "cfg3_small": W.config(3, N=16, V=12000),
    "cfg3_small_f32": W.config(3, N=12, V=9000, dtype="f32"),
    "cfg4_small": W.config(4, N=40, V=7000, greedy_count=10),
    "cfg5_small": W.config(5, N=48, V=6144),
    "unaligned_bf16": W.config(2, N=16, V=4999),
    "unaligned_f32_topk": W.config(3, N=10, V=3001, dtype="f32"),
    "null_q_topk": W.config(3, N=12, V=8000, q_mode="null"),
    "top_p_only": W.config(2, N=16, V=6000, top_p=0.8),
    "large_k_general_path": W.config(3, N=8, V=6000, top_k=300, top_p=1.0),
    "large_k_top_p": W.config(3, N=8, V=6000, top_k=500, top_p=0.7),
    "top_k_one": W.config(2, N=16, V=3000, top_k=1),
    "k_128_edge": W.config(3, N=8, V=4096, top_k=128, top_p=0.95),
    "greedy_all": W.config(4, N=24, V=5000, greedy_count=24),
    "low_temperature": W.config(2, N=16, V=4000, temperature=0.05),
    # low temperature on each path that forms tempered draft weights in fp32
    "low_temperature_general_topk": W.config(2, N=16, V=8000, gmax=8, top_k=65, top_p=0.5, temperature=0.05,
                                             dtype="f32"),
    "low_temperature_unfiltered": W.config(2, N=16, V=6000, top_k=0, top_p=1.0, temperature=0.08),
    "low_temperature_top_p_only": W.config(3, N=12, V=9000, top_k=0, top_p=0.9, temperature=0.15, dtype="f32"),
    "high_temperature": W.config(2, N=16, V=4000, temperature=3.0),
    "gamma_zero": W.config(2, N=12, gmax=0, V=3000),
    "gamma_max_64": W.config(2, N=3, gmax=64, V=2048),
    "tiny_vocab": W.config(1, N=20, V=3),
    "vocab_one": W.config(1, N=6, V=1),
    # more requests than the row planner lists per round, ragged drafts
    "many_requests_ragged": W.config(5, N=1500, gmax=3, V=1024, q_mode="dense"),
    # padded, ragged, gmax a multiple of 8: each request's draft positions take gmax + 1 row-pass slots
    "ragged_gmax_16": W.config(5, N=40, gmax=16, V=3000, q_mode="dense"),
    # 128 to 384 requests without token lists: the fused draw pass, unfiltered rows (every draw left to it)
    "fused_draw_unfiltered": W.config(2, N=160, gmax=3, V=5000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    b = W.generate(SMALL[name], threads=8)
    parity(b, name)


def test_mixed_per_request_parameters():
    rng = np.random.default_rng(5)
    b = W.generate(W.config(3, N=40, V=7000, top_k=0, top_p=1.0), threads=8)
    b["temperature"] = rng.choice([0.0, 0.5, 1.0, 1.7], 40).astype(np.float32)
    b["top_k"] = rng.choice([0, 1, 5, 50, 128, 129, 400, 7000, -3], 40).astype(np.int32)
    b["top_p"] = rng.choice([1.0, 0.95, 0.5, 0.1, 2.0], 40).astype(np.float32)
    parity(b, "mixed parameters")


def test_draft_equals_target_accepts_all():
    b = W.generate(W.config(1, N=16, V=2048), threads=8)
    l = b["target_logits"][:, :-1].astype(np.float64)
    e = np.exp(l - l.max(axis=2, keepdims=True))
    b["draft_probs"] = (e / e.sum(axis=2, keepdims=True)).astype(np.float32)
    g, o, _ = parity(b, "q equals p")
    amb = o["margin"] < 1e-6
    assert (g["num_accepted"][~amb] == b["draft_ids"].shape[1]).all()


def test_one_hot_q_equals_null_q():
    b = W.generate(W.config(2, N=16, V=3000), threads=8)
    oh = np.zeros_like(b["draft_probs"])
    for i in range(16):
        for j in range(4):
            oh[i, j, b["draft_ids"][i, j]] = 1.0
    g1 = gpu_run(dict(b, draft_probs=oh))
    g2 = gpu_run(dict(b, draft_probs=None, has_q=np.zeros(16, bool)))
    np.testing.assert_array_equal(g1["tokens"], g2["tokens"])
    np.testing.assert_array_equal(g1["num_accepted"], g2["num_accepted"])


def test_batch_composition_does_not_matter():
    # one request's result must not depend on its neighbours (no crosstalk)
    b = W.generate(W.config(5, N=32, V=4096), threads=8)
    full = gpu_run(b)
    for lo, hi in ((0, 1), (5, 9), (16, 17), (20, 32)):
        sub = {k: (v[lo:hi] if isinstance(v, np.ndarray) and v.shape[:1] == (32,) else v) for k, v in b.items()}
        if sub["draft_probs"] is not None:
            sub["draft_probs"] = b["draft_probs"][lo:hi]
        r = gpu_run(sub)
        np.testing.assert_array_equal(r["tokens"], full["tokens"][lo:hi])


def test_repeat_calls_are_identical():
    b = W.generate(W.config(3, N=16, V=20000), threads=8)
    r1, r2 = gpu_run(b), gpu_run(b)
    for k in ("tokens", "num_accepted", "p_y", "q_y", "resid_mass", "fault"):
        np.testing.assert_array_equal(r1[k], r2[k])


# ------------------------------------------------------------------------------------------
# faults and special values
# ------------------------------------------------------------------------------------------

def test_fault_injection():
    base = W.generate(W.config(2, N=16, V=2048), threads=8)
    b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
    nan16, inf16, ninf16 = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
    b["draft_ids"][0, 2] = 2048                 # id out of range
    b["temperature"][1] = -1.0                  # bad temperature
    b["temperature"][2] = np.nan
    b["top_p"][3] = 0.0                         # bad top_p
    b["target_logits"][4, 1, 77] = nan16        # NaN in a read target row
    b["target_logits"][5, 4, 5] = inf16         # +inf in the bonus row
    b["target_logits"][6, 2, :] = ninf16        # no finite value
    b["target_logits"][7, 0, 9] = ninf16        # a single -inf is fine
    b["draft_probs"][8, 3, 100] = -1e-3         # negative draft probability
    b["draft_probs"][9, 0, :] = 0.0             # zero draft mass
    b["draft_probs"][10, 1, 5] = np.inf
    b["temperature"][11] = 0.0                  # greedy: NaN in q rows is never read
    b["draft_probs"][11, 0, 3] = np.nan
    b["temperature"][12] = 0.0
    b["target_logits"][12, 3, 4] = nan16        # greedy: NaN in a target row is a fault
    b["draft_ids"][13, 1] = -1                  # padding: later rows are never read
    b["target_logits"][13, 2:, :] = nan16
    b["draft_probs"][13, 1:, :] = np.nan
    b["temperature"][14] = 1e-40                # subnormal temperature
    g, o, _ = parity(b, "fault injection")
    assert o["fault"][[0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 12, 14]].all()
    assert (o["fault"][[7, 11, 13, 15]] == 0).all()
    # a plain call's only fault output besides num_accepted = -1: the count in
    # its workspace, which the next call on that workspace starts again from zero
    import torch
    import rejection_sampling_verify_13_amd as sv
    log("[parity] fault count through spec_verify_device_errors")
    d = sv.to_device(b)
    ws = torch.empty((sv.workspace_size(16, 4, 2048),), dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # whatever the memory held before
    t, n = sv.verify_batch(d, workspace=ws)
    assert sv.device_errors(ws) == 12
    assert int((n.cpu().numpy() == -1).sum()) == 12
    t, n = sv.verify_batch(sv.to_device(base), workspace=ws)
    assert sv.device_errors(ws) == 0
    t, n = sv.verify_batch(d, workspace=ws)
    assert sv.device_errors(ws) == 12
    # the flattened entry point counts the same way
    t, n = sv.verify_flat_batch(sv.to_device_flat(W.flatten(b)), workspace=ws)
    assert sv.device_errors(ws) == int((n.cpu().numpy() == -1).sum())


def test_zero_residual_falls_back_to_target():
    """p' and q' both keep only the common argmax (top-p 0.05 alone, so the
    radix path and the draw pass serve it) and the draft token lies outside:
    it is rejected, max(0, p' - q') is zero everywhere, and the token is drawn
    from p' (zwjcode.cn page, section 04, residual; the zero-mass case is this
    build's reading), i.e. the argmax, for every u_sample."""
    rng = np.random.default_rng(31)
    V, reqs = 3000, []
    for r in range(12):
        l = rng.standard_normal((2, V)).astype(np.float32)
        a = int(rng.integers(V))
        l[:, a] = 6.0
        d = l[0].astype(np.float64) + 0.05 * rng.standard_normal(V)
        q = np.exp(d - d.max())
        q = (q / q.sum()).astype(np.float32)
        y = (a + 1 + int(rng.integers(V - 1))) % V
        reqs.append(one_request([y], q[None], l, p=0.05, ua=[float(rng.uniform())], us=float(rng.uniform())))
    b = stack(reqs)
    g, o, _ = parity(b, "zero residual")
    assert (g["num_accepted"] == 0).all()
    for r in range(12):
        assert g["tokens"][r, 0] == int(np.argmax(b["target_logits"][r, 0]))


def test_special_rows():
    V = 2048
    rng = np.random.default_rng(9)
    reqs = []
    l = (rng.standard_normal((3, V)) * 3).astype(np.float32)
    q = np.full((2, V), 1.0 / V, np.float32)
    # all logits equal (maximal ties) with top-k / top-p
    flat = np.zeros((3, V), np.float32)
    reqs.append(one_request([3, 7], q, flat, k=5, p=0.5, ua=[0.3, 0.9], us=0.77))
    reqs.append(one_request([3, 7], q, flat, k=0, p=0.3, ua=[0.3, 0.9], us=0.21))
    # mostly -inf rows (masked vocabulary)
    masked = np.full((3, V), -np.inf, np.float32)
    masked[:, [1, 500, 1999]] = [[1, 2, 3], [0, 0, 5], [2, 2, 2]]
    qm = np.zeros((2, V), np.float32)
    qm[:, [1, 500, 1999, 7]] = 0.25
    reqs.append(one_request([500, 7], qm, masked, ua=[0.1, 0.5], us=0.6))
    reqs.append(one_request([1999, 1], qm, masked, T=0.0))
    # draft token outside the target's top-k (p'(y) = 0): rejected
    reqs.append(one_request([int(np.argmin(l[0])), 1], q, l, k=10, ua=[0.0, 0.0], us=0.4))
    # huge logits (no overflow relative to the max)
    big = l * 1e4
    reqs.append(one_request([1, 2], q, big, ua=[0.5, 0.5], us=0.5))
    b = stack(reqs)
    parity(b, "special rows")


def test_all_64_drafts_accepted():
    """gmax = 64 with q' = p' at every position: every draft is accepted and the
    bonus token is drawn from the 65th row."""
    V = 3000
    rng = np.random.default_rng(33)
    reqs = []
    for r in range(2):
        l = (rng.standard_normal((65, V)) * 2).astype(np.float32)
        e = np.exp(l[:64].astype(np.float64) - l[:64].max(axis=1, keepdims=True))
        q = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
        y = [int(np.argmax(l[j])) for j in range(64)]
        reqs.append(one_request(y, q, l, k=0 if r == 0 else 20, ua=rng.uniform(0, 0.5, 64), us=float(rng.uniform())))
    b = stack(reqs)
    g, o, res = parity(b, "all 64 drafts accepted")
    assert list(g["num_accepted"]) == [64, 64]


def test_top_k_candidates_clustered_in_one_wave():
    """Rows whose values rise smoothly across the tokens one wave of the
    workgroup streams (so nearly every token of that wave's best chunks passes
    its own threshold), while the true top-k values sit in another wave's
    tokens: the kept set must still be exact."""
    V = 32000
    rng = np.random.default_rng(21)
    ids = np.arange(V)
    wave = (ids % 2048) // 512
    reqs = []
    for r in range(3):
        rows_l, rows_q = [], []
        for j in range(3):
            l = rng.standard_normal(V) * 0.5
            l[wave == 0] = 3.0 + 1e-4 * ids[wave == 0]
            spikes = rng.choice(np.flatnonzero(wave == 1), 80, replace=False)
            l[spikes] = 10.0 + rng.standard_normal(80)
            rows_l.append(l.astype(np.float32))
            d = l + 0.3 * rng.standard_normal(V)
            e = np.exp(d - d.max())
            rows_q.append((e / e.sum()).astype(np.float32))
        y = [int(np.argmax(rows_q[0])), int(rng.choice(np.flatnonzero(wave == 0)))]
        reqs.append(one_request(y, np.stack(rows_q[:2]), np.stack(rows_l), k=50, p=0.9,
                                ua=rng.uniform(size=2), us=float(rng.uniform())))
    parity(stack(reqs), "top-k candidates clustered in one wave")


# ------------------------------------------------------------------------------------------
# full workloads, launched exactly as the benchmark does, every request checked
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_every_request(cfg):
    import torch
    import rejection_sampling_verify_13_amd as sv
    spec = W.config(cfg)
    log("[parity] full config %d: N=%d gmax=%d V=%d (generating)" % (cfg, spec.N, spec.gmax, spec.V))
    b = W.generate(spec, threads=16)
    # the benchmark's call: config 5 (ragged, half draft-free) as one flattened call, the others padded
    log("[parity] full config %d: the benchmark's call on the GPU" % cfg)
    if cfg == 5:
        t, n = sv.verify_flat_batch(sv.to_device_flat(W.flatten(b)))
    else:
        t, n = sv.verify_batch(sv.to_device(b))
    torch.cuda.synchronize()
    bench_tokens, bench_num = t.cpu().numpy(), n.cpu().numpy()
    del t, n
    log("[parity] full config %d: the same call with diagnostics" % cfg)
    g = gpu_run_flat(b) if cfg == 5 else gpu_run(b)
    np.testing.assert_array_equal(g["tokens"], bench_tokens)
    np.testing.assert_array_equal(g["num_accepted"], bench_num)
    check_layout(b, g)
    log("[parity] full config %d: oracle on all %d requests" % (cfg, spec.N))
    o = oracle_run(b, threads=16)
    rows = int((b["gamma"] + 1).sum())
    res = compare(g, o, rows=rows, label="config %d" % cfg)
    # greedy requests: every one of them also against numpy's argmax
    greedy = np.nonzero(b["temperature"] == 0)[0]
    for i in greedy:
        gam = int(b["gamma"][i])
        tl = b["target_logits"][i, : gam + 1]
        am = np.argmax(W.bf16_bits_to_f32(tl) if b["dtype"] == "bf16" else tl, axis=1)
        A = gam
        for j in range(gam):
            if b["draft_ids"][i, j] != am[j]:
                A = j
                break
        assert g["num_accepted"][i] == A and g["tokens"][i, A] == am[A]
    assert (g["fault"] == 0).all()
    log("[parity] full config %d ok over %d rows %s, greedy checked %d" % (cfg, rows, res, len(greedy)))


# ------------------------------------------------------------------------------------------
# precision at the decision margins
# ------------------------------------------------------------------------------------------

def test_near_copy_drafts_full_vocabulary():
    """Drafts close to the target (draft logits = target + N(0, sigma^2), sigma
    0.02 and 0.05) at V = 128256 without top-k: the residual max(0, p' - q')
    then holds a few percent of the mass and the draw pass forms it from two
    nearly equal distributions.  Uniforms near 1 reject position 0 about half
    the time.  Every request is compared.  The residual mass S must agree with
    the oracle to 2e-7 absolute: p' and q' are each formed from fp32 weights
    (about 1e-7 relative per weight, not systematic), so S, a small difference
    of two unit masses, carries an absolute error near that size whatever its
    own size."""
    reqs = []
    for t, (sigma, T) in enumerate([(0.02, 1.0), (0.02, 0.7), (0.05, 1.0), (0.05, 0.7)]):
        spec = W.config(2, N=96, gmax=2, V=128256, peak=None, noise_sigma=sigma, temperature=T)
        spec.seed = 5100 + t
        b = W.generate(spec, threads=16)
        rng = np.random.default_rng(t)
        k = rng.integers(1, int(0.03 * (1 << 24)), size=b["u_accept"].shape)
        b["u_accept"] = (1.0 - k * 2.0 ** -24).astype(np.float32)
        reqs.append(b)
    b = {k: (np.concatenate([r[k] for r in reqs]) if isinstance(reqs[0][k], np.ndarray) else reqs[0][k])
         for k in reqs[0]}
    log("[parity] near-copy drafts: N=%d V=128256" % b["draft_ids"].shape[0])
    g = gpu_run(b)
    o = oracle_run(b, threads=16)
    res = compare(g, o, rows=int((b["gamma"] + 1).sum()), label="near-copy")
    ok = (o["fault"] == 0) & np.isfinite(o["resid_mass"])
    err = np.abs(g["resid_mass"][ok] - o["resid_mass"][ok])
    rejected = int((o["num_accepted"] < b["gamma"]).sum())
    log("[parity] near-copy ok %s, %d residual draws, min S %.3g, max S err %.3g (relative %.3g)" % (
        res, rejected, o["resid_mass"][ok].min(), err.max(), (err / o["resid_mass"][ok]).max()))
    assert rejected >= 150
    assert err.max() <= 2e-7


@pytest.mark.parametrize("k,p", [(0, 1.0), (20, 0.9), (0, 0.9)])
def test_low_temperature_decisions(k, p):
    """More than 10^5 accept decisions at T in [0.05, 0.1], drafts near the
    target (sigma 0.3) so that most positions are reached: the accept ratio
    p'(y)/q'(y) must stay within 2e-7 of the oracle's wherever it is below 1
    (five times inside the 1e-6 decision margin), and no request may differ."""
    spec = W.config(2, N=24000, gmax=8, V=2048, peak=None, noise_sigma=0.3, temp_range=(0.05, 0.1), top_k=k,
                    top_p=p)
    spec.seed = 7000 + k + int(p * 10)
    b = W.generate(spec, threads=16)
    log("[parity] low temperature k=%d p=%g: N=%d gmax=8 V=2048" % (k, p, spec.N))
    g = gpu_run(b)
    o = oracle_run(b, threads=16)
    res = compare(g, o, rows=int((b["gamma"] + 1).sum()), label="low T")
    ok = o["fault"] == 0
    decisions = int(np.minimum(o["num_accepted"][ok] + 1, b["gamma"][ok]).sum())
    log("[parity] low temperature ok %s, %d decisions" % (res, decisions))
    assert decisions >= 100000
    assert res["max_ratio_err"] <= 2e-7


# ------------------------------------------------------------------------------------------
# flattened (ragged) layout: one call, a per-request draft-row mask
# ------------------------------------------------------------------------------------------

FLAT = {
    "flat_cfg5_small_mixed": W.config(5, N=48, V=6144),
    "flat_cfg3_small": W.config(3, N=16, V=12000),
    "flat_cfg4_small_greedy": W.config(4, N=40, V=7000, greedy_count=10),
    "flat_null_q": W.config(3, N=12, V=8000, q_mode="null"),
    "flat_unaligned_f32": W.config(5, N=20, V=3001, dtype="f32"),
    "flat_gamma_max_64": W.config(2, N=3, gmax=64, V=2048),
    "flat_gamma_zero": W.config(2, N=12, gmax=0, V=3000),
    "flat_many_requests_mixed": W.config(5, N=1500, gmax=3, V=1024),
}


@pytest.mark.parametrize("name", list(FLAT))
def test_flat_layout_parity(name):
    b = W.generate(FLAT[name])
    log("[parity] %s: N=%d gmax=%d V=%d (flattened, one call)" % (name, b["draft_ids"].shape[0],
                                                                   b["draft_ids"].shape[1],
                                                                   b["target_logits"].shape[-1]))
    g = gpu_run_flat(b)
    res = compare(g, oracle_run(b), label=name)
    check_layout(b, g)
    log("[parity] %s ok %s" % (name, res))


def test_flat_equals_padded_bit_for_bit():
    # the two layouts run the same arithmetic: identical tokens, masses and faults
    b = W.generate(W.config(5, N=40, V=5000))
    log("[parity] flat vs padded: N=40 V=5000")
    f, p = gpu_run_flat(b), gpu_run(b)
    for k in ("tokens", "num_accepted", "fault"):
        np.testing.assert_array_equal(f[k], p[k])
    for k in ("p_y", "q_y", "resid_mass"):
        np.testing.assert_array_equal(f[k].view(np.uint64), p[k].view(np.uint64))


def _flat_call(flat, gmax, T):
    """verify_flat with num_drafts = T, which may stop short of the prefix sums:
    the arrays sized by num_drafts are cut to it (a faulted request reads none
    of its rows)."""
    import torch
    import rejection_sampling_verify_13_amd as sv
    d = sv.to_device_flat(flat)
    N = d["cu_num_draft_tokens"].shape[0]
    t, n, dg = sv.verify_flat(d["cu_num_draft_tokens"], d["draft_ids"][:T].contiguous(), d["draft_probs"],
                              d["has_draft_probs"], d["target_logits"][: T + N].contiguous(), gmax,
                              d["temperature"], d["top_k"], d["top_p"], d["u_accept"][:T].contiguous(),
                              d["u_sample"], diag=True)
    torch.cuda.synchronize()
    return dict(tokens=t.cpu().numpy(), num_accepted=n.cpu().numpy(), **{k: v.cpu().numpy() for k, v in dg.items()})


def test_flat_count_above_gmax_faults_only_that_request():
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(5, N=24, V=3000, q_mode="dense"))
    gam = b["gamma"]
    gcall = int(gam.max()) - 1
    assert gcall >= 1 and (gam > gcall).any() and (gam <= gcall).any()
    log("[parity] flat counts above gmax=%d" % gcall)
    g = _flat_call(W.flatten(b), gcall, int(gam.sum()))
    o = oracle_run(b)
    bad = gam > gcall
    assert (g["fault"][bad] == sv.FAULT_DRAFT_COUNT).all()
    assert (g["tokens"][bad] == -1).all() and (g["num_accepted"][bad] == -1).all()
    ok = ~bad
    np.testing.assert_array_equal(g["fault"][ok], o["fault"][ok])
    amb = o["margin"][ok] < 1e-6
    tok_g, tok_o = g["tokens"][ok], o["tokens"][ok][:, : gcall + 1]
    same = (tok_g == tok_o).all(axis=1) & (g["num_accepted"][ok] == o["num_accepted"][ok])
    assert (same | amb).all()
    assert (o["tokens"][ok][:, gcall + 1:] == -1).all()


def test_flat_prefix_past_num_drafts_faults_the_tail():
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(3, N=10, V=4000))
    gam = b["gamma"]
    T = int(gam.sum())
    log("[parity] flat prefix sums past num_drafts = %d" % (T - 1))
    g = _flat_call(W.flatten(b), int(b["draft_ids"].shape[1]), T - 1)
    o = oracle_run(b)
    cu = np.cumsum(gam)
    bad = cu > T - 1
    assert bad[-1] and (g["fault"][bad] == sv.FAULT_DRAFT_COUNT).all()
    ok = ~bad
    amb = o["margin"][ok] < 1e-6
    same = (g["tokens"][ok] == o["tokens"][ok]).all(axis=1) & (g["num_accepted"][ok] == o["num_accepted"][ok])
    assert (same | amb).all()


# ------------------------------------------------------------------------------------------
# KV bookkeeping after verification
# ------------------------------------------------------------------------------------------

def _rollback_case(rng, N, G, flat):
    gam = rng.integers(0, G + 1, N)
    A = np.array([rng.integers(-1, g + 1) for g in gam], np.int32)
    nct = rng.integers(-3, 5000, N).astype(np.int32)
    nop = rng.integers(0, 10, N).astype(np.int32)
    slots = [rng.integers(0, 1 << 30, g).astype(np.int32) for g in gam]
    return gam, A, nct, nop, slots


@pytest.mark.parametrize("flat", [False, True])
def test_rollback_matches_oracle(flat):
    import torch
    import oracle
    import rejection_sampling_verify_13_amd as sv
    rng = np.random.default_rng(11 + flat)
    N, G = 700, 8
    gam, A, nct, nop, slots = _rollback_case(rng, N, G, flat)
    log("[parity] rollback %s N=%d" % ("flattened" if flat else "padded", N))
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    nct_d, nop_d = t(nct), t(nop)
    if flat:
        cu = np.cumsum(gam).astype(np.int32)
        sl_d = t(np.concatenate(slots + [np.zeros(0, np.int32)]))
        sv.rollback(t(A), cu_num_draft_tokens=t(cu), gmax=G, num_computed_tokens=nct_d,
                    num_output_placeholders=nop_d, slot_mapping=sl_d)
    else:
        ids = np.full((N, G), -1, np.int32)
        sl = np.full((N, G), 7, np.int32)
        for i in range(N):
            ids[i, : gam[i]] = rng.integers(0, 100, gam[i])
            sl[i, : gam[i]] = slots[i]
        sl_d = t(sl)
        sv.rollback(t(A), draft_ids=t(ids), num_computed_tokens=nct_d, num_output_placeholders=nop_d,
                    slot_mapping=sl_d)
    torch.cuda.synchronize()
    c, p, s = oracle.rollback(A, gam, nct, nop, slots)
    np.testing.assert_array_equal(nct_d.cpu().numpy(), np.array(c, np.int32))
    np.testing.assert_array_equal(nop_d.cpu().numpy(), np.array(p, np.int32))
    got = sl_d.cpu().numpy()
    if flat:
        np.testing.assert_array_equal(got, np.concatenate([np.array(r, np.int32) for r in s] + [np.zeros(0, np.int32)]))
    else:
        for i in range(N):
            np.testing.assert_array_equal(got[i, : gam[i]], np.array(s[i], np.int32))
            assert (got[i, gam[i]:] == 7).all()  # padding positions are not touched


def test_verify_then_rollback_on_one_stream():
    import torch
    import oracle
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(5, N=64, V=4096))
    f = W.flatten(b)
    log("[parity] verify then rollback: N=64 flattened, one stream")
    d = sv.to_device_flat(f)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nct = torch.full((64,), 1000, dtype=torch.int32, device="cuda")
        sl = torch.arange(d["draft_ids"].shape[0], dtype=torch.int32, device="cuda")
        _, n = sv.verify_flat_batch(d, stream=s)
        sv.rollback(n, cu_num_draft_tokens=d["cu_num_draft_tokens"], gmax=f["gmax"], num_computed_tokens=nct,
                    slot_mapping=sl, stream=s)
    torch.cuda.synchronize()
    A = n.cpu().numpy()
    o = oracle_run(b)
    amb = o["margin"] < 1e-6
    assert ((A == o["num_accepted"]) | amb).all()
    gam = b["gamma"]
    slots = [list(range(a, b_)) for a, b_ in zip(np.r_[0, np.cumsum(gam)[:-1]], np.cumsum(gam))]
    c, _, ss = oracle.rollback(A, gam, np.full(64, 1000), None, slots)
    np.testing.assert_array_equal(nct.cpu().numpy(), np.array(c))
    np.testing.assert_array_equal(sl.cpu().numpy(), np.array([x for r in ss for x in r], np.int32))


# ------------------------------------------------------------------------------------------
# synthetic acceptance mode (u_j < rate_j; only row A is read)
# ------------------------------------------------------------------------------------------

SYN_RATES = np.array([0.9, 0.8, 0.7, 0.55, 0.4, 0.3, 0.2, 0.1], np.float32)
SYN = {
    "syn_cfg3_small": W.config(3, N=16, V=12000),
    "syn_cfg5_small_mixed": W.config(5, N=48, V=6144),
    "syn_cfg4_small_greedy": W.config(4, N=40, V=7000, greedy_count=10),
    "syn_cfg2_unaligned": W.config(2, N=16, V=4999),
    "syn_gamma_zero": W.config(2, N=8, gmax=0, V=3000),
}


@pytest.mark.parametrize("name", list(SYN))
def test_synthetic_parity(name):
    b = W.generate(SYN[name])
    G = b["draft_ids"].shape[1]
    rates = SYN_RATES[:G]
    log("[parity] %s: synthetic acceptance, N=%d gmax=%d V=%d" % (name, b["draft_ids"].shape[0], G,
                                                                  b["target_logits"].shape[-1]))
    g = gpu_run_flat(b, synthetic_rates=rates)
    res = compare(g, oracle_run(b, synthetic_rates=rates), label=name)
    check_layout(b, g)
    log("[parity] %s ok %s" % (name, res))


# ------------------------------------------------------------------------------------------
# banned tokens (identical in p and q)
# ------------------------------------------------------------------------------------------

def _ban_lists(b, seed, n):
    """n random banned ids per request, plus, for every third request, its first
    draft token and, for every fifth, the argmax of its first target row."""
    rng = np.random.default_rng(seed)
    N, V = b["draft_ids"].shape[0], b["target_logits"].shape[-1]
    tl = b["target_logits"]
    lists = []
    for i in range(N):
        x = set(rng.choice(V, size=min(n, V), replace=False).tolist())
        if i % 3 == 0 and b["draft_ids"].shape[1] and b["draft_ids"][i, 0] >= 0:
            x.add(int(b["draft_ids"][i, 0]))
        if i % 5 == 0:
            row = W.bf16_bits_to_f32(tl[i, 0]) if b["dtype"] == "bf16" else tl[i, 0]
            x.add(int(np.argmax(row)))
        lists.append(np.array(sorted(x), np.int32))
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    return off, np.concatenate(lists).astype(np.int32)


BAN = {
    "ban_cfg3_small_topk": (W.config(3, N=16, V=12000), 60),
    "ban_cfg2_tempered": (W.config(2, N=24, V=5000), 40),
    "ban_cfg4_small_greedy": (W.config(4, N=40, V=7000, greedy_count=10), 30),
    "ban_cfg5_small_mixed": (W.config(5, N=48, V=6144), 50),
    "ban_top_p_only": (W.config(2, N=12, V=6000, top_p=0.8), 25),
    "ban_unaligned_f32_topk": (W.config(3, N=10, V=3001, dtype="f32"), 20),
    "ban_long_lists": (W.config(3, N=8, V=9000), 512),
    "ban_low_temperature_top_p": (W.config(2, N=12, V=6000, top_k=0, top_p=0.9, temperature=0.1), 40),
}


@pytest.mark.parametrize("name", list(BAN))
def test_banned_tokens_parity(name):
    cfg, n = BAN[name]
    b = W.generate(cfg)
    banned = _ban_lists(b, 5, n)
    log("[parity] %s: N=%d V=%d, %d banned ids" % (name, b["draft_ids"].shape[0], b["target_logits"].shape[-1],
                                                      len(banned[1])))
    g = gpu_run_flat(b, banned=banned)
    res = compare(g, oracle_run(b, banned=banned), label=name)
    off, ids = banned
    for i in range(len(off) - 1):
        A = g["num_accepted"][i]
        if A >= 0:
            assert not np.isin(g["tokens"][i, : A + 1], ids[off[i]:off[i + 1]]).any()
    log("[parity] %s ok %s" % (name, res))


def test_banned_list_faults_and_full_ban():
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(1, N=6, gmax=2, V=16))
    lists = [[3, 1], [16], [-1, 2], list(range(16)), [5, 5], [2, 9]]
    off = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    ids = np.concatenate([np.array(x, np.int32) for x in lists])
    log("[parity] malformed and full ban lists")
    g = gpu_run_flat(b, banned=(off, ids))
    o = oracle_run(b, banned=(off, ids))
    np.testing.assert_array_equal(g["fault"], o["fault"])
    assert (g["fault"][[0, 1, 2, 4]] == sv.FAULT_BAN_LIST).all() and g["fault"][3] == sv.FAULT_TARGET_ROW
    assert g["fault"][5] == 0
    compare(g, o, label="ban lists")


# ------------------------------------------------------------------------------------------
# target rows addressed through row indices (vLLM's target_logits_indices and
# bonus_logits_indices), inside a larger logits tensor whose other rows are NaN
# ------------------------------------------------------------------------------------------

SCAT = {
    "rows_cfg3_small_topk": (W.config(3, N=24, V=12000), 0),
    "rows_cfg5_small_mixed": (W.config(5, N=48, V=6144), 0),
    "rows_cfg4_small_greedy": (W.config(4, N=40, V=7000, greedy_count=10), 0),
    "rows_unaligned_f32_banned": (W.config(2, N=16, V=3001, dtype="f32"), 30),
    "rows_cfg2_ragged": (W.config(2, N=20, V=5000), 0),
}


@pytest.mark.parametrize("name", list(SCAT))
def test_row_indices_parity(name):
    cfg, nban = SCAT[name]
    b = W.generate(cfg)
    N = b["draft_ids"].shape[0]
    banned = _ban_lists(b, 9, nban) if nban else None
    log("[parity] %s: N=%d V=%d, rows scattered over %d extra NaN rows" % (name, N, b["target_logits"].shape[-1],
                                                                       N // 2 + 3))
    g = gpu_run_flat(b, banned=banned, scatter=(11, N // 2 + 3))
    res = compare(g, oracle_run(b, banned=banned), label=name)
    log("[parity] %s ok %s" % (name, res))


def test_row_index_faults():
    """An index outside [0, R) faults its request alone; the others match the
    oracle on the ordered rows."""
    import torch
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(3, N=8, V=4096))
    flat = W.scatter_rows(W.flatten(b), 3, 5)
    R = flat["target_logits"].shape[0]
    cu = flat["cu_num_draft_tokens"]
    assert cu[1] > cu[0] and cu[6] > cu[5]
    flat["target_logits_indices"][cu[0]] = R           # request 1: first draft row past the end
    flat["bonus_logits_indices"][4] = -1               # request 4: negative bonus row
    flat["target_logits_indices"][cu[6] - 1] = R + 99  # request 6: last draft row
    log("[parity] out-of-range row indices, R=%d" % R)
    d = sv.to_device_flat(flat)
    t, n, dg = sv.verify_flat_batch(d, diag=True)
    torch.cuda.synchronize()
    g = dict(tokens=t.cpu().numpy(), num_accepted=n.cpu().numpy(), **{k: v.cpu().numpy() for k, v in dg.items()})
    o = oracle_run(b)
    bad = [1, 4, 6]
    assert (g["fault"][bad] == sv.FAULT_ROW_INDEX).all()
    assert (g["tokens"][bad] == -1).all() and (g["num_accepted"][bad] == -1).all()
    keep = np.setdiff1d(np.arange(8), bad)
    compare({k: v[keep] for k, v in g.items()}, {k: v[keep] for k, v in o.items()}, label="row index faults")


# ------------------------------------------------------------------------------------------
# repetition penalties (per-position lists, identical in p and q)
# ------------------------------------------------------------------------------------------

def _penalty_params(b, seed, lists):
    """theta may differ from 1 only on greedy or draft-free requests; presence
    and frequency anywhere."""
    rng = np.random.default_rng(seed)
    N = b["draft_ids"].shape[0]
    if b["draft_probs"] is None:
        dense = np.zeros(N, bool)
    else:
        dense = np.asarray(b.get("has_q", np.ones(N, bool)), bool)
    stoch = b["temperature"] != 0
    theta = np.where(dense & stoch, 1.0, rng.uniform(0.8, 1.6, N)).astype(np.float32)
    return dict(lists=lists, repetition=theta, presence=rng.uniform(-0.3, 1.5, N).astype(np.float32),
                frequency=rng.uniform(0.0, 0.8, N).astype(np.float32))


PEN = {
    "pen_cfg3_small_topk": (W.config(3, N=16, V=12000), 200, 0, None),
    "pen_cfg5_small_mixed": (W.config(5, N=48, V=6144), 100, 0, None),
    "pen_cfg4_small_greedy": (W.config(4, N=40, V=7000, greedy_count=10), 150, 0, None),
    "pen_cfg2_tempered": (W.config(2, N=24, V=5000), 300, 0, None),
    "pen_unaligned_f32_banned": (W.config(2, N=12, V=3001, dtype="f32"), 64, 20, None),
    "pen_long_lists": (W.config(3, N=8, V=9000), 1024 - 5, 0, None),
    "pen_rows_scattered": (W.config(3, N=12, V=8192), 120, 10, (13, 9)),
    # penalised draft rows streamed unfiltered at low temperature
    "pen_low_temperature": (W.config(2, N=16, V=6000, top_k=0, top_p=1.0, temperature=0.1), 200, 0, None),
}


@pytest.mark.parametrize("name", list(PEN))
def test_penalties_parity(name):
    cfg, n_ctx, nban, scatter = PEN[name]
    b = W.generate(cfg)
    pen = _penalty_params(b, 21, W.penalty_lists(b, 22, n_ctx))
    banned = _ban_lists(b, 23, nban) if nban else None
    npen = sum(len(r[0]) for req in pen["lists"] for r in req)
    log("[parity] %s: N=%d V=%d, %d penalty entries" % (name, b["draft_ids"].shape[0], b["target_logits"].shape[-1],
                                                        npen))
    g = gpu_run_flat(b, banned=banned, scatter=scatter, penalties=pen)
    o = oracle_run(b, banned=banned, penalties=pen)
    assert (o["fault"] == 0).all()
    res = compare(g, o, label=name)
    log("[parity] %s ok %s" % (name, res))


def test_penalty_faults():
    b = W.generate(W.config(1, N=10, gmax=2, V=16))
    b["draft_ids"][:, :] = np.abs(b["draft_ids"])  # gamma = 2 everywhere
    b["temperature"][8] = -1.0
    ok = (np.array([1, 4], np.int32), np.array([0, 2], np.int32))
    lists = [[ok, ok, ok] for _ in range(10)]
    lists[1][2] = (np.array([4, 1], np.int32), np.array([0, 0], np.int32))    # not ascending
    lists[2][0] = (np.array([16], np.int32), np.array([1], np.int32))         # outside [0, V)
    lists[3][1] = (np.array([2, 3], np.int32), np.array([1, -1], np.int32))   # negative count
    lists[4][0] = (np.arange(1025, dtype=np.int32) % 16, np.zeros(1025, np.int32))  # too long
    theta = np.ones(10, np.float32)
    pres = np.zeros(10, np.float32)
    theta[5] = 1.5      # theta != 1 with draft rows at a nonzero temperature
    theta[6] = 0.0
    pres[7] = np.inf
    theta[8] = 2.0      # and a temperature fault
    pen = dict(lists=lists, repetition=theta, presence=pres)
    log("[parity] malformed penalty lists and values")
    g = gpu_run_flat(b, penalties=pen)
    o = oracle_run(b, penalties=pen)
    np.testing.assert_array_equal(g["fault"], o["fault"])
    import rejection_sampling_verify_13_amd as sv
    assert (g["fault"][1:8] == sv.FAULT_PENALTY).all() and g["fault"][0] == 0 and g["fault"][9] == 0
    compare(g, o, label="penalty faults")


def test_empty_option_lists_change_nothing():
    """Offsets whose lists are all empty, with the id arrays left NULL, give the
    plain call's outputs bit for bit (the options' kernels, nothing to apply)."""
    import torch
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(5, N=32, V=4096))
    d = sv.to_device_flat(W.flatten(b))
    N = b["draft_ids"].shape[0]
    T = d["draft_ids"].shape[0]
    log("[parity] empty option lists, N=%d" % N)
    t0, n0, g0 = sv.verify_flat_batch(d, diag=True)
    z = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
    f = lambda v: torch.full((N,), v, dtype=torch.float32, device="cuda")
    t1, n1, g1 = sv.verify_flat_batch(d, diag=True, banned_offsets=z(N + 1), penalty_offsets=z(T + N + 1),
                                      repetition_penalty=f(1.0), presence_penalty=f(0.7),
                                      frequency_penalty=f(0.3))
    torch.cuda.synchronize()
    assert torch.equal(t0, t1) and torch.equal(n0, n1)
    for k in ("p_y", "q_y", "fault"):
        assert torch.equal(torch.nan_to_num(g0[k], nan=-7.0), torch.nan_to_num(g1[k], nan=-7.0)), k



# ------------------------------------------------------------------------------------------
# brute force on tiny vocabularies: one request per cell of (y, u_accept,
# u_sample) space at the cell's midpoint; the GPU matches the oracle request by
# request and its law, summed over the cells, is the closed form
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("V,gam,T,k,p,null_q,seed", [
    (3, 2, 1.0, 0, 1.0, False, 1), (4, 2, 0.7, 0, 1.0, False, 2), (4, 2, 1.0, 2, 1.0, False, 3),
    (4, 2, 1.0, 0, 0.7, False, 4), (4, 1, 1.3, 3, 0.8, False, 5), (4, 2, 0.8, 0, 0.9, True, 7)])
def test_enumerated_cells_on_gpu(V, gam, T, k, p, null_q, seed):
    from scipy.special import softmax
    from test_oracle_pins import closed_form_law, law_cells
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((gam + 1, V)) * 1.5).astype(np.float32)
    q = None if null_q else softmax(rng.standard_normal((gam, V)) * 1.5, axis=1).astype(np.float32)
    ids_fixed = [int(x) for x in rng.integers(0, V, gam)] if null_q else None
    b, cases, P, Qd = law_cells(logits, q, T, k, p, gam, V, ids_fixed)
    log("[parity] enumerated cells V=%d gamma=%d T=%g k=%d p=%g null_q=%s: %d requests" % (
        V, gam, T, k, p, null_q, len(cases)))
    g = gpu_run(b)
    o = oracle_run(b)
    compare(g, o, label="cells")
    amb = (o["margin"] < 1e-6)
    law, slack = {}, 0.0
    for t, c in enumerate(cases):
        toks = tuple(int(x) for x in g["tokens"][t] if x >= 0)
        law[toks] = law.get(toks, 0.0) + c[3]
        if amb[t]:
            slack += c[3]
    want = closed_form_law(P, Qd, gam, ids_fixed)
    for key in set(want) | set(law):
        assert abs(law.get(key, 0.0) - want.get(key, 0.0)) <= 1e-9 + slack, key
