"""The two forms of the draw pass agree bit for bit.  A call of 128 to 384
requests without token lists runs the fused draw pass (one workgroup per
request: block sums in LDS, then the search); any other call runs the split
one (block sums over many workgroups, then a search launch).  Both form the
same weights, lane sums and 512-token block sums, so the same requests
verified as one 128-request call and as two 64-request calls must commit the
same tokens and report the same residual mass.  Unfiltered rows (every draw
left to the draw pass), near-copy drafts (small residual mass), drafts equal
to the target (a residual of rounding size), and T = 0.4 (the fp64 draft
weights) are included."""
import numpy as np
import pytest

import workloads as W
from parity import log

pytestmark = pytest.mark.gpu


def _run(b, parts):
    import torch
    import rejection_sampling_verify_13_amd as sv
    N = b["draft_ids"].shape[0]
    outs = []
    for lo, hi in parts:
        p = {k: (v[lo:hi] if isinstance(v, np.ndarray) and v.shape[:1] == (N,) else v) for k, v in b.items()}
        t, n, dg = sv.verify_batch(sv.to_device(p), diag=True)
        outs.append((t, n, dg["resid_mass"]))
    torch.cuda.synchronize()
    return (np.concatenate([o[0].cpu().numpy() for o in outs]), np.concatenate([o[1].cpu().numpy() for o in outs]),
            np.concatenate([o[2].cpu().numpy() for o in outs]))


CASES = ["peaked_T08", "near_copy", "low_T", "draft_equals_target"]


@pytest.mark.parametrize("case", CASES)
def test_fused_and_split_draw_pass_agree(case):
    if case == "peaked_T08":
        spec = W.config(2, N=128, V=20000)
    elif case == "near_copy":
        spec = W.config(2, N=128, gmax=3, V=20000, peak=None, noise_sigma=0.03, temperature=1.0)
    elif case == "low_T":
        spec = W.config(2, N=128, V=6000, peak=None, noise_sigma=0.5, temperature=0.4)
    else:
        spec = W.config(2, N=128, gmax=2, V=3000, peak=None, noise_sigma=1.0, temperature=1.0)
    spec.seed = 9100 + CASES.index(case)
    b = W.generate(spec, threads=8)
    if case == "near_copy":
        b["u_accept"] = np.full_like(b["u_accept"], 0.999)  # reject often: residual draws
    if case == "draft_equals_target":
        # q = p (T = 1) at every draft position, rounded to fp32: with u = 1 a draft is kept only where
        # rounding leaves q'(y) < p'(y), and the residual holds rounding-size mass
        tl = W.bf16_bits_to_f32(b["target_logits"]).astype(np.float64)
        e = np.exp(tl - tl.max(axis=-1, keepdims=True))
        b["draft_probs"] = (e / e.sum(axis=-1, keepdims=True))[:, :-1].astype(np.float32)
        b["u_accept"] = np.ones_like(b["u_accept"])
    log("[draw paths] %s: N=128 V=%d" % (case, spec.V))
    t1, n1, s1 = _run(b, [(0, 128)])      # fused draw pass
    t2, n2, s2 = _run(b, [(0, 64), (64, 128)])  # split draw pass
    assert np.array_equal(n1, n2)
    assert np.array_equal(t1, t2)
    assert np.array_equal(np.isnan(s1), np.isnan(s2))
    ok = ~np.isnan(s1)
    assert np.array_equal(s1[ok], s2[ok])
    log("[draw paths] %s ok: 128 requests, %d residual draws" % (case, int((n1 < b["gamma"]).sum())))
