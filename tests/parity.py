"""Helpers shared by the GPU parity tests: run a batch through the HIP library
and through the CPU oracle, and compare the two by the stated tolerances.

Tolerances: token ids and num_accepted bit-exact on every request the oracle
does not flag as ambiguous; a request is ambiguous when one of its decisions
lies within 1e-6 of a boundary (|u - p'/q'| at a read position, |u - C_x/S| of
the draw, the top-p cut fraction).  Draws over the whole vocabulary land on a
token whose CDF interval is narrower than 2e-6 of S a few times in a hundred;
for those the accepted drafts must still match and the drawn token must lie in
the oracle's window of equally valid draws (see ``compare``).  Requests with
an ambiguous accept test or top-p cut must stay below 1e-4 of the rows
compared (at least one allowed per comparison only when 1e-4 of the rows
rounds up to one).  p'(y) and q'(y) must agree within 1e-5 absolute at every
draft position.  Fault bits must agree exactly.
"""
import math
import sys

import numpy as np

MARGIN = 1e-6
PROB_ATOL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(batch, diag=True, stream=None):
    """Run a numpy batch on cuda:0; mixed dense / draft-free batches go as two
    calls on contiguous halves, on the same stream."""
    import torch
    import rejection_sampling_verify_13_amd as sv
    import workloads as W
    parts = [batch]
    if batch["draft_probs"] is not None and "has_q" in batch and not batch["has_q"].all():
        parts = W.split_by_q(batch)
    outs = []
    for p in parts:
        d = sv.to_device(p)
        if diag:
            t, n, dg = sv.verify_batch(d, diag=True, stream=stream)
            outs.append(dict(tokens=t, num_accepted=n, **dg))
        else:
            t, n = sv.verify_batch(d, stream=stream)
            outs.append(dict(tokens=t, num_accepted=n))
    torch.cuda.synchronize()
    res = {}
    for k in outs[0]:
        res[k] = np.concatenate([o[k].cpu().numpy() for o in outs], axis=0)
    return res


def gpu_run_flat(batch, diag=True, stream=None, synthetic_rates=None, banned=None, scatter=None, penalties=None):
    """Run a numpy batch on cuda:0 as one call in the flattened layout (a mixed
    dense / draft-free batch included: the draft-row mask selects per request);
    with synthetic_rates, in the synthetic acceptance mode; with scatter =
    (seed, extra rows), its target rows scattered over a larger NaN-filled
    logits tensor and addressed through row indices; with penalties (the
    oracle's dict: lists, repetition, presence, frequency), repetition
    penalties."""
    import torch
    import rejection_sampling_verify_13_amd as sv
    import workloads as W
    flat = W.flatten(batch)
    if scatter is not None:
        flat = W.scatter_rows(flat, *scatter)
    d = sv.to_device_flat(flat)
    kw = {}
    if synthetic_rates is not None:
        kw["synthetic_rates"] = torch.from_numpy(np.ascontiguousarray(synthetic_rates, np.float32)).cuda()
    if banned is not None:
        kw["banned_offsets"] = torch.from_numpy(np.ascontiguousarray(banned[0], np.int32)).cuda()
        kw["banned_ids"] = torch.from_numpy(np.ascontiguousarray(banned[1], np.int32)).cuda()
    if penalties is not None:
        off, pid, cnt = W.flatten_penalties(penalties["lists"])
        for k, v in (("penalty_offsets", off), ("penalty_ids", pid), ("penalty_counts", cnt)):
            kw[k] = torch.from_numpy(v).cuda()
        for k in ("repetition", "presence", "frequency"):
            if penalties.get(k) is not None:
                kw[k + "_penalty"] = torch.from_numpy(np.ascontiguousarray(penalties[k], np.float32)).cuda()
    if diag:
        t, n, dg = sv.verify_flat_batch(d, diag=True, stream=stream, **kw)
        out = dict(tokens=t, num_accepted=n, **dg)
    else:
        t, n = sv.verify_flat_batch(d, stream=stream, **kw)
        out = dict(tokens=t, num_accepted=n)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_run(batch, threads=8, synthetic_rates=None, banned=None, penalties=None):
    import oracle
    import workloads as W
    parts = [batch]
    if batch["draft_probs"] is not None and "has_q" in batch and not batch["has_q"].all():
        parts = W.split_by_q(batch)
    bans = [None] * len(parts)
    if banned is not None:  # the lists of each contiguous part
        off, ids = np.asarray(banned[0], np.int64), np.asarray(banned[1])
        lo, bans = 0, []
        for p in parts:
            hi = lo + p["draft_ids"].shape[0]
            bans.append((off[lo:hi + 1] - off[lo], ids[off[lo]:off[hi]]))
            lo = hi
    pens = [None] * len(parts)
    if penalties is not None:  # each contiguous part's requests
        lo, pens = 0, []
        for p in parts:
            hi = lo + p["draft_ids"].shape[0]
            d = dict(lists=penalties["lists"][lo:hi])
            for k in ("repetition", "presence", "frequency"):
                if penalties.get(k) is not None:
                    d[k] = np.asarray(penalties[k])[lo:hi]
            pens.append(d)
            lo = hi
    outs = [oracle.run(p["draft_ids"], p["draft_probs"], p["target_logits"], p["dtype"], p["temperature"],
                       p["top_k"], p["top_p"], p["u_accept"], p["u_sample"], threads=threads,
                       synthetic_rates=synthetic_rates, banned=bn, penalties=pn)
            for p, bn, pn in zip(parts, bans, pens)]
    return {k: np.concatenate([o[k] for o in outs], axis=0) for k in outs[0]}


def compare(g, o, rows=None, label=""):
    """Assert parity of GPU results g with oracle results o; return counts.

    Tokens and num_accepted must be bit-exact on every request whose margin is
    at least MARGIN.  A request below it is ambiguous.  If only its draw is
    (u_sample within MARGIN of a CDF boundary), the accepted count must still
    be exact and the drawn token must lie in the oracle's window [z_lo, z_hi],
    the tokens drawn at u_sample -+ MARGIN: any of them is an equally valid
    draw at that precision.  Requests with an accept ratio or a top-p cut
    within MARGIN (their outcome can differ from there on) must stay below
    1e-4 of the rows.  p'(y) and q'(y) are compared at every draft position of
    every request without a fault, except rows whose own top-p cut lies within
    MARGIN of its threshold (the oracle's row_margin): such a row may keep a
    different set and still decide nothing.  The largest error of the accept
    ratio p'(y)/q'(y) where it is below 1 (where a decision can turn) is
    returned as max_ratio_err."""
    import oracle
    N = o["tokens"].shape[0]
    if rows is None:
        rows = max(1, N)
    ok = o["fault"] == 0
    amb = (o["margin"] < MARGIN) & ok
    undecided = ok & ((o["amb_kind"] & (oracle.AMB_ACCEPT | oracle.AMB_TOP_P)) != 0)
    window = amb & ~undecided  # only the draw is near a boundary
    fault_mismatch = np.nonzero(g["fault"] != o["fault"])[0] if "fault" in g else np.array([], int)
    assert len(fault_mismatch) == 0, "%s fault bits differ at requests %s: gpu %s oracle %s" % (
        label, fault_mismatch[:10], g["fault"][fault_mismatch[:10]], o["fault"][fault_mismatch[:10]])
    differ = (g["tokens"] != o["tokens"]).any(axis=1) | (g["num_accepted"] != o["num_accepted"])
    tok_bad = np.nonzero(~amb & differ)[0]
    if len(tok_bad):
        i = tok_bad[0]
        raise AssertionError("%s %d token mismatches (first request %d): gpu %s/%d oracle %s/%d margin %.3g" % (
            label, len(tok_bad), i, g["tokens"][i], g["num_accepted"][i], o["tokens"][i], o["num_accepted"][i],
            o["margin"][i]))
    for i in np.nonzero(window)[0]:
        A = int(o["num_accepted"][i])
        assert g["num_accepted"][i] == A and (g["tokens"][i, :A] == o["tokens"][i, :A]).all(), (
            "%s request %d: accepted drafts differ where only the draw is near a boundary" % (label, i))
        z = int(g["tokens"][i, A])
        assert o["z_lo"][i] <= z <= o["z_hi"][i], "%s request %d: token %d outside the window [%d, %d]" % (
            label, i, z, o["z_lo"][i], o["z_hi"][i])
    allowed = max(0, math.ceil(1e-4 * rows))
    assert undecided.sum() <= allowed, "%s %d requests with an accept ratio or top-p cut within %g, allowed %d" % (
        label, undecided.sum(), MARGIN, allowed)
    worst = ratio = 0.0
    rows_excused = 0
    if "p_y" in g:
        G = o["p_y"].shape[1]
        near_cut = o["row_margin"][:, :G] < MARGIN
        rows_excused = int((near_cut & ~np.isnan(o["p_y"]) & ok[:, None]).sum())
        both = ~np.isnan(o["p_y"]) & ok[:, None] & ~near_cut
        for key in ("p_y", "q_y"):
            a, b = g[key], o[key]
            assert not np.isnan(a[both]).any(), "%s %s missing on GPU" % (label, key)
            if both.any():
                d = np.abs(a[both] - b[both]).max()
                worst = max(worst, d)
                assert d <= PROB_ATOL, "%s %s differs by %.3g" % (label, key, d)
        with np.errstate(divide="ignore", invalid="ignore"):
            ro = o["p_y"] / o["q_y"]
            rg = g["p_y"] / g["q_y"]
        turn = both & (o["q_y"] > 0) & (ro < 1.0)
        if turn.any():
            ratio = float(np.abs(rg[turn] - ro[turn]).max())
    return dict(requests=N, ambiguous=int(amb.sum()), draw_window=int(window.sum()),
                draw_window_exact=int((window & ~differ).sum()), undecided=int(undecided.sum()),
                faults=int((o["fault"] != 0).sum()), max_prob_err=worst, max_ratio_err=ratio,
                rows_near_top_p_cut=rows_excused)


def check_layout(batch, g):
    """Properties that hold for every request at any size: -1 padding after
    the committed tokens, the accepted prefix equals the drafts, ids in range,
    num_accepted within the draft length."""
    ids = batch["draft_ids"]
    N, G = ids.shape
    V = batch["target_logits"].shape[-1]
    gam = np.full(N, G) if G == 0 else np.where((ids < 0).any(axis=1), np.argmax(ids < 0, axis=1), G)
    A = g["num_accepted"]
    ok = A >= 0
    assert (A[ok] <= gam[ok]).all()
    for i in np.nonzero(ok)[0]:
        a = A[i]
        assert (g["tokens"][i, :a] == ids[i, :a]).all()
        assert 0 <= g["tokens"][i, a] < V
        assert (g["tokens"][i, a + 1:] == -1).all()
    assert (g["tokens"][~ok] == -1).all()
