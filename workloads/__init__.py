"""Seeded synthetic inputs for batched draft-verify rejection sampling.

This module is shared by the tests, the benchmark and the smoke check; it feeds
both the HIP path and the CPU oracle.  It contains no step of the verifier
itself (no temperature/top-k/top-p transform, no acceptance test, no residual):
it only stands in for the two models that produce the verifier's inputs.

Shapes follow the batched verify interface: draft ids [N, gmax] padded with -1,
draft probabilities q [N, gmax, V] (float32) or None for draft-free (n-gram)
requests, target logits [N, gmax+1, V] (bfloat16 bit patterns as uint16, or
float32), per-request temperature / top_k / top_p, and the injected uniforms
u_accept [N, gmax] and u_sample [N].

Every request i draws from its own stream ``SeedSequence(seed, spawn_key=(i,))``,
so any subset of requests can be regenerated on its own and a batch is the
concatenation of its requests.  Batch-wide choices (which requests are greedy,
the ragged draft lengths) come from the stream ``SeedSequence(seed)``.
Uniforms are k * 2**-24 with k uniform in [0, 2**24): exact float32 values in
[0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    return (rng.integers(0, 1 << 24, size=shape, dtype=np.int64) * (2.0 ** -24)).astype(np.float32)


def _softmax64(d: np.ndarray) -> np.ndarray:
    d = d.astype(np.float64)
    e = np.exp(d - d.max())
    return e / e.sum()


def _draw(rng: np.random.Generator, probs: np.ndarray) -> int:
    c = np.cumsum(probs)
    return int(min(np.searchsorted(c, rng.random() * c[-1], side="right"), probs.shape[0] - 1))


@dataclasses.dataclass
class Spec:
    """Recipe of one synthetic batch."""
    N: int
    gmax: int
    V: int
    seed: int
    dtype: str = "bf16"               # target logits: "bf16" or "f32"
    logit_sigma: float = 3.0          # target logits ~ N(0, sigma^2)
    peak: Optional[float] = None      # + peak on one uniformly chosen token per row
    zipf: Optional[float] = None      # - zipf * ln(rank), rank a random permutation of 1..V
    noise_sigma: float = 1.0          # draft logits = target logits + N(0, noise^2)
    q_mode: str = "dense"             # "dense" q, "null" (draft-free), or "mixed": dense for i < N/2
    temperature: float = 1.0          # used when temp_range is None
    temp_range: Optional[tuple] = None  # T ~ U[lo, hi] per request
    greedy_count: int = 0             # this many requests (seeded choice) get T = 0
    top_k: int = 0
    top_p: float = 1.0
    draft_top_k: int = 0              # the draft model samples from its k most likely tokens
    argmax_prob: float = 0.0          # draft id = target argmax with this probability
    ragged: bool = False              # gamma_i ~ U{0..gmax-1}, -1 padded
    canaries: bool = False            # NaN in every row the verifier must not read

    def request_rng(self, i: int) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence(self.seed, spawn_key=(i,)))

    def batch_rng(self) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence(self.seed))


def _batch_params(spec: Spec):
    rng = spec.batch_rng()
    N = spec.N
    if spec.ragged:
        gam = rng.integers(0, spec.gmax, size=N) if spec.gmax > 0 else np.zeros(N, np.int64)
    else:
        gam = np.full(N, spec.gmax, np.int64)
    if spec.temp_range is not None:
        T = rng.uniform(spec.temp_range[0], spec.temp_range[1], size=N).astype(np.float32)
    else:
        T = np.full(N, spec.temperature, np.float32)
    if spec.greedy_count:
        T[rng.choice(N, size=spec.greedy_count, replace=False)] = 0.0
    return gam.astype(np.int64), T


def generate(spec: Spec, requests=None, threads: int = 1) -> dict:
    """Build the batch (or the listed subset of its requests, in that order).

    Requests are independent streams, so ``threads`` only changes the speed."""
    gam_all, T_all = _batch_params(spec)
    idx = np.arange(spec.N) if requests is None else np.asarray(requests, dtype=np.int64)
    n, G, V = len(idx), spec.gmax, spec.V
    bf16 = spec.dtype == "bf16"
    logits = np.empty((n, G + 1, V), np.uint16 if bf16 else np.float32)
    dense = spec.q_mode in ("dense", "mixed")
    q = np.empty((n, G, V), np.float32) if dense else None
    ids = np.full((n, G), -1, np.int32)
    ua = np.empty((n, G), np.float32)
    us = np.empty((n,), np.float32)
    has_q = np.zeros(n, bool)

    def one(r):
        i = int(idx[r])
        rng = spec.request_rng(i)
        g = int(gam_all[i])
        T = float(T_all[i])
        Td = T if T > 0 else 1.0
        req_dense = spec.q_mode == "dense" or (spec.q_mode == "mixed" and i < spec.N // 2)
        has_q[r] = req_dense
        for j in range(G + 1):
            if spec.canaries and j > g:
                logits[r, j] = BF16_NAN if bf16 else np.float32(np.nan)
                continue
            l = rng.standard_normal(V, dtype=np.float32) * np.float32(spec.logit_sigma)
            if spec.peak is not None:
                l[rng.integers(V)] += np.float32(spec.peak)
            if spec.zipf is not None:
                rank = rng.permutation(V).astype(np.float64) + 1.0
                l = (l.astype(np.float64) - spec.zipf * np.log(rank)).astype(np.float32)
            if bf16:
                logits[r, j] = f32_to_bf16_bits(l)
                lf = bf16_bits_to_f32(logits[r, j])
            else:
                logits[r, j] = l
                lf = l
            if j == G:
                continue
            if j >= g:
                if q is not None:
                    q[r, j] = np.nan if spec.canaries else 0.0
                continue
            # the draft model: noisy copy of the target logits
            d = lf.astype(np.float64) + spec.noise_sigma * rng.standard_normal(V)
            qrow = _softmax64(d)
            if q is not None:
                q[r, j] = qrow.astype(np.float32) if req_dense else (np.nan if spec.canaries else 0.0)
            # the draft model's own sampling of the proposed token
            if spec.argmax_prob > 0 and rng.random() < spec.argmax_prob:
                y = int(np.argmax(lf))
            else:
                sp = _softmax64(d / Td)
                if spec.draft_top_k:
                    top = np.argpartition(-sp, spec.draft_top_k - 1)[: spec.draft_top_k]
                    y = int(top[_draw(rng, sp[top])])
                else:
                    y = _draw(rng, sp)
            ids[r, j] = y
        ua[r] = uniforms(rng, (G,))
        us[r] = uniforms(rng, ())

    if threads > 1 and n > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(threads, n)) as ex:
            list(ex.map(one, range(n)))
    else:
        for r in range(n):
            one(r)
    out = dict(draft_ids=ids, draft_probs=q, target_logits=logits, dtype=spec.dtype,
               temperature=T_all[idx].copy(), top_k=np.full(n, spec.top_k, np.int32),
               top_p=np.full(n, spec.top_p, np.float32), u_accept=ua, u_sample=us, has_q=has_q,
               gamma=gam_all[idx].copy())
    return out


def config(cfg: int, **overrides) -> Spec:
    """The five benchmark workloads (K about 4-5, V from 1k to 152k, batched decode)."""
    base = {
        # tiny fp32 case
        1: dict(N=4, gmax=4, V=1024, dtype="f32", logit_sigma=2.0, noise_sigma=1.0),
        # peaked bf16 rows, T = 0.8
        2: dict(N=64, gmax=4, V=32000, logit_sigma=3.0, peak=8.0, noise_sigma=1.5, temperature=0.8),
        # Zipf-biased rows with top-k 50 / top-p 0.9 on both distributions
        3: dict(N=256, gmax=5, V=128256, logit_sigma=3.0, zipf=1.1, noise_sigma=1.0, top_k=50, top_p=0.9,
                draft_top_k=50),
        # 25 % greedy requests, the rest T ~ U[0.5, 1.2]; drafts agree with the target argmax w.p. 0.7
        4: dict(N=512, gmax=8, V=151936, logit_sigma=3.0, noise_sigma=1.0, temp_range=(0.5, 1.2),
                greedy_count=128, argmax_prob=0.7),
        # ragged gamma in {0..7}, NaN canaries in padding rows, half draft-free (n-gram style)
        5: dict(N=1024, gmax=8, V=128256, logit_sigma=3.0, noise_sigma=1.0, q_mode="mixed", ragged=True,
                canaries=True),
    }[cfg]
    base.update(overrides)
    return Spec(seed=1000 + cfg, **base)


def worked_example() -> dict:
    """Two-token case: q = (0.2, 0.8), p = (0.6, 0.4) at the draft position and
    (0.3, 0.7) at the bonus position, draft token B (id 1), u = 0.7."""
    l = np.log(np.array([[[0.6, 0.4], [0.3, 0.7]]], np.float64)).astype(np.float32)
    return dict(draft_ids=np.array([[1]], np.int32), draft_probs=np.array([[[0.2, 0.8]]], np.float32),
                target_logits=l, dtype="f32", temperature=np.ones(1, np.float32),
                top_k=np.zeros(1, np.int32), top_p=np.ones(1, np.float32),
                u_accept=np.array([[0.7]], np.float32), u_sample=np.array([0.5], np.float32),
                has_q=np.ones(1, bool), gamma=np.ones(1, np.int64))


def split_by_q(batch: dict):
    """Split a mixed batch into (dense-q part, draft-free part), each a batch of
    its own with contiguous requests, for a verifier that takes one q pointer."""
    hq = batch["has_q"]
    n_dense = int(hq.sum())
    assert hq[:n_dense].all() and not hq[n_dense:].any(), "dense requests must come first"
    parts = []
    for lo, hi, dense in ((0, n_dense, True), (n_dense, len(hq), False)):
        if hi <= lo:
            continue
        p = {}
        for k, v in batch.items():
            if isinstance(v, np.ndarray) and v.shape[:1] == hq.shape:
                p[k] = v[lo:hi]
            else:
                p[k] = v
        p["draft_probs"] = batch["draft_probs"][lo:hi] if (dense and batch["draft_probs"] is not None) else None
        parts.append(p)
    return parts


def flatten(batch: dict) -> dict:
    """The same batch in the flattened (ragged) layout: no padding rows.

    Request i's drafts occupy draft_ids[cu[i-1]:cu[i]] (cu = inclusive prefix
    sums of gamma_i), its target rows are its gamma_i draft positions followed
    by its bonus position, and draft_probs holds only the draft rows of the
    requests that carry them, in request order (has_draft_probs marks those
    requests).  Pure data movement: nothing of the verifier is computed."""
    ids = batch["draft_ids"]
    N, G = ids.shape
    if "gamma" in batch:
        gam = np.asarray(batch["gamma"], np.int64)
    elif G == 0:
        gam = np.zeros(N, np.int64)
    else:
        gam = np.where((ids < 0).any(axis=1), np.argmax(ids < 0, axis=1), G).astype(np.int64)
    cu = np.cumsum(gam).astype(np.int32)
    T = int(cu[-1]) if N else 0
    V = batch["target_logits"].shape[-1]
    flat_ids = np.concatenate([ids[i, :gam[i]] for i in range(N)] + [np.zeros(0, np.int32)]).astype(np.int32)
    ua = np.concatenate([batch["u_accept"][i, :gam[i]] for i in range(N)] + [np.zeros(0, np.float32)])
    tl = batch["target_logits"]
    logits = np.empty((T + N, V), tl.dtype)
    r = 0
    for i in range(N):
        logits[r:r + gam[i] + 1] = tl[i, :gam[i] + 1]
        r += gam[i] + 1
    q = batch.get("draft_probs")
    has_q = None
    flat_q = None
    if q is not None:
        hq = np.asarray(batch.get("has_q", np.ones(N, bool)), bool)
        has_q = hq.astype(np.uint8)
        rows = [q[i, :gam[i]] for i in range(N) if hq[i]]
        flat_q = np.concatenate(rows + [np.zeros((0, V), np.float32)]).astype(np.float32)
    return dict(cu_num_draft_tokens=cu, draft_ids=flat_ids, draft_probs=flat_q, has_draft_probs=has_q,
                target_logits=logits, dtype=batch["dtype"], gmax=G, temperature=batch["temperature"],
                top_k=batch["top_k"], top_p=batch["top_p"], u_accept=ua.astype(np.float32),
                u_sample=batch["u_sample"])


def scatter_rows(flat: dict, seed: int, extra: int) -> dict:
    """The flattened batch with its target rows scattered over a larger logits
    tensor, as a target model's output holds them among rows of other
    positions: target_logits becomes [T + N + extra, V] with the rows at a
    seeded random placement and NaN in every row no index names;
    target_logits_indices [T] and bonus_logits_indices [N] give each draft and
    bonus position's row.  Pure data movement."""
    cu = np.asarray(flat["cu_num_draft_tokens"], np.int64)
    N = cu.shape[0]
    tl = flat["target_logits"]
    R0, V = tl.shape
    T = R0 - N
    R = R0 + int(extra)
    rng = np.random.default_rng(seed)
    place = rng.permutation(R)[:R0].astype(np.int32)  # row r of the ordered layout goes to place[r]
    nan = np.uint16(0x7FC0) if flat["dtype"] == "bf16" else np.float32(np.nan)
    out = np.full((R, V), nan, tl.dtype)
    out[place] = tl
    # ordered-layout row of draft t of request i is t + i; of its bonus, cu[i] + i
    req_of_t = np.searchsorted(cu, np.arange(T), side="right")
    tidx = place[np.arange(T) + req_of_t].astype(np.int32)
    bidx = place[cu + np.arange(N)].astype(np.int32) if N else np.zeros(0, np.int32)
    res = dict(flat)
    res.update(target_logits=out, target_logits_indices=tidx, bonus_logits_indices=bidx)
    return res


def penalty_lists(batch: dict, seed: int, n_ctx: int) -> list:
    """Per-position repetition-penalty lists for a padded batch: request i
    gets a context of n_ctx distinct tokens with output counts (0: prompt only,
    else geometric), and position j's list is that context plus the draft
    tokens y_0 .. y_{j-1} before it, each adding one to its count.  Every
    third request's context also holds its first draft token and the argmax
    of its first target row, so that penalties reach the tokens that decide.
    lists[i][j] = (ids ascending, counts), int32."""
    rng = np.random.default_rng(seed)
    ids = batch["draft_ids"]
    N, G = ids.shape
    tl = batch["target_logits"]
    V = tl.shape[-1]
    neg = np.concatenate([ids < 0, np.ones((N, 1), bool)], axis=1)
    gam = np.argmax(neg, axis=1)
    out = []
    for i in range(N):
        ctx = set(rng.choice(V, size=min(n_ctx, V), replace=False).tolist())
        if i % 3 == 0:
            if gam[i] > 0:
                ctx.add(int(ids[i, 0]))
            row = bf16_bits_to_f32(tl[i, 0]) if batch["dtype"] == "bf16" else tl[i, 0]
            ctx.add(int(np.argmax(row)))
        ctx = sorted(ctx)[:n_ctx]
        base = dict(zip(ctx, (rng.geometric(0.5, size=len(ctx)) - 1).tolist()))
        rows = []
        for j in range(gam[i] + 1):
            d = dict(base)
            for t in range(j):
                d[int(ids[i, t])] = d.get(int(ids[i, t]), 0) + 1
            keys = sorted(d)
            rows.append((np.array(keys, np.int32), np.array([d[k] for k in keys], np.int32)))
        out.append(rows)
    return out


def flatten_penalties(lists: list):
    """The per-position lists in the flattened layout: positions in request
    order (request i's positions 0 .. gamma_i), offsets [positions + 1], ids,
    counts.  Pure data movement."""
    rows = [r for req in lists for r in req]
    off = np.concatenate([[0], np.cumsum([len(r[0]) for r in rows])]).astype(np.int32)
    ids = np.concatenate([r[0] for r in rows] + [np.zeros(0, np.int32)]).astype(np.int32)
    cnt = np.concatenate([r[1] for r in rows] + [np.zeros(0, np.int32)]).astype(np.int32)
    return off, ids, cnt
