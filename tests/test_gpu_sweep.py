"""A seeded random sweep: many small configurations drawn from the five
workloads (V from 3 to 12000, ragged and empty draft lengths, top-k across
the candidate path's limit, top-p, temperatures down to 0.05, greedy mixes,
both layouts), each compared request by request with the oracle under the
parity bar.  The allowance for ambiguous requests is lifted: a batch of a few
requests cannot hold it, and ambiguous requests are excluded from the
comparison anyway."""
import json

import numpy as np
import pytest

import workloads as W
from parity import compare, gpu_run, gpu_run_flat, log, oracle_run

pytestmark = pytest.mark.gpu


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        cfg = int(rng.choice([1, 2, 3, 4, 5]))
        V = int(rng.choice([3, 17, 255, 1024, 3001, 4096, 8000, 12000]))
        N = int(rng.integers(1, 40))
        kw = dict(N=N, V=V, gmax=int(rng.choice([0, 1, 2, 5, 8])))
        if cfg in (2, 3):
            kw["top_k"] = int(rng.choice([0, 1, 5, 50, 64, 65, 300]))
            kw["top_p"] = float(rng.choice([1.0, 0.9, 0.5, 0.99]))
            kw["temperature"] = float(rng.choice([1.0, 0.7, 1.5, 0.05, 0.1, 0.25]))
        if cfg == 3:
            kw["draft_top_k"] = 0
        if cfg == 4:
            kw["greedy_count"] = int(rng.integers(0, N + 1))
        kw["dtype"] = str(rng.choice(["bf16", "f32"])) if cfg != 1 else "f32"
        flat = bool(rng.integers(0, 2))
        case_seed = int(rng.integers(1, 1 << 30))
        if cfg == 5 and V < 64:
            continue
        out.append((cfg, kw, case_seed, flat))
    return out


def test_random_sweep():
    fails = []
    done = 0
    for cfg, kw, seed, flat in _cases(20240, 600):
        b = W.generate(W.Spec(**{**W.config(cfg, **kw).__dict__, "seed": seed}))
        label = json.dumps(dict(cfg=cfg, kw=kw, seed=seed, flat=flat))
        try:
            g = gpu_run_flat(b) if flat else gpu_run(b)
            compare(g, oracle_run(b), rows=10 ** 9, label="sweep")
        except AssertionError as e:
            fails.append("%s: %s" % (label, str(e)[:200]))
        done += 1
        if done % 100 == 0:
            log("[sweep] %d cases, %d failures" % (done, len(fails)))
    log("[sweep] %d cases, %d failures" % (done, len(fails)))
    assert done == 600 and not fails, "\n".join(fails[:10])
