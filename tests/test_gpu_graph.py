"""A verify call captured in a HIP graph (the padded drafter batch of the vLLM
page exists so that the decode step can be captured): with the workspace and
outputs passed in, a call allocates nothing and launches only kernels, so it
can be captured once and replayed on new inputs copied into the same buffers.
Each replay, with eager work and synchronisations in between, must equal an
eager call on the same inputs, bit for bit."""
import numpy as np
import pytest

import workloads as W
from parity import log

pytestmark = pytest.mark.gpu


def _batches(cfg_kw, n):
    base = W.config(**cfg_kw)
    return [W.generate(W.Spec(**{**base.__dict__, "seed": base.seed + 17 * s})) for s in range(n)]


@pytest.mark.parametrize("cfg_kw", [dict(cfg=3, N=16, V=12000), dict(cfg=4, N=24, V=7000, greedy_count=6),
                                    dict(cfg=2, N=12, V=4999)])
def test_graph_replays_equal_eager_calls(cfg_kw):
    import torch
    import rejection_sampling_verify_13_amd as sv
    batches = _batches(cfg_kw, 4)
    devs = [sv.to_device(b, "cuda") for b in batches]
    d = {k: (None if v is None else v.clone()) for k, v in devs[0].items()}
    N, G = d["draft_ids"].shape
    V = d["target_logits"].shape[-1]
    ws = torch.empty(sv.workspace_size(N, G, V), dtype=torch.uint8, device="cuda")
    out_t = torch.empty((N, G + 1), dtype=torch.int32, device="cuda")
    out_n = torch.empty((N,), dtype=torch.int32, device="cuda")
    log("[graph] capture, %s" % cfg_kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's pool, as torch asks
        sv.verify_batch(d, out_tokens=out_t, out_num_accepted=out_n, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sv.verify_batch(d, out_tokens=out_t, out_num_accepted=out_n, workspace=ws)
    torch.cuda.synchronize()
    for r, src in enumerate(devs[1:] + devs[:1]):
        for k, v in src.items():
            if v is not None:
                d[k].copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_t, got_n = out_t.clone(), out_n.clone()
        want_t, want_n = sv.verify_batch(src)  # eager, its own workspace and outputs
        torch.cuda.synchronize()
        log("[graph] replay %d: %d requests, %d accepted drafts" % (r, N, int(want_n.clamp(min=0).sum())))
        assert torch.equal(got_t, want_t) and torch.equal(got_n, want_n), "replay %d differs" % r
