"""The bound call (Prepared): the same outputs as verify() on the same
buffers, with and without timing events, on calls repeated in place."""
import numpy as np
import pytest

import workloads as W
from parity import log

pytestmark = pytest.mark.gpu


def test_prepared_call_matches_verify():
    import torch
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(3, N=24, V=5000))
    d = sv.to_device(b)
    log("[prepared] N=24 gamma=5 V=5000")
    t0, n0 = sv.verify_batch(d)
    call = sv.Prepared(d["draft_ids"], d["draft_probs"], d["target_logits"], d["temperature"], d["top_k"],
                       d["top_p"], d["u_accept"], d["u_sample"])
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), None)
    for e in ev[:2]:
        e.record()
    for events in (None, ev, None):
        t1, n1 = call(events)
        torch.cuda.synchronize()
        assert np.array_equal(t1.cpu().numpy(), t0.cpu().numpy())
        assert np.array_equal(n1.cpu().numpy(), n0.cpu().numpy())
    assert ev[0].elapsed_time(ev[1]) > 0.0
    # inputs refilled in place: the bound call sees the new values
    d["u_accept"].fill_(0.0)  # every draft with p'(y) > 0 is accepted
    t2, n2 = call()
    t3, n3 = sv.verify_batch(d)
    torch.cuda.synchronize()
    assert np.array_equal(t2.cpu().numpy(), t3.cpu().numpy()) and np.array_equal(n2.cpu().numpy(), n3.cpu().numpy())
