"""The timed entry points: the row pass's start and end events travel in its
own dispatch and the third event follows the draw pass.  Timing must not
change a result: tokens and counts equal those of the same call without
events, bit for bit, in both layouts, and the recorded intervals are
positive."""
import pytest

import workloads as W
from parity import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg_kw,flat", [(dict(cfg=3, N=16, V=12000), False), (dict(cfg=3, N=16, V=12000), True),
                                         (dict(cfg=4, N=24, V=7000, greedy_count=6), False),
                                         (dict(cfg=5, N=40, V=6144), True)])
def test_events_leave_results_unchanged(cfg_kw, flat):
    import torch
    import rejection_sampling_verify_13_amd as sv
    b = W.generate(W.config(**cfg_kw), threads=8)
    if flat:
        d = sv.to_device_flat(W.flatten(b), "cuda")
        run = sv.verify_flat_batch
    else:
        d = sv.to_device(b, "cuda")
        run = sv.verify_batch
    log("[timed] %s flat=%s" % (cfg_kw, flat))
    want_t, want_n = run(d)
    evs = tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
    stream = torch.cuda.current_stream()
    for e in evs:  # torch creates an event's handle on its first record
        e.record(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        got_t, got_n = run(d, events=evs, stream=stream)
        torch.cuda.synchronize()
        row_ms, draw_ms = evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])
        log("[timed] call %d: row pass %.1f us, draw pass %.1f us" % (rep, row_ms * 1e3, draw_ms * 1e3))
        assert torch.equal(got_t, want_t) and torch.equal(got_n, want_n)
        assert row_ms > 0.0 and draw_ms >= 0.0
