"""The entry point that allocates nothing (spec_verify_static, for callers
that cannot allocate: HIP graph capture, allocation-free serving loops)
against spec_verify with a caller workspace: two calls in a row through the C
ABI, the second with a smaller batch, each bit-exact with spec_verify on the
same inputs (the same kernels run on the library's scratch array instead of
the caller's workspace) and with the oracle by the parity rules."""
import ctypes

import pytest

from parity import check_layout, compare, log, oracle_run

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402


def _run_static(sv, d, out_t, out_n):
    import torch
    N, G1, V = d["target_logits"].shape
    dt = sv.BF16 if d["target_logits"].dtype == torch.bfloat16 else sv.F32
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return sv.lib.spec_verify_static(N, G1 - 1, V, p(d["draft_ids"]), p(d["draft_probs"]), p(d["target_logits"]), dt,
                                     p(d["temperature"]), p(d["top_k"]), p(d["top_p"]), p(d["u_accept"]),
                                     p(d["u_sample"]), p(out_t), p(out_n), s)


@pytest.mark.parametrize("specs", [
    (W.config(3, N=48, V=12000), W.config(3, N=9, V=3001, dtype="f32")),
    (W.config(4, N=40, V=20000, greedy_count=10), W.config(2, N=6, V=5000, temperature=0.1)),
], ids=["topk_then_smaller_unaligned", "mixed_then_smaller_low_temperature"])
def test_static_entry_point_matches_workspace_entry_point(specs):
    import torch
    import rejection_sampling_verify_13_amd as sv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert sv.lib.spec_verify_static_scratch_bytes() == 16 << 20
    for k, spec in enumerate(specs):
        b = W.generate(spec, threads=8)
        N, G = b["draft_ids"].shape
        log("[static] call %d: N=%d gmax=%d V=%d %s" % (k, N, G, spec.V, spec.dtype))
        d = sv.to_device(b)
        ref_t, ref_n = sv.verify_batch(d)
        out_t = torch.full((N, G + 1), -7, dtype=torch.int32, device="cuda")
        out_n = torch.full((N,), -7, dtype=torch.int32, device="cuda")
        assert _run_static(sv, d, out_t, out_n) == 0
        torch.cuda.synchronize()
        assert torch.equal(out_t, ref_t) and torch.equal(out_n, ref_n)
        g = dict(tokens=out_t.cpu().numpy(), num_accepted=out_n.cpu().numpy())
        o = oracle_run(b, threads=8)
        res = compare(g, o, label="static call %d" % k)
        check_layout(b, g)
        log("[static] call %d ok %s" % (k, res))


def test_static_entry_point_refuses_sizes_beyond_its_scratch():
    import torch
    import rejection_sampling_verify_13_amd as sv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big_n = 8192
    assert sv.lib.spec_verify_workspace_size(big_n, 8, 151936) > sv.lib.spec_verify_static_scratch_bytes()
    P = ctypes.c_void_p(0x1000)  # never dereferenced: the size check comes first
    rc = sv.lib.spec_verify_static(big_n, 8, 151936, P, P, P, 1, None, None, None, P, P, P, P, None)
    assert rc == 6
