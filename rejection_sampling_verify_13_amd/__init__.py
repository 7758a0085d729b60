"""MI355X batched draft-verify rejection sampler.

Python binding of the C ABI in include/spec_verify.h.  It only marshals
arguments: every step of the verification runs in the HIP kernels of
``libspecverify.so``.  PyTorch supplies device memory and the stream.  There
is no fallback: if the library is not built, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

F32 = 0
BF16 = 1
STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "bad dtype", 4: "workspace too small", 5: "HIP error",
          6: "sizes exceed the static scratch"}
FAULT_DRAFT_ID = 1
FAULT_TEMPERATURE = 2
FAULT_TOP_P = 4
FAULT_TARGET_ROW = 8
FAULT_DRAFT_ROW = 16
FAULT_DRAFT_MASS = 32
FAULT_DRAFT_COUNT = 64
FAULT_BAN_LIST = 128
FAULT_ROW_INDEX = 256
FAULT_PENALTY = 512

EXPORTS = ("spec_verify", "spec_verify_diag", "spec_verify_timed", "spec_verify_flat", "spec_verify_flat_timed",
           "spec_verify_flat_synthetic", "spec_verify_flat_ex", "spec_verify_rollback", "spec_verify_device_errors",
           "spec_verify_static", "spec_verify_static_scratch_bytes", "spec_verify_workspace_size",
           "spec_verify_status_string", "spec_verify_version")


class SpecVerifyError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libspecverify.so is not built (%s); run __graft_entry__.build() or "
            "python rejection_sampling_verify_13_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.spec_verify.restype = I
    lib.spec_verify.argtypes = [I, I, I, P, P, P, I, P, P, P, P, P, P, P, P, Z, P]
    lib.spec_verify_diag.restype = I
    lib.spec_verify_diag.argtypes = [I, I, I, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.spec_verify_timed.restype = I
    lib.spec_verify_timed.argtypes = [I, I, I, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P, Z, P, P, P, P]
    lib.spec_verify_flat.restype = I
    lib.spec_verify_flat.argtypes = [I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P, Z, P]
    lib.spec_verify_flat_timed.restype = I
    lib.spec_verify_flat_timed.argtypes = [I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P, P, P, Z, P,
                                           P, P, P]
    lib.spec_verify_flat_synthetic.restype = I
    lib.spec_verify_flat_synthetic.argtypes = [I, I, I, I, P, P, P, P, P, I, P, P, P, P, P, P, P, P, P, P, Z, P,
                                               P, P, P]
    lib.spec_verify_flat_ex.restype = I
    lib.spec_verify_flat_ex.argtypes = ([I, I, I, I] + [P] * 5 + [I, P, P, I] + [P] * 3 + [P, P] + [P] * 6 +
                                        [P] * 4 + [P] * 4 + [P, Z, P] + [P] * 3)
    lib.spec_verify_rollback.restype = I
    lib.spec_verify_rollback.argtypes = [I, I, P, P, P, P, P, P, P]
    lib.spec_verify_workspace_size.restype = Z
    lib.spec_verify_workspace_size.argtypes = [I, I, I]
    lib.spec_verify_device_errors.restype = I
    lib.spec_verify_device_errors.argtypes = [P, Z, P, P]
    lib.spec_verify_static.restype = I
    lib.spec_verify_static.argtypes = [I, I, I, P, P, P, I, P, P, P, P, P, P, P, P]
    lib.spec_verify_static_scratch_bytes.restype = Z
    lib.spec_verify_static_scratch_bytes.argtypes = []
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [I]
    lib.spec_verify_version.restype = I
    lib.spec_verify_version.argtypes = []
    return lib


lib = _load()


def workspace_size(N: int, gmax: int, V: int) -> int:
    return int(lib.spec_verify_workspace_size(N, gmax, V))


def device_errors(workspace, stream=None) -> int:
    """Number of requests the most recent call on ``workspace`` (a uint8 CUDA
    tensor passed to that call) reported as faulted; waits for ``stream``
    (default: torch's current stream on the workspace's device)."""
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device)
    n = ctypes.c_int32(-1)
    with torch.cuda.device(workspace.device):
        rc = lib.spec_verify_device_errors(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           ctypes.c_void_p(stream.cuda_stream), ctypes.byref(n))
    if rc != 0:
        raise SpecVerifyError("spec_verify_device_errors: %s" % STATUS.get(rc, rc))
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def verify(draft_ids, draft_probs, target_logits, temperature=None, top_k=None, top_p=None, u_accept=None,
           u_sample=None, *, out_tokens=None, out_num_accepted=None, workspace=None, stream=None, diag=False,
           events=None, static=False):
    """Verify a batch on the GPU.

    draft_ids int32 [N, gmax] (-1 padded), draft_probs float32 [N, gmax, V] or
    None, target_logits bfloat16/float32 [N, gmax+1, V], temperature float32
    [N] or None, top_k int32 [N] or None, top_p float32 [N] or None, u_accept
    float32 [N, gmax], u_sample float32 [N]; all on one CUDA (HIP) device.
    Returns (out_tokens int32 [N, gmax+1], out_num_accepted int32 [N]) and,
    with diag=True, a dict of p_y, q_y [N, gmax] float64, resid_mass [N]
    float64 and fault [N] int32.  The work is enqueued on ``stream`` (default:
    torch's current stream); nothing synchronises.  ``events`` = (start, mid,
    end) torch.cuda.Event objects (or None) are recorded on the stream before
    the row pass, between the two kernels and after the finish kernel.  With
    static=True the call goes to spec_verify_static, which uses the library's
    own device scratch array instead of a workspace and allocates nothing
    (the outputs must then be passed in for no allocation at all).
    """
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [N, gmax+1, V]")
    N, G1, V = target_logits.shape
    G = G1 - 1
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = BF16
    elif target_logits.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError("target_logits must be bfloat16 or float32")
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _check(draft_ids, "draft_ids", torch.int32, (N, G), dev)
    _check(draft_probs, "draft_probs", torch.float32, (N, G, V), dev)
    _check(temperature, "temperature", torch.float32, (N,), dev)
    _check(top_k, "top_k", torch.int32, (N,), dev)
    _check(top_p, "top_p", torch.float32, (N,), dev)
    _check(u_accept, "u_accept", torch.float32, (N, G), dev)
    _check(u_sample, "u_sample", torch.float32, (N,), dev)
    if out_tokens is None:
        out_tokens = torch.empty((N, G + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((N,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", torch.int32, (N, G + 1), dev)
    _check(out_num_accepted, "out_num_accepted", torch.int32, (N,), dev)
    if static and (workspace is not None or diag or events is not None):
        raise ValueError("static=True takes no workspace, diag or events")
    if workspace is None and not static:
        workspace = torch.empty((workspace_size(N, G, V),), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if static else workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    with torch.cuda.device(dev):
        if static:
            rc = lib.spec_verify_static(N, G, V, _ptr(draft_ids), _ptr(draft_probs), _ptr(target_logits), dt,
                                        _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept),
                                        _ptr(u_sample), _ptr(out_tokens), _ptr(out_num_accepted), sptr)
        elif events is not None:
            evp = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in events]
            rc = lib.spec_verify_timed(N, G, V, _ptr(draft_ids), _ptr(draft_probs), _ptr(target_logits), dt,
                                       _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept), _ptr(u_sample),
                                       _ptr(out_tokens), _ptr(out_num_accepted), None, None, None, None,
                                       _ptr(workspace), ws_bytes, sptr, *evp)
        elif diag:
            d = dict(p_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                     q_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                     resid_mass=torch.empty((N,), dtype=torch.float64, device=dev),
                     fault=torch.empty((N,), dtype=torch.int32, device=dev))
            rc = lib.spec_verify_diag(N, G, V, _ptr(draft_ids), _ptr(draft_probs), _ptr(target_logits), dt,
                                      _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept), _ptr(u_sample),
                                      _ptr(out_tokens), _ptr(out_num_accepted), _ptr(d["p_y"]), _ptr(d["q_y"]),
                                      _ptr(d["resid_mass"]), _ptr(d["fault"]), _ptr(workspace), ws_bytes, sptr)
        else:
            rc = lib.spec_verify(N, G, V, _ptr(draft_ids), _ptr(draft_probs), _ptr(target_logits), dt,
                                 _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept), _ptr(u_sample),
                                 _ptr(out_tokens), _ptr(out_num_accepted), _ptr(workspace), ws_bytes, sptr)
    if rc != 0:
        raise SpecVerifyError("spec_verify failed: %s" % lib.spec_verify_status_string(rc).decode())
    if diag:
        return out_tokens, out_num_accepted, d
    return out_tokens, out_num_accepted


def verify_flat(cu_num_draft_tokens, draft_ids, draft_probs, has_draft_probs, target_logits, gmax,
                temperature=None, top_k=None, top_p=None, u_accept=None, u_sample=None, *, out_tokens=None,
                out_num_accepted=None, workspace=None, stream=None, diag=False, events=None, synthetic_rates=None,
                banned_offsets=None, banned_ids=None, target_logits_indices=None, bonus_logits_indices=None,
                penalty_offsets=None, penalty_ids=None, penalty_counts=None, repetition_penalty=None,
                presence_penalty=None, frequency_penalty=None):
    """Verify a batch in the flattened layout (spec_verify_flat in include/spec_verify.h).

    cu_num_draft_tokens int32 [N] (inclusive prefix sums of the draft counts),
    draft_ids int32 [T], draft_probs float32 [Q, V] or None (the draft rows of
    the requests that carry them, in request order), has_draft_probs uint8 [N]
    or None, target_logits bfloat16/float32 [T + N, V] (each request's draft
    positions, then its bonus position), gmax (the output width is gmax + 1),
    temperature / top_k / top_p / u_sample [N] as for verify(), u_accept
    float32 [T].  Returns what verify() returns; with diag=True p_y and q_y
    are [N, gmax].  ``events`` as for verify().  With ``synthetic_rates``
    (float32 [gmax]) the synthetic acceptance mode runs (spec_verify_flat_synthetic):
    draft j is accepted iff u_accept < rate_j; diag then returns only ``fault``.
    With ``banned_offsets`` (int32 [N + 1]) and ``banned_ids`` (int32, ascending
    per request) those tokens are banned in p and q alike.  With
    ``target_logits_indices`` (int32 [T]) and ``bonus_logits_indices`` (int32
    [N]) target_logits is any [R, V] tensor and those indices name the row of
    each draft and bonus position.  With ``penalty_offsets`` (int32 [T + N + 1],
    one list per position in request order), ``penalty_ids`` / ``penalty_counts``
    (int32) and the optional per-request ``repetition_penalty``,
    ``presence_penalty`` and ``frequency_penalty`` (float32 [N]) the
    penalties apply to p and q alike.  Any option runs spec_verify_flat_ex.
    """
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [T + N, V] (or [R, V] with row indices)")
    N = cu_num_draft_tokens.shape[0]
    G = int(gmax)
    R, V = target_logits.shape
    indexed = target_logits_indices is not None or bonus_logits_indices is not None
    if indexed:
        if draft_ids is None or draft_ids.dim() != 1:
            raise ValueError("draft_ids must be a 1-d int32 tensor")
        T = draft_ids.shape[0]
    else:
        T = R - N
        if T < 0:
            raise ValueError("target_logits has fewer rows than requests")
    dev = target_logits.device
    if target_logits.dtype == torch.bfloat16:
        dt = BF16
    elif target_logits.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError("target_logits must be bfloat16 or float32")
    if not target_logits.is_contiguous():
        raise ValueError("target_logits must be contiguous")
    _check(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, (N,), dev)
    _check(draft_ids, "draft_ids", torch.int32, (T,), dev)
    if draft_probs is not None:
        if draft_probs.dim() != 2 or draft_probs.shape[1] != V:
            raise ValueError("draft_probs must be [Q, V]")
        _check(draft_probs, "draft_probs", torch.float32, tuple(draft_probs.shape), dev)
    _check(has_draft_probs, "has_draft_probs", torch.uint8, (N,), dev)
    _check(temperature, "temperature", torch.float32, (N,), dev)
    _check(top_k, "top_k", torch.int32, (N,), dev)
    _check(top_p, "top_p", torch.float32, (N,), dev)
    _check(u_accept, "u_accept", torch.float32, (T,), dev)
    _check(u_sample, "u_sample", torch.float32, (N,), dev)
    if out_tokens is None:
        out_tokens = torch.empty((N, G + 1), dtype=torch.int32, device=dev)
    if out_num_accepted is None:
        out_num_accepted = torch.empty((N,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", torch.int32, (N, G + 1), dev)
    _check(out_num_accepted, "out_num_accepted", torch.int32, (N,), dev)
    if workspace is None:
        workspace = torch.empty((workspace_size(N, G, V),), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    head = (N, G, V, T, _ptr(cu_num_draft_tokens), _ptr(draft_ids), _ptr(draft_probs), _ptr(has_draft_probs),
            _ptr(target_logits), dt, _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(u_accept), _ptr(u_sample),
            _ptr(out_tokens), _ptr(out_num_accepted))
    d = None
    if synthetic_rates is not None:
        _check(synthetic_rates, "synthetic_rates", torch.float32, (G,), dev)
        if diag:
            d = dict(fault=torch.empty((N,), dtype=torch.int32, device=dev))
        evp = (None, None, None) if events is None else tuple(
            None if e is None else ctypes.c_void_p(e.cuda_event) for e in events)
        with torch.cuda.device(dev):
            rc = lib.spec_verify_flat_synthetic(*head[:13], _ptr(synthetic_rates), *head[13:],
                                                _ptr(d["fault"]) if diag else None, _ptr(workspace), ws_bytes, sptr,
                                                *evp)
        if rc != 0:
            raise SpecVerifyError("spec_verify_flat_synthetic failed: %s" % lib.spec_verify_status_string(rc).decode())
        return (out_tokens, out_num_accepted, d) if diag else (out_tokens, out_num_accepted)
    pen_args = (penalty_offsets, penalty_ids, penalty_counts, repetition_penalty, presence_penalty, frequency_penalty)
    penalised = any(x is not None for x in pen_args)
    if banned_offsets is not None or banned_ids is not None or indexed or penalised:
        if banned_offsets is not None or banned_ids is not None:
            _check(banned_offsets, "banned_offsets", torch.int32, (N + 1,), dev)
            if banned_ids is not None:  # None: every list is empty
                if banned_ids.dim() != 1:
                    raise ValueError("banned_ids must be a 1-d int32 tensor")
                _check(banned_ids, "banned_ids", torch.int32, tuple(banned_ids.shape), dev)
        if indexed:
            _check(target_logits_indices, "target_logits_indices", torch.int32, (T,), dev)
            _check(bonus_logits_indices, "bonus_logits_indices", torch.int32, (N,), dev)
        if penalised:
            _check(penalty_offsets, "penalty_offsets", torch.int32, (T + N + 1,), dev)
            for name, t in (("penalty_ids", penalty_ids), ("penalty_counts", penalty_counts)):
                if t is not None and t.dim() != 1:
                    raise ValueError("%s must be a 1-d int32 tensor" % name)
                _check(t, name, torch.int32, None if t is None else tuple(t.shape), dev)
            if penalty_ids is not None and penalty_counts is not None and penalty_ids.shape != penalty_counts.shape:
                raise ValueError("penalty_ids and penalty_counts must have the same length")
            for name, t in (("repetition_penalty", repetition_penalty), ("presence_penalty", presence_penalty),
                            ("frequency_penalty", frequency_penalty)):
                _check(t, name, torch.float32, (N,), dev)
        if diag:
            d = dict(p_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                     q_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                     resid_mass=torch.empty((N,), dtype=torch.float64, device=dev),
                     fault=torch.empty((N,), dtype=torch.int32, device=dev))
            dp = (_ptr(d["p_y"]), _ptr(d["q_y"]), _ptr(d["resid_mass"]), _ptr(d["fault"]))
        else:
            dp = (None, None, None, None)
        evp = (None, None, None) if events is None else tuple(
            None if e is None else ctypes.c_void_p(e.cuda_event) for e in events)
        with torch.cuda.device(dev):
            rc = lib.spec_verify_flat_ex(*head[:9], R, _ptr(target_logits_indices), _ptr(bonus_logits_indices),
                                         *head[9:13], _ptr(banned_offsets), _ptr(banned_ids),
                                         *[_ptr(x) for x in pen_args], *head[13:], *dp,
                                         _ptr(workspace), ws_bytes, sptr, *evp)
        if rc != 0:
            raise SpecVerifyError("spec_verify_flat_ex failed: %s" % lib.spec_verify_status_string(rc).decode())
        return (out_tokens, out_num_accepted, d) if diag else (out_tokens, out_num_accepted)
    with torch.cuda.device(dev):
        if diag or events is not None:
            if diag:
                d = dict(p_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                         q_y=torch.empty((N, G), dtype=torch.float64, device=dev),
                         resid_mass=torch.empty((N,), dtype=torch.float64, device=dev),
                         fault=torch.empty((N,), dtype=torch.int32, device=dev))
                dp = (_ptr(d["p_y"]), _ptr(d["q_y"]), _ptr(d["resid_mass"]), _ptr(d["fault"]))
            else:
                dp = (None, None, None, None)
            evp = (None, None, None) if events is None else tuple(
                None if e is None else ctypes.c_void_p(e.cuda_event) for e in events)
            rc = lib.spec_verify_flat_timed(*head, *dp, _ptr(workspace), ws_bytes, sptr, *evp)
        else:
            rc = lib.spec_verify_flat(*head, _ptr(workspace), ws_bytes, sptr)
    if rc != 0:
        raise SpecVerifyError("spec_verify_flat failed: %s" % lib.spec_verify_status_string(rc).decode())
    if diag:
        return out_tokens, out_num_accepted, d
    return out_tokens, out_num_accepted


def to_device(batch: dict, device="cuda"):
    """Move a numpy batch (the layout of the workloads module) to torch tensors."""
    import numpy as np
    out = {}
    for k in ("draft_ids", "draft_probs", "temperature", "top_k", "top_p", "u_accept", "u_sample"):
        v = batch.get(k)
        out[k] = None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(device)
    tl = batch["target_logits"]
    if batch["dtype"] == "bf16":
        out["target_logits"] = torch.from_numpy(np.ascontiguousarray(tl).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        out["target_logits"] = torch.from_numpy(np.ascontiguousarray(tl)).to(device)
    return out


class Prepared:
    """A padded-layout verify call bound once to its buffers.

    The arguments are those of verify() (outputs, workspace and stream
    allocated or taken as there) and are checked and marshalled here, once;
    each call then makes one C call, spec_verify (spec_verify_timed with
    ``events``), with no checks or allocations on the host.  For loops that
    refill the same input buffers in place every step.  The tensors must stay
    alive and in place while the object is used, and calls are made with
    their device current (one GPU per process)."""

    def __init__(self, draft_ids, draft_probs, target_logits, temperature=None, top_k=None, top_p=None,
                 u_accept=None, u_sample=None, *, out_tokens=None, out_num_accepted=None, workspace=None,
                 stream=None):
        if target_logits.dim() != 3 or not target_logits.is_contiguous():
            raise ValueError("target_logits must be a contiguous [N, gmax+1, V] tensor")
        N, G1, V = target_logits.shape
        G = G1 - 1
        dev = target_logits.device
        if target_logits.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("target_logits must be bfloat16 or float32")
        dt = BF16 if target_logits.dtype == torch.bfloat16 else F32
        _check(draft_ids, "draft_ids", torch.int32, (N, G), dev)
        _check(draft_probs, "draft_probs", torch.float32, (N, G, V), dev)
        _check(temperature, "temperature", torch.float32, (N,), dev)
        _check(top_k, "top_k", torch.int32, (N,), dev)
        _check(top_p, "top_p", torch.float32, (N,), dev)
        _check(u_accept, "u_accept", torch.float32, (N, G), dev)
        _check(u_sample, "u_sample", torch.float32, (N,), dev)
        if out_tokens is None:
            out_tokens = torch.empty((N, G + 1), dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty((N,), dtype=torch.int32, device=dev)
        _check(out_tokens, "out_tokens", torch.int32, (N, G + 1), dev)
        _check(out_num_accepted, "out_num_accepted", torch.int32, (N,), dev)
        if workspace is None:
            workspace = torch.empty((workspace_size(N, G, V),), dtype=torch.uint8, device=dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        self.out_tokens, self.out_num_accepted = out_tokens, out_num_accepted
        self._keep = (draft_ids, draft_probs, target_logits, temperature, top_k, top_p, u_accept, u_sample,
                      workspace, stream)
        self._head = (N, G, V, _ptr(draft_ids), _ptr(draft_probs), _ptr(target_logits), dt, _ptr(temperature),
                      _ptr(top_k), _ptr(top_p), _ptr(u_accept), _ptr(u_sample), _ptr(out_tokens),
                      _ptr(out_num_accepted))
        self._tail = (_ptr(workspace), workspace.numel() * workspace.element_size(),
                      ctypes.c_void_p(stream.cuda_stream))

    def __call__(self, events=None):
        """Enqueue the call; ``events`` = (start, mid, end) as for verify()."""
        if events is None:
            rc = lib.spec_verify(*self._head, *self._tail)
        else:
            evp = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in events]
            rc = lib.spec_verify_timed(*self._head, None, None, None, None, *self._tail, *evp)
        if rc != 0:
            raise SpecVerifyError("spec_verify failed: %s" % lib.spec_verify_status_string(rc).decode())
        return self.out_tokens, self.out_num_accepted


def verify_batch(dev_batch: dict, **kw):
    """verify() with the arguments taken from a to_device() dict."""
    return verify(dev_batch["draft_ids"], dev_batch["draft_probs"], dev_batch["target_logits"],
                  dev_batch["temperature"], dev_batch["top_k"], dev_batch["top_p"], dev_batch["u_accept"],
                  dev_batch["u_sample"], **kw)


def to_device_flat(flat: dict, device="cuda"):
    """Move a flattened numpy batch (workloads.flatten) to torch tensors."""
    import numpy as np
    out = {"gmax": flat["gmax"]}
    for k in ("cu_num_draft_tokens", "draft_ids", "draft_probs", "has_draft_probs", "temperature", "top_k",
              "top_p", "u_accept", "u_sample", "target_logits_indices", "bonus_logits_indices",
              "penalty_offsets", "penalty_ids", "penalty_counts", "repetition_penalty", "presence_penalty",
              "frequency_penalty"):
        v = flat.get(k)
        out[k] = None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(device)
    tl = flat["target_logits"]
    if flat["dtype"] == "bf16":
        out["target_logits"] = torch.from_numpy(np.ascontiguousarray(tl).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        out["target_logits"] = torch.from_numpy(np.ascontiguousarray(tl)).to(device)
    return out


def verify_flat_batch(dev_flat: dict, **kw):
    """verify_flat() with the arguments taken from a to_device_flat() dict."""
    return verify_flat(dev_flat["cu_num_draft_tokens"], dev_flat["draft_ids"], dev_flat["draft_probs"],
                       dev_flat["has_draft_probs"], dev_flat["target_logits"], dev_flat["gmax"],
                       dev_flat["temperature"], dev_flat["top_k"], dev_flat["top_p"], dev_flat["u_accept"],
                       dev_flat["u_sample"], **dict({k: dev_flat.get(k) for k in _FLAT_OPTIONS}, **kw))


_FLAT_OPTIONS = ("target_logits_indices", "bonus_logits_indices", "penalty_offsets", "penalty_ids", "penalty_counts",
                 "repetition_penalty", "presence_penalty", "frequency_penalty")


def rollback(num_accepted, *, cu_num_draft_tokens=None, draft_ids=None, gmax=None, num_computed_tokens=None,
             num_output_placeholders=None, slot_mapping=None, stream=None):
    """KV bookkeeping after a verify call (spec_verify_rollback in include/spec_verify.h).

    Give the draft counts as cu_num_draft_tokens int32 [N] (flattened layout,
    slot_mapping [T]) or draft_ids int32 [N, gmax] (padded, slot_mapping
    [N, gmax]).  num_computed_tokens, num_output_placeholders (int32 [N]) and
    slot_mapping are updated in place on ``stream``; each may be None."""
    N = num_accepted.shape[0]
    dev = num_accepted.device
    _check(num_accepted, "num_accepted", torch.int32, (N,), dev)
    if (cu_num_draft_tokens is None) == (draft_ids is None):
        raise ValueError("give exactly one of cu_num_draft_tokens and draft_ids")
    if draft_ids is not None:
        G = draft_ids.shape[1]
        _check(draft_ids, "draft_ids", torch.int32, (N, G), dev)
        if slot_mapping is not None:
            _check(slot_mapping, "slot_mapping", torch.int32, (N, G), dev)
    else:
        if gmax is None:
            raise ValueError("gmax is required with cu_num_draft_tokens")
        G = int(gmax)
        _check(cu_num_draft_tokens, "cu_num_draft_tokens", torch.int32, (N,), dev)
        if slot_mapping is not None:
            _check(slot_mapping, "slot_mapping", torch.int32, tuple(slot_mapping.shape), dev)
            if slot_mapping.dim() != 1:
                raise ValueError("slot_mapping must be [T] in the flattened layout")
    _check(num_computed_tokens, "num_computed_tokens", torch.int32, (N,), dev)
    _check(num_output_placeholders, "num_output_placeholders", torch.int32, (N,), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = lib.spec_verify_rollback(N, G, _ptr(cu_num_draft_tokens), _ptr(draft_ids), _ptr(num_accepted),
                                      _ptr(num_computed_tokens), _ptr(num_output_placeholders), _ptr(slot_mapping),
                                      ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecVerifyError("spec_verify_rollback failed: %s" % lib.spec_verify_status_string(rc).decode())
