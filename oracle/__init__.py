"""fp64 CPU oracle for batched draft-verify rejection sampling.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library never loads it, and it imports nothing from the product package.

The arithmetic lives in ``spec_verify_oracle.c`` (plain C, fp64, single
threaded); this module compiles it with gcc and marshals numpy arrays.  Three
parts are written out here in plain Python instead: ``rollback``, the integer
KV bookkeeping after a verify call, and the two token-list transforms that
``run`` applies to its inputs before calling the C routine (banned tokens, and
the repetition penalties of ``penalty_deltas`` / ``penalize_logits``).
``run(..., threads=n)`` splits the batch into contiguous request ranges and
calls the C routine on each range from a thread pool: requests are independent,
so the result does not depend on ``n``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_verify_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# fault bits (same meaning as the OF_* constants of the C source)
FAULT_DRAFT_ID = 1
FAULT_TEMPERATURE = 2
FAULT_TOP_P = 4
FAULT_TARGET_ROW = 8
FAULT_DRAFT_ROW = 16
FAULT_DRAFT_MASS = 32
FAULT_BAN_LIST = 128
TOL = 1e-6  # decisions within it of their boundary may go either way
AMB_ACCEPT = 1
AMB_TOP_P = 2
AMB_CDF = 4
FAULT_PENALTY = 512
BAN_MAX = 512
PEN_MAX = 1024


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    global _lib
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.oracle_spec_verify.restype = ctypes.c_int
    lib.oracle_spec_verify.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int] + [P] * 2 + \
        [P, ctypes.c_int] + [P] * 12 + [P] * 8
    lib.oracle_spec_verify_synthetic.restype = ctypes.c_int
    lib.oracle_spec_verify_synthetic.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int] + [P] * 2 + \
        [P, ctypes.c_int] + [P] * 11 + [P] * 8
    lib.oracle_target_probs.restype = ctypes.c_int
    lib.oracle_target_probs.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                        ctypes.c_double, P, P]
    lib.oracle_draft_probs.restype = ctypes.c_int
    lib.oracle_draft_probs.argtypes = [ctypes.c_int, P, ctypes.c_double, ctypes.c_int, ctypes.c_double, P, P]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def run(draft_ids, draft_probs, target_logits, dtype, temperature=None, top_k=None, top_p=None,
        u_accept=None, u_sample=None, threads: int = 1, _lib_override=None, synthetic_rates=None,
        banned=None, penalties=None) -> dict:
    """Verify a batch on the CPU.

    ``dtype`` is "f32" (``target_logits`` float32) or "bf16" (``target_logits``
    uint16 bit patterns).  Returns a dict with tokens [N,gmax+1], num_accepted
    [N], p_y / q_y [N,gmax] (NaN where not computed), resid_mass [N], margin [N]
    and fault [N], and per row (zwjcode.cn page, section 14: record the
    filtered support set and its probability sum) row_margin [N,gmax+1] (the
    top-p cut margin of the row's target and draft transforms, the smaller of
    the two; +inf without top-p), kept_p [N,gmax+1] / kept_q [N,gmax] (kept-set
    sizes) and frac_p / frac_q (kept mass over the tempered row's whole mass);
    NaN / -1 for rows not computed.  Per request, amb_kind says which decisions
    lie within TOL = 1e-6 of their boundary (AMB_ACCEPT: an accept ratio,
    AMB_TOP_P: a top-p cut, AMB_CDF: the draw), and z_lo / z_hi bound the
    draw window: the tokens drawn by inverse CDF at u_sample - TOL and
    u_sample + TOL, between which every token with positive weight is an
    equally valid draw when only the CDF margin is small.  With ``synthetic_rates`` (float32 [gmax]) the synthetic
    acceptance mode runs instead: draft j is accepted iff u_j < rate_j.

    ``banned`` = (offsets [N + 1], ids): request i's banned tokens are
    ids[offsets[i]:offsets[i+1]].  Following the zwjcode.cn page, section 06
    (p and q go through identical transforms, banned tokens among them), a
    banned token is a token whose logit is -inf in every target row of the
    request and whose probability is 0 in every draft row; the batch is run on
    inputs changed that way.  A list longer than BAN_MAX, not strictly
    ascending, or with an id outside [0, V) faults its request (FAULT_BAN_LIST,
    with the request's parameter faults and no row read).

    ``penalties`` = dict(lists=..., repetition=[N] or None, presence=[N] or
    None, frequency=[N] or None): repetition penalties, the other transform
    that section names.  lists[i][j] = (ids, counts) for each row j = 0 ..
    gamma_i of request i: the tokens of the context that position j continues
    (the draft tokens before j included) and how often each occurs in the
    generated output (0: only in the prompt).  Each listed token's logit is
    changed as ``penalize_logits`` states and its draft probability multiplied
    by exp(-delta) (``penalty_deltas``), the same change on the probability
    scale, before temperature, top-k and top-p.  A list longer than PEN_MAX,
    not strictly ascending, with an id outside [0, V) or a negative count, a
    repetition penalty that is not a positive finite number, a presence or
    frequency penalty that is not finite, or a repetition penalty other than 1
    on a request that carries draft rows and has a nonzero temperature (a
    multiplicative change of logits has no counterpart on probabilities, whose
    logits are fixed only up to a constant), faults the request
    (FAULT_PENALTY, with its parameter faults).
    """
    lib = _lib_override or _load()
    ids = _c(draft_ids, np.int32)
    N, gmax = ids.shape
    dt = {"f32": 0, "bf16": 1}[dtype]
    tl = _c(target_logits, np.uint16 if dt == 1 else np.float32)
    V = tl.shape[-1]
    assert tl.shape == (N, gmax + 1, V), tl.shape
    q = _c(draft_probs, np.float32)
    if q is not None:
        assert q.shape == (N, gmax, V), q.shape
    bad_pen = np.zeros(N, bool)
    if penalties is not None:
        tl = tl.copy()
        q = None if q is None else q.copy()
        neg = np.concatenate([ids < 0, np.ones((N, 1), bool)], axis=1)
        gam = np.argmax(neg, axis=1)  # the first negative id, else gmax
        for i in range(N):
            bad_pen[i] = not _penalize_request(i, gam[i], penalties, tl, q, dtype, temperature, V)
    bad_list = np.zeros(N, bool)
    if banned is not None:
        off, bid = np.asarray(banned[0], np.int64), np.asarray(banned[1], np.int64)
        tl = tl.copy()
        q = None if q is None else q.copy()
        for i in range(N):
            n = off[i + 1] - off[i]
            lst = bid[off[i]:off[i + 1]] if n >= 0 else bid[:0]
            if n < 0 or n > BAN_MAX or (lst < 0).any() or (lst >= V).any() or (np.diff(lst) <= 0).any():
                bad_list[i] = True
                continue
            tl[i][:, lst] = 0xFF80 if dt == 1 else -np.inf
            if q is not None:
                q[i][:, lst] = 0.0
    T = _c(temperature, np.float32)
    k = _c(top_k, np.int32)
    p = _c(top_p, np.float32)
    ua = _c(u_accept, np.float32) if u_accept is not None else np.zeros((N, gmax), np.float32)
    us = _c(u_sample, np.float32) if u_sample is not None else np.zeros((N,), np.float32)
    out = dict(tokens=np.empty((N, gmax + 1), np.int32), num_accepted=np.empty((N,), np.int32),
               p_y=np.empty((N, gmax), np.float64), q_y=np.empty((N, gmax), np.float64),
               resid_mass=np.empty((N,), np.float64), margin=np.empty((N,), np.float64),
               fault=np.empty((N,), np.int32), row_margin=np.empty((N, gmax + 1), np.float64),
               kept_p=np.empty((N, gmax + 1), np.int32), kept_q=np.empty((N, gmax), np.int32),
               frac_p=np.empty((N, gmax + 1), np.float64), frac_q=np.empty((N, gmax), np.float64),
               amb_kind=np.empty((N,), np.int32), z_lo=np.empty((N,), np.int32), z_hi=np.empty((N,), np.int32))
    rows = [out[k] for k in ("row_margin", "kept_p", "kept_q", "frac_p", "frac_q", "amb_kind", "z_lo", "z_hi")]

    def sl(a, lo):
        return None if a is None else a[lo:].ctypes.data

    rates = None if synthetic_rates is None else _c(synthetic_rates, np.float32)
    if rates is not None:
        assert rates.shape == (gmax,), rates.shape
        out["p_y"][:] = np.nan
        out["q_y"][:] = np.nan

    def one(lo, hi):
        n = hi - lo
        if n <= 0:
            return 0
        if rates is not None:
            return lib.oracle_spec_verify_synthetic(
                n, gmax, V, sl(ids, lo), sl(q, lo), sl(tl, lo), dt, sl(T, lo), sl(k, lo), sl(p, lo),
                rates.ctypes.data, sl(ua, lo), sl(us, lo), sl(out["tokens"], lo), sl(out["num_accepted"], lo),
                sl(out["resid_mass"], lo), sl(out["margin"], lo), sl(out["fault"], lo), *[sl(a, lo) for a in rows])
        return lib.oracle_spec_verify(n, gmax, V, sl(ids, lo), sl(q, lo), sl(tl, lo), dt, sl(T, lo), sl(k, lo),
                                      sl(p, lo), sl(ua, lo), sl(us, lo), sl(out["tokens"], lo),
                                      sl(out["num_accepted"], lo), sl(out["p_y"], lo), sl(out["q_y"], lo),
                                      sl(out["resid_mass"], lo), sl(out["margin"], lo), sl(out["fault"], lo),
                                      *[sl(a, lo) for a in rows])

    threads = max(1, min(int(threads), N)) if N else 1
    if threads == 1:
        rc = [one(0, N)]
    else:
        bounds = np.linspace(0, N, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            rc = list(ex.map(lambda t: one(bounds[t], bounds[t + 1]), range(threads)))
    if any(rc):
        raise ValueError("oracle rejected the shapes or dtype")
    for i in np.nonzero(bad_list | bad_pen)[0]:
        out["fault"][i] = ((out["fault"][i] & (FAULT_DRAFT_ID | FAULT_TEMPERATURE | FAULT_TOP_P)) |
                           (FAULT_BAN_LIST if bad_list[i] else 0) | (FAULT_PENALTY if bad_pen[i] else 0))
        out["tokens"][i] = -1
        out["num_accepted"][i] = -1
        out["p_y"][i] = np.nan
        out["q_y"][i] = np.nan
        out["resid_mass"][i] = np.nan
        out["margin"][i] = np.inf
        out["row_margin"][i] = np.nan
        out["kept_p"][i] = -1
        out["kept_q"][i] = -1
        out["frac_p"][i] = np.nan
        out["frac_q"][i] = np.nan
        out["amb_kind"][i] = 0
        out["z_lo"][i] = -1
        out["z_hi"][i] = -1
    return out


def penalty_deltas(counts, presence, frequency):
    """The additive penalty of each listed token, float32: frequency * count +
    presence for a token that occurs in the generated output (count > 0), 0 for
    one that occurs only in the prompt; the product and the sum are each
    rounded to float32."""
    c = np.asarray(counts, np.int64)
    with np.errstate(all="ignore"):
        d = np.float32(frequency) * c.astype(np.float32)
        d = (d + np.float32(presence)).astype(np.float32)
    return np.where(c > 0, d, np.float32(0.0)).astype(np.float32)


def penalize_logits(values, dtype, theta, deltas):
    """Penalised logits of listed tokens: a positive logit is divided by the
    repetition penalty theta and any other multiplied by it, then the token's
    delta is subtracted, in float32 with each operation rounded; bf16 logits
    (uint16 bit patterns in and out) are rounded back to bf16, to nearest
    even, NaN staying NaN."""
    bf16 = dtype == "bf16"
    v = np.asarray(values)
    if bf16:
        l = (v.astype(np.uint32) << 16).view(np.float32)
    else:
        l = v.astype(np.float32)
    th = np.float32(theta)
    with np.errstate(all="ignore"):
        l1 = np.where(l > 0, l / th, l * th).astype(np.float32)
        l2 = (l1 - np.asarray(deltas, np.float32)).astype(np.float32)
    if not bf16:
        return l2
    u = l2.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(l2), np.uint16(0x7FC0), r).astype(np.uint16)


def _penalize_request(i, gamma, pen, tl, q, dtype, temperature, V):
    """Apply request i's penalties to its rows in place; False if they fault."""
    def scalar(key, default):
        a = pen.get(key)
        return np.float32(default if a is None else a[i])
    theta, pres, freq = scalar("repetition", 1.0), scalar("presence", 0.0), scalar("frequency", 0.0)
    if not (np.isfinite(theta) and theta > 0 and np.isfinite(pres) and np.isfinite(freq)):
        return False
    T = 1.0 if temperature is None else np.float32(temperature[i])
    if theta != 1 and q is not None and T != 0:
        return False
    rows = pen["lists"][i]
    assert len(rows) == gamma + 1, "one list per row j = 0 .. gamma_i"
    for pid, cnt in rows:
        pid, cnt = np.asarray(pid, np.int64), np.asarray(cnt, np.int64)
        if (len(pid) > PEN_MAX or len(cnt) != len(pid) or (pid < 0).any() or (pid >= V).any() or
                (np.diff(pid) <= 0).any() or (cnt < 0).any()):
            return False
    for j, (pid, cnt) in enumerate(rows):
        pid = np.asarray(pid, np.int64)
        d = penalty_deltas(cnt, pres, freq)
        tl[i, j, pid] = penalize_logits(tl[i, j, pid], dtype, theta, d)
        if q is not None and j < gamma:
            q[i, j, pid] = (q[i, j, pid].astype(np.float64) * np.exp(-d.astype(np.float64))).astype(np.float32)
    return True


def target_probs(row, dtype, T=1.0, top_k=0, top_p=1.0, _lib_override=None):
    """p' of one target row as V doubles; returns (probs, fault, topp_margin)."""
    lib = _lib_override or _load()
    dt = {"f32": 0, "bf16": 1}[dtype]
    r = _c(row, np.uint16 if dt == 1 else np.float32)
    out = np.zeros(r.shape[0], np.float64)
    m = np.zeros(1, np.float64)
    f = lib.oracle_target_probs(r.shape[0], _ptr(r), dt, float(T), int(top_k), float(top_p), _ptr(out), _ptr(m))
    return out, f, float(m[0])


def draft_probs(row, T=1.0, top_k=0, top_p=1.0, _lib_override=None):
    """q' of one draft row as V doubles; returns (probs, fault, topp_margin)."""
    lib = _lib_override or _load()
    r = _c(row, np.float32)
    out = np.zeros(r.shape[0], np.float64)
    m = np.zeros(1, np.float64)
    f = lib.oracle_draft_probs(r.shape[0], _ptr(r), float(T), int(top_k), float(top_p), _ptr(out), _ptr(m))
    return out, f, float(m[0])


class Variant:
    """The same interface bound to another build of the oracle source (used to
    check that the pins reject deliberately altered copies of it)."""

    def __init__(self, so_path):
        self._lib = _bind(so_path)
        for name in ("FAULT_DRAFT_ID", "FAULT_TEMPERATURE", "FAULT_TOP_P", "FAULT_TARGET_ROW",
                     "FAULT_DRAFT_ROW", "FAULT_DRAFT_MASS"):
            setattr(self, name, globals()[name])

    def run(self, *a, **k):
        return run(*a, _lib_override=self._lib, **k)

    def target_probs(self, *a, **k):
        return target_probs(*a, _lib_override=self._lib, **k)

    def draft_probs(self, *a, **k):
        return draft_probs(*a, _lib_override=self._lib, **k)


def build_variant(source_text: str, out_dir: str) -> "Variant":
    """Compile an altered copy of the oracle source and bind it."""
    src = os.path.join(out_dir, "variant.c")
    so = os.path.join(out_dir, "libvariant.so")
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", so, src, "-lm"])
    return Variant(so)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def rollback(num_accepted, gamma, num_computed_tokens=None, num_output_placeholders=None, slot_rows=None):
    """KV bookkeeping after verification, one request at a time.

    KV page "投机解码如何与 KV Cache 交互：Placeholder、回滚与草稿 KV", section 3.1:
    the rejected drafts are gamma_i - A_i; num_computed_tokens steps back by
    that many when it is positive, and so does num_output_placeholders.
    vLLM page, the padded drafter batch paragraph: a rejected draft's KV slot
    becomes PADDING_SLOT_ID (-1).  slot_rows[i] is request i's slot array
    (one entry per draft position).  A request whose A_i is outside
    [0, gamma_i] (a faulted verify) is left unchanged.  Returns new copies."""
    n = len(num_accepted)
    nct = None if num_computed_tokens is None else [int(x) for x in num_computed_tokens]
    nop = None if num_output_placeholders is None else [int(x) for x in num_output_placeholders]
    slots = None if slot_rows is None else [list(int(x) for x in r) for r in slot_rows]
    for i in range(n):
        A, g = int(num_accepted[i]), int(gamma[i])
        if A < 0 or A > g:
            continue
        rejected = g - A
        if nct is not None and nct[i] > 0:
            nct[i] -= rejected
        if nop is not None and nop[i] > 0:
            nop[i] -= rejected
        if slots is not None:
            for j in range(A, g):
                slots[i][j] = -1
    return nct, nop, slots
