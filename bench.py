#!/usr/bin/env python3
"""Throughput of the batched draft-verify rejection sampler on one MI355X.

One step = one spec_verify call (row pass + per-request finish) over the
whole batch of the workload.  The default workload is N = 256 requests,
gamma = 5 drafts, V = 128256, bf16 target logits, fp32 draft probabilities,
top_k = 50 / top_p = 0.9 on both distributions, T = 1 (the N=256, V=128256
configuration).  Inputs are seeded synthetic tensors resident in HBM before
the timed region; ceil(512 MB / bytes per step) copies of them (at least 2, at
most 64) rotate between steps so that no step reads data an earlier step left
in the 256 MB Infinity Cache.

Before the timed steps the step runs at least --warmup times and for at
least --warmup-ms of wall time, so that the GPU's clocks have settled.  The
padded call is bound once (rejection_sampling_verify_13_amd.Prepared), so a
step costs the host one C call.  The row kernel is timed with HIP events
carried by its own dispatch, created without a system-scope release
(hipEventDisableSystemFence), so timing a step does not slow the next one.

Prints one JSON line: verified draft positions per second (sum of gamma_i per
step / time), the roofline of the dominant kernel (the row pass, timed with
HIP events on its stream), and the CPU oracle timed on a bounded sample of the
same workload.
"""
import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SRC = os.path.join(ROOT, "rejection_sampling_verify_13_amd", "csrc", "spec_verify.hip")
COUNTERS = os.path.join(ROOT, "profiles", "row_kernel_counters.md")


def source_digest():
    with open(SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload_bytes(batch):
    """Algorithmic HBM bytes of one step: every real target row once (rows
    0..gamma_i), every real draft row once (rows 0..gamma_i-1 of sampled
    requests that carry draft probabilities), plus the small per-request
    arrays and outputs."""
    import numpy as np
    V = batch["target_logits"].shape[-1]
    s_l = 2 if batch["dtype"] == "bf16" else 4
    gam = batch["gamma"].astype(np.int64)
    N, G = batch["draft_ids"].shape
    sampled = batch["temperature"] > 0
    with_q = sampled & batch["has_q"] if batch["draft_probs"] is not None else np.zeros(N, bool)
    target = int((gam + 1).sum()) * V * s_l
    draft = int(gam[with_q].sum()) * V * 4
    small = N * G * 4 * 2 + N * 4 * 4 + N * (G + 1) * 4 + N * 4
    return target + draft + small, target, draft


def synthetic_bytes(batch, rates):
    """Algorithmic bytes of the synthetic acceptance mode: only row A_i of each
    request is read (A_i = the first j with u_j >= rate_j, else gamma_i), its
    draft row too when A_i < gamma_i and the request carries draft rows."""
    import numpy as np
    V = batch["target_logits"].shape[-1]
    s_l = 2 if batch["dtype"] == "bf16" else 4
    N, G = batch["draft_ids"].shape
    gam = batch["gamma"].astype(np.int64)
    hq = batch["has_q"] if batch["draft_probs"] is not None else np.zeros(N, bool)
    total = 0
    for i in range(N):
        A = next((j for j in range(gam[i]) if not batch["u_accept"][i, j] < rates[j]), gam[i])
        total += V * s_l + (V * 4 if (A < gam[i] and hq[i]) else 0)
    return total + N * G * 4 * 2 + N * 4 * 4 + N * (G + 1) * 4 + N * 4


def traffic_from_profile(digest, workload):
    """HBM bytes per row-kernel launch from the committed counter summary, if
    it was taken on this exact kernel source and workload; else None."""
    if not os.path.exists(COUNTERS):
        return None
    text = open(COUNTERS).read()
    for b, src, wl in re.findall(r"traffic_bytes_per_launch:\s*(\d+)\s+source:\s*(\w+)\s+workload:\s*(\S+)", text):
        if src == digest and wl == workload:
            return int(b)
    return None


class TimingEvent:
    """A HIP event that only times the row kernel, created through the HIP
    runtime this process already loaded (found by its path in
    /proc/self/maps, so no second runtime is loaded).  With
    hipEventDisableSystemFence (the default here) recording it makes no
    system-scope release: a default event's release writes back and
    invalidates the caches, which costs the step after it a few microseconds.
    elapsed_time() is read only after a device-wide synchronisation."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self, fence=False):
        h = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(h), 0 if fence else self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.cuda_event = h.value

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                 ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value


def host_threads():
    """Threads for the host-side work (input generation, the CPU oracle): the
    CPUs this process may run on, limited by OMP_NUM_THREADS when that is set
    (the share of a shared host that one GPU's job is given)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    lim = os.environ.get("OMP_NUM_THREADS", "")
    if lim.isdigit() and int(lim) > 0:
        n = min(n, int(lim))
    return max(1, n)


def acceptance_stats(num_accepted, gamma, temperature):
    """What the zwjcode.cn page, section 12, asks to record with the
    throughput: how far each request advanced (the distribution of the
    rejection position A_i, i.e. of the accepted draft count), the mean
    accepted length and committed tokens per target step, and the acceptance
    rate over the drafts proposed."""
    import numpy as np
    A = np.asarray(num_accepted, np.int64)
    gam = np.asarray(gamma, np.int64)
    ok = A >= 0
    G = int(gam.max()) if len(gam) else 0
    hist = np.bincount(A[ok], minlength=G + 1)[: G + 1]
    all_acc = ok & (A == gam)
    return {
        "requests": int(len(A)), "faulted": int((~ok).sum()),
        "accepted_count_histogram": [int(x) for x in hist],
        "all_drafts_accepted": int(all_acc.sum()),
        "mean_accepted_length": round(float(A[ok].mean()), 4) if ok.any() else None,
        "mean_committed_per_step": round(float((A[ok] + 1).mean()), 4) if ok.any() else None,
        "acceptance_rate": round(float(A[ok].sum() / max(1, gam[ok].sum())), 4),
        "greedy_requests": int((np.asarray(temperature) == 0).sum()),
    }


def cpu_baseline(spec, n_req, threads, min_seconds=10.0):
    """The fp64 C oracle timed on the host over the first n_req requests of
    the same workload, repeated until about min_seconds have passed."""
    import numpy as np
    import oracle
    import workloads as W
    oracle.build(force=False)
    sub = W.generate(spec, requests=range(n_req), threads=threads)
    pos = int(np.asarray(sub["gamma"]).sum())
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.run(sub["draft_ids"], sub["draft_probs"], sub["target_logits"], sub["dtype"], sub["temperature"],
                   sub["top_k"], sub["top_p"], sub["u_accept"], sub["u_sample"], threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return dict(value=pos * passes / dt, unit="positions/s", cores=threads, kind="oracle",
                host_cpus=os.cpu_count(), threads=threads,
                sample="first %d of %d requests of the same workload (%d verified positions) x %d passes, "
                       "fp64 C oracle, %d threads over requests, %.1f s wall" % (n_req, spec.N, pos, passes, threads, dt))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3)")
    ap.add_argument("--cpu-sample", type=int, default=256, help="requests timed on the CPU oracle (0: skip)")
    ap.add_argument("--layout", choices=("auto", "padded", "flat"), default="auto",
                    help="input layout: padded [N, gmax] calls, or one flattened (ragged) call; auto: flattened "
                         "for a batch that mixes requests with and without draft rows (config 5), else padded")
    ap.add_argument("--rollback", action="store_true",
                    help="also enqueue the KV bookkeeping (spec_verify_rollback) after every verify call, "
                         "inside the timed step")
    ap.add_argument("--synthetic-rates", default=None,
                    help="comma-separated per-position acceptance rates: run the synthetic acceptance mode "
                         "(flattened layout; only row A of each request is read)")
    ap.add_argument("--banned", type=int, default=0,
                    help="ban this many seeded random token ids per request (flattened layout, identical in p and q)")
    ap.add_argument("--penalties", type=int, default=0,
                    help="repetition penalties over a seeded context of this many tokens per request (flattened "
                         "layout; presence 0.5, frequency 0.25, repetition 1.2 on greedy and draft-free requests)")
    ap.add_argument("--time-every", type=int, default=0,
                    help="time the row kernel with HIP events on every Nth timed step (the events travel in the "
                         "row kernel's own dispatch; the wall-clock throughput covers every step); default: every "
                         "step when --steps is below 100, else every 4th")
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="keep warming up past --warmup steps until this much wall time has passed")
    ap.add_argument("--timing-events", choices=("nofence", "fence"), default="nofence",
                    help="the row kernel's HIP events: without a system-scope release (default) or with one "
                         "(hipEventDefault)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run a plain elementwise copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the verify path is measured on one MI355X and no "
              "multi-GPU run is part of this build (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import rejection_sampling_verify_13_amd as sv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = W.config(args.config)
    threads = host_threads()
    print("[bench] generating workload %d (N=%d gmax=%d V=%d)" % (args.config, spec.N, spec.gmax, spec.V),
          file=sys.stderr, flush=True)
    batch = W.generate(spec, threads=threads)
    mixed = batch["draft_probs"] is not None and not batch["has_q"].all()
    rates = None if args.synthetic_rates is None else np.array(
        [float(x) for x in args.synthetic_rates.split(",")], np.float32)
    if rates is not None and len(rates) != spec.gmax:
        sys.exit("--synthetic-rates needs %d rates" % spec.gmax)
    flat = (args.layout == "flat" or (args.layout == "auto" and mixed) or rates is not None or args.banned > 0 or
            args.penalties > 0)
    ban = None
    if args.banned > 0:
        brng = np.random.default_rng(7)
        lists = [np.sort(brng.choice(spec.V, size=args.banned, replace=False)) for _ in range(spec.N)]
        ban = (np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32),
               np.concatenate(lists).astype(np.int32))
    pen = None
    if args.penalties > 0:
        off, pid, cnt = W.flatten_penalties(W.penalty_lists(batch, 8, args.penalties))
        dense = batch["has_q"] if batch["draft_probs"] is not None else np.zeros(spec.N, bool)
        theta = np.where(dense & (batch["temperature"] != 0), 1.0, 1.2).astype(np.float32)
        pen = dict(penalty_offsets=off, penalty_ids=pid, penalty_counts=cnt, repetition_penalty=theta,
                   presence_penalty=np.full(spec.N, 0.5, np.float32),
                   frequency_penalty=np.full(spec.N, 0.25, np.float32))
    if flat:
        parts = [W.flatten(batch)]
    else:
        parts = W.split_by_q(batch) if mixed else [batch]
    B_alg, B_target, B_draft = workload_bytes(batch)
    if rates is not None:
        B_alg = synthetic_bytes(batch, rates)
        B_target = B_draft = None
    positions = int(batch["gamma"].sum())
    rows = int((batch["gamma"] + 1).sum())

    # resident copies of the inputs, rotated between steps: together at least
    # 512 MB, twice the Infinity Cache
    n_sets = int(min(64, max(2, -(-(512 << 20) // max(1, B_alg)))))
    sets = []
    for _ in range(n_sets):
        ps = []
        for p in parts:
            if flat:
                d = sv.to_device_flat(p, dev)
                Np, Gp = p["cu_num_draft_tokens"].shape[0], p["gmax"]
            else:
                d = sv.to_device(p, dev)
                Np, Gp = p["draft_ids"].shape
            Vp = p["target_logits"].shape[-1]
            d["ws"] = torch.empty((sv.workspace_size(Np, Gp, Vp),), dtype=torch.uint8, device=dev)
            d["out_t"] = torch.empty((Np, Gp + 1), dtype=torch.int32, device=dev)
            d["out_n"] = torch.empty((Np,), dtype=torch.int32, device=dev)
            if args.rollback:
                d["nct"] = torch.full((Np,), 1 << 20, dtype=torch.int32, device=dev)
                d["slots"] = torch.arange(d["draft_ids"].numel(), dtype=torch.int32, device=dev).view(
                    d["draft_ids"].shape)
            if rates is not None:
                d["rates"] = torch.from_numpy(rates).to(dev)
            if ban is not None:
                d["ban_off"] = torch.from_numpy(ban[0]).to(dev)
                d["ban_ids"] = torch.from_numpy(ban[1]).to(dev)
            if pen is not None:
                d.update({k: torch.from_numpy(v).to(dev) for k, v in pen.items()})
            if not flat and rates is None and ban is None and pen is None:
                # the padded call bound once: one C call per step on the host
                d["call"] = sv.Prepared(d["draft_ids"], d["draft_probs"], d["target_logits"], d["temperature"],
                                        d["top_k"], d["top_p"], d["u_accept"], d["u_sample"],
                                        out_tokens=d["out_t"], out_num_accepted=d["out_n"], workspace=d["ws"],
                                        stream=torch.cuda.current_stream(dev))
            ps.append(d)
        sets.append(ps)
    del batch["target_logits"], batch["draft_probs"]
    stream = torch.cuda.current_stream(dev)

    def step(k, events=None):
        for pi, d in enumerate(sets[k % n_sets]):
            ev = None
            if events is not None:
                ev = events[pi]
            if "call" in d:
                d["call"](ev)
                if args.rollback:
                    sv.rollback(d["out_n"], num_computed_tokens=d["nct"], slot_mapping=d["slots"], stream=stream,
                                draft_ids=d["draft_ids"])
                continue
            kw = dict(out_tokens=d["out_t"], out_num_accepted=d["out_n"], workspace=d["ws"], stream=stream, events=ev)
            if rates is not None:
                kw.update(synthetic_rates=d["rates"])
            if ban is not None:
                kw.update(banned_offsets=d["ban_off"], banned_ids=d["ban_ids"])
            if flat:
                sv.verify_flat_batch(d, **kw)
            else:
                sv.verify_batch(d, **kw)
            if args.rollback:
                lay = dict(cu_num_draft_tokens=d["cu_num_draft_tokens"], gmax=d["gmax"]) if flat else \
                    dict(draft_ids=d["draft_ids"])
                sv.rollback(d["out_n"], num_computed_tokens=d["nct"], slot_mapping=d["slots"], stream=stream, **lay)

    K = args.steps
    every = args.time_every if args.time_every > 0 else (1 if args.steps < 100 else 4)
    timed = list(range(0, K, every))
    # start and end of the row kernel (the third event of the entry point, after the draw pass, is not used),
    # created before the warm-up so that no host work separates it from the timed steps
    fence = args.timing_events == "fence"
    evs = {k: [(TimingEvent(fence), TimingEvent(fence), None) for _ in parts] for k in timed}

    # warm-up: the requested steps, and more until the GPU has run the step for
    # at least --warmup-ms (its clocks settle over tens of milliseconds of
    # load: a 20-step run right after 5 warm-up steps measured its row kernel
    # 3 % slower than after 2000)
    t_w = time.perf_counter()
    warm = 0
    while warm < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
        step(warm)
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(k, evs.get(k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    row_ms = np.array([sum(e[0].elapsed_time(e[1]) for e in evs[k]) for k in timed])
    ms_per_step = wall * 1e3 / K
    value = positions * K / wall
    # every input set holds the same batch: the outputs of the first one stand for all steps
    acc = acceptance_stats(np.concatenate([d["out_n"].cpu().numpy() for d in sets[0]]), batch["gamma"],
                           batch["temperature"])

    digest = source_digest()
    workload_name = "cfg%d" % args.config
    traffic = traffic_from_profile(digest, workload_name)
    row_avg_s = float(row_ms.mean()) * 1e-3
    row_pct = [round(float(x) * 1e3, 2) for x in np.percentile(row_ms, [10, 50, 90])]
    achieved = B_alg / row_avg_s / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel="row_kernel", kernel_avg_us=round(row_avg_s * 1e6, 2),
                    kernel_us_p10_p50_p90=row_pct, input_sets_rotated=n_sets, launches_timed=len(timed),
                    timing_events=("hipEventDefault" if args.timing_events == "fence" else
                                   "hipEventDisableSystemFence"),
                    algorithmic_bytes_per_launch=B_alg,
                    fetch_gbps=None if traffic is None else round(traffic / row_avg_s / 1e9, 1),
                    scope="the row kernel alone (the dominant kernel); the whole verify step (plan, row, draw "
                          "and find kernels) is hbm_gbps_step / hbm_frac_step")

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    cpu = None
    if args.cpu_sample > 0:
        n_req = min(args.cpu_sample, spec.N)
        print("[bench] timing the CPU oracle on %d requests" % n_req, file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, n_req, threads)

    desc = {1: "tiny fp32: N=4 gamma=4 V=1024",
            2: "N=64 gamma=4 V=32000 bf16 T=0.8",
            3: "N=256 gamma=5 V=128256 bf16 top_k=50 top_p=0.9 T=1",
            4: "N=512 gamma=8 V=151936 bf16 25% greedy, T~U[0.5,1.2]",
            5: "N=1024 ragged gamma in 0..7 V=128256 bf16, half draft-free"}[args.config]
    out = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X",
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "requests": spec.N, "gamma": spec.gmax, "vocab": spec.V,
                   "layout": "flattened, one call" if flat else "padded, %d call(s)" % len(parts),
                   "kv_rollback_in_step": bool(args.rollback),
                   "synthetic_rates": None if rates is None else [float(x) for x in rates],
                   "banned_per_request": args.banned,
                   "penalty_context_per_request": args.penalties,
                   "target_logits": spec.dtype, "draft_probs": "f32" if spec.q_mode != "null" else None,
                   "verified_positions_per_step": positions, "rows_per_step": rows,
                   "algorithmic_bytes_per_step": B_alg, "target_bytes": B_target, "draft_bytes": B_draft},
        "hbm_gbps_step": round(B_alg / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(B_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "rows_per_s": round(rows * K / wall, 1),
        "bytes_per_verified_position": round(B_alg / max(1, positions), 1),
        "acceptance": acc,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source": digest,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
