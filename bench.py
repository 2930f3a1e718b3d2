#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verification sampler on one MI355X.

One step = one spec_verify call over one batch (row statistics, accept scan and final draw for
every sequence). Default workload: B=64 sequences, D=7 draft positions, V=128256, bf16 logits,
T=1, Zipf(1.1)+N(0,1) target and target+N(0,1) draft (seed 0). Several copies of the inputs
are resident in HBM and rotated so that no step can be served from the 256 MB Infinity Cache.

Prints ONE JSON line: verified rows/s (sequences per second) as `value`, the HBM bandwidth of
the algorithmic bytes, the roofline of the dominant kernel (row statistics) timed with HIP
events on the launch stream, and the fp64 CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/s + HBM GB/s (% of peak), B=64 D=7 V=128256 bf16"
HBM_PEAK_GBPS = 8000.0
ROW_SLICE = 32767          # sequences per row launch (larger batches launch in slices)
SRC = os.path.join(ROOT, "sampling_spec_verify_02_amd", "csrc", "spec_verify.hip")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic_row_kernel_c3.json")

WORKLOADS = {
    "c1": "B=1 D=4 V=1024 fp32 T=1, N(0,2^2) target, draft +N(0,0.5^2)",
    "c2": "B=16 D=4 V=32000 fp32 T=1, Zipf(1.1)+N(0,1) target, draft +N(0,1)",
    "c3": "B=64 D=7 V=128256 bf16 T=1, Zipf(1.1)+N(0,1) target, draft +N(0,1)",
    "c4": "B=256 D=3 V=128256 bf16, half greedy / half T=0.7, 10% draft==target, else +N(0,1.5^2)",
    "c5": "B=512 D=7 V=129280 bf16 T=1, ragged L~U{1..7}, draft sigma_b~U[0.25,2]",
    "mtp": "B=1024 D=1 V=129280 bf16 T=1, single-token verify, Zipf(1.1)+N(0,1) target, "
           "draft +N(0,1)",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def valid_row_bytes(w, threshold=False) -> int:
    """Algorithmic logit bytes: every row the method needs, once (target rows 0..L_b, draft rows
    0..L_b-1, no draft rows for greedy sequences or for threshold acceptance)."""
    rows = 0
    for b in range(w.B):
        L = int(w.lens[b])
        rows += (L + 1) + (0 if (w.temperature[b] == 0 or threshold) else L)
    return rows * w.V * w.elem_bytes, rows


def fetched_row_bytes(w, al, cuts, threshold=False) -> int:
    """Logit bytes the staged row launches read for this batch, given each sequence's AL from the
    call: launch s reads positions [cuts[s], cuts[s+1]) of a sequence unless its first rejection
    j lies before cuts[s] (then the rows past j are skipped)."""
    rows = 0
    for b in range(w.B):
        L = int(w.lens[b])
        if al[b] < 1:
            continue                      # invalid row: nothing past the check is read
        j = int(al[b]) - 1
        stop = cuts[-1]
        for s in range(1, len(cuts) - 1):
            if j < cuts[s]:
                stop = cuts[s]
                break
        last = min(L, stop - 1)
        draft = not (w.temperature[b] == 0 or threshold)
        rows += (last + 1) + (min(last + 1, L) if draft else 0)
    return rows * w.V * w.elem_bytes


def source_digest() -> str:
    return hashlib.sha256(open(SRC, "rb").read()).hexdigest()


def read_traffic(config: str, seed: int):
    """HBM bytes of a call's row phase (its row launches, FETCH_SIZE and WRITE_SIZE summed over
    them) from the committed rocprofv3 PMC summary, or None if the kernel source changed since
    the counters were taken or the counters were taken on another workload."""
    try:
        t = json.load(open(TRAFFIC))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest() or (config, seed) != ("c3", 0):
        return None
    return t.get("traffic_bytes_row_phase")


def cpu_baseline(w, seconds: float, tau=None):
    from oracle import verify, verify_threshold

    tgt, drf = w.target_f32(), w.draft_f32()
    lens = w.lens if w.lens_given else None

    def run(k):
        t0 = time.perf_counter()
        lk = None if lens is None else lens[:k]
        if tau is None:
            verify(tgt[:k], drf[:k], w.tokens[:k], lk, w.uniforms[:k], w.temperature[:k])
        else:
            verify_threshold(tgt[:k], w.tokens[:k], lk, w.uniforms[:k], w.temperature[:k], tau)
        return time.perf_counter() - t0

    per = run(min(2, w.B)) / min(2, w.B)
    k = int(max(1, min(w.B, seconds / max(per, 1e-6))))
    reps, dt = 0, 0.0
    while True:                      # whole-batch repeats until the sample is ~`seconds` long
        dt += run(k)
        reps += 1
        if dt >= seconds or k < w.B or reps >= 1000:
            break
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                     if l.startswith("model name"))
    except (OSError, StopIteration):
        model = platform.processor()
    return {"value": reps * k / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x first {k} of {w.B} sequences of the same workload, numpy fp64, "
                      f"one thread, {dt:.1f} s on {model} "
                      f"({len(os.sched_getaffinity(0))} cores visible)",
            "ms_per_call_extrapolated": 1000 * dt / (reps * k) * w.B}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--threshold", type=float, default=None,
                    help="time threshold acceptance with this tau instead of the standard rule "
                         "(target rows only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device-to-device copies of 256 MiB (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (sequences would shard over B with no exchange; "
              "a multi-GPU run is not implemented). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sampling_spec_verify_02_amd as sv
    from workloads import make

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = 256 << 20
        src = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(3)]
        dst = [torch.empty_like(x) for x in src]
        for k in range(args.steps):
            dst[k % 3].copy_(src[k % 3])
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written":
                          nbytes, "copies": args.steps}), flush=True)
        return
    log(f"bench: generating {args.config} seed {args.seed}")
    w = make(args.config, args.seed)
    tau = args.threshold
    alg_bytes, rows = valid_row_bytes(w, tau is not None)

    def logits(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    ncopy = max(1, args.copies)
    tgts = [logits(w.target) for _ in range(ncopy)]
    drfs = [logits(w.draft) if tau is None else None for _ in range(ncopy)]
    tok = torch.from_numpy(w.tokens).to(dev)
    lens = torch.from_numpy(w.lens).to(dev) if w.lens_given else None
    uni = torch.from_numpy(w.uniforms).to(dev)
    temp = torch.from_numpy(w.temperature).to(dev)
    al = torch.empty(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.D + 1), dtype=torch.int32, device=dev)
    lib = sv.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)  # noqa: E731
    if tau is None:
        fn = lib.spec_verify_bf16 if w.dtype == "bf16" else lib.spec_verify_f32
        calls = [(P(tgts[c]), P(drfs[c]), P(tok), P(lens), P(uni), w.B, w.D, w.V, P(temp),
                  P(al), P(out), sp) for c in range(ncopy)]
    else:
        fn = lib.spec_verify_threshold
        calls = [(1 if w.dtype == "bf16" else 0, P(tgts[c]), P(tok), P(lens), P(uni), w.B, w.D,
                  w.V, P(temp), float(tau), P(al), P(out), sp) for c in range(ncopy)]

    def step(k):
        rc = fn(*calls[k % ncopy])
        if rc != 0:
            raise RuntimeError(f"spec_verify failed: {sv.strerror(rc)}")

    # correctness of the benchmarked call against the oracle on this workload
    step(0)
    torch.cuda.synchronize()
    from oracle import verify_threshold_workload, verify_workload
    ref = verify_workload(w) if tau is None else verify_threshold_workload(w, tau)
    g_al, g_tok = al.cpu().numpy(), out.cpu().numpy()
    ok = ~ref.flagged
    mism = int(np.sum(ok & ((g_al != ref.accept_len) | np.any(g_tok != ref.tokens, axis=1))))
    log(f"bench: parity vs oracle on the benched batch: {mism} unflagged mismatches "
        f"({int(ref.flagged.sum())} flagged rows)")

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(K):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1000.0 * wall / K
    ev_ms_step = e0.elapsed_time(e1) / K

    # the dominant kernel (the row kernel): every launch timed with its own start and end stamps
    # (HIP events on its launch stream); a call makes one launch per stage and per slice
    cuts_c = (ctypes.c_int * 8)()
    nst = lib.spec_verify_row_stages(1 if w.dtype == "bf16" else 0, w.B, w.D, w.V, cuts_c, 8)
    if nst < 1:
        raise RuntimeError(sv.strerror(nst))
    cuts = [int(cuts_c[i]) for i in range(nst + 1)]
    per_call = nst * ((w.B + ROW_SLICE - 1) // ROW_SLICE)
    rc = lib.spec_verify_profile_start(K * per_call)
    if rc != 0:
        raise RuntimeError(sv.strerror(rc))
    for k in range(K):
        step(k)
    durs = (ctypes.c_float * (K * per_call))()
    n = ctypes.c_int(0)
    rc = lib.spec_verify_profile_stop(durs, K * per_call, ctypes.byref(n))
    if rc != 0:
        raise RuntimeError(sv.strerror(rc))
    if n.value != K * per_call:
        raise RuntimeError(f"{n.value} row launches timed, {K * per_call} expected")
    launch_ms = np.array(durs[:n.value], dtype=np.float64).reshape(K, per_call)
    kern_ms = float(launch_ms.sum(axis=1).mean())          # the row launches of one call
    # the bytes the row launches read for this batch
    fetched = fetched_row_bytes(w, g_al, cuts, tau is not None)
    kern_gbps = fetched / (kern_ms * 1e-3) / 1e9

    # the epilogue (each sequence's window of its W = D+1 latest tokens moved by AL, lengths
    # grown by AL) on the benched batch's outputs, timed alone with events on the same stream
    W = w.D + 1
    ids = torch.zeros((w.B, W), dtype=torch.int32, device=dev)
    slen = torch.zeros(w.B, dtype=torch.int32, device=dev)
    adv_args = (P(al), P(out), w.B, w.D, P(ids), W, P(slen), sp)
    for _ in range(20):
        if lib.spec_verify_advance(*adv_args) != 0:
            raise RuntimeError("spec_verify_advance failed")
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        lib.spec_verify_advance(*adv_args)
    e1.record(stream)
    torch.cuda.synchronize()
    adv_us = 1000.0 * e0.elapsed_time(e1) / K

    # Saguaro draft reshaping (top-5 of every needed draft row) timed alone with events on the
    # same stream, on three rotated scratch copies of the draft logits (together larger than the
    # 256 MB Infinity Cache, so that every call reads its rows from HBM). The factor is 1 (ln 1 =
    # 0): each call writes back the values it read, so every call sees the same rows, where a
    # factor below 1 would lower the same top logits again and again; the kernels' work does not
    # depend on the factor's value.
    sag = None
    if tau is None and w.D > 0:
        scratch = [d.clone() for d in drfs[:3]]
        sag_args = [(1 if w.dtype == "bf16" else 0, P(x), P(lens), P(temp), w.B, w.D, w.V,
                     1.0, 5, sp) for x in scratch]
        for i in range(10):
            if lib.spec_verify_saguaro_reshape(*sag_args[i % len(sag_args)]) != 0:
                raise RuntimeError("spec_verify_saguaro_reshape failed")
        torch.cuda.synchronize()
        ks = min(K, 200)
        e0.record(stream)
        for i in range(ks):
            lib.spec_verify_saguaro_reshape(*sag_args[i % len(sag_args)])
        e1.record(stream)
        torch.cuda.synchronize()
        sag_us = 1000.0 * e0.elapsed_time(e1) / ks
        draft_rows = int(sum(int(w.lens[b]) for b in range(w.B) if w.temperature[b] > 0))
        sag_bytes = draft_rows * w.V * w.elem_bytes
        sag = {"us_per_call": sag_us, "k": 5, "factor": 1.0, "draft_rows": draft_rows,
               "gbps": sag_bytes / (sag_us * 1e-6) / 1e9,
               "note": "spec_verify_saguaro_reshape alone (not part of the step): reads every "
                       "needed draft row once (one wavefront per 8 KB unit, then one wavefront "
                       "per row merges the units' candidates) and rewrites its top-5 logits"}

    gbps = alg_bytes / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": w.B / (ms_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOADS[args.config]}", "B": w.B, "D": w.D,
                   "V": w.V, "seed": args.seed, "input_copies_rotated": ncopy,
                   "acceptance": "standard" if tau is None else f"threshold tau={tau}"},
        "hbm_gbps": gbps,
        "pct_of_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "logit_rows_per_s": rows / (ms_step * 1e-3),
        "algorithmic_bytes_per_step": alg_bytes,
        "bytes_note": "hbm_gbps and pct_of_hbm_peak count every logit row the call is given up "
                      "to L_b (the algorithmic bytes of the workload); the row launches skip the "
                      "rows past a rejection already known, so they read "
                      "fetched_row_bytes_per_step (fetched_hbm_gbps over the whole call)",
        "event_ms_per_step": ev_ms_step,
        "mean_accept_len": float(g_al.mean()),
        "parity_unflagged_mismatches": mism,
        "fetched_row_bytes_per_step": fetched,
        "fetched_hbm_gbps": fetched / (ms_step * 1e-3) / 1e9,
        "row_stages": cuts,
        "roofline": {"bound": "hbm",
                     "kernel": f"row_kernel, {per_call} launch(es) per call"
                               + ("" if nst == 1 else f" (positions {cuts})"),
                     "achieved": kern_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": kern_gbps / HBM_PEAK_GBPS,
                     "traffic": read_traffic(args.config, args.seed), "kernel_ms": kern_ms,
                     "launch_ms": [float(x) for x in launch_ms.mean(axis=0)],
                     "bytes": fetched,
                     "note": "kernel_ms = the row launches of one call, each timed with its own "
                             "start and end stamps (HIP events on the launch stream); achieved = "
                             "the logit bytes those launches read for this batch / kernel_ms. "
                             "The decision kernels between stages (latency-bound, about 4.6 us "
                             "each) are not part of it; the whole call's rate is hbm_gbps"},
        "cpu_baseline": None,
        "saguaro_reshape": sag,
        "advance": {"us_per_call": adv_us, "W": W,
                    "note": "spec_verify_advance alone (not part of the step): window and "
                            "lengths of the batch moved by AL on the GPU, no host sync"},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, tau)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
