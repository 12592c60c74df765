"""Benchmark: Mamba-2 SSD forward tokens/s on one MI355X, with the roofline of
the dominant kernel and the fp64 oracle timed on the host as a CPU baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mma bf16|f32]

One step = one ssd_forward call (cumsum -> chunk states -> state passing ->
fused chunk output) over one batch of the workload, inputs resident in HBM.
The timed steps alternate between two batches of the same shape (seeds s and
s + 1, each with its own y), so that no step finds its inputs left in the
last-level cache by the step before, as consecutive layers of a model would
not; the rate with every step on the same batch is reported beside it.
Warm-up runs at least W steps and at least --min-warmup-s seconds of steps
(GPU clocks ramp under sustained load: a few milliseconds of warm-up measure
the ramp, not the steady state); both counts are reported.
Per-kernel durations come from HIP events recorded on the launch stream around
each ABI call of the same pipeline (a second timed loop).  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def algorithmic_costs(w, in_bytes, y_bytes, carried_bytes=4, states_bytes=4):
    """Algorithmic bytes and flops per launch of each kernel (each tensor read
    or written once; causal interaction terms only; C.B^T once per group).
    ``carried_bytes`` is the element size of the carried states handed from the
    state passing to the chunk scan and ``states_bytes`` that of the chunk
    states (both 2 on the bf16-operand path)."""
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = L // Q
    blh = B * L * H
    st = B * nc * H * N * P
    k = {}
    k["chunk_cumsum"] = dict(bytes=4 * blh + 4 * H + 2 * 4 * blh, flops=2 * blh)
    k["chunk_state"] = dict(bytes=in_bytes * blh * P + in_bytes * B * L * G * N + 2 * 4 * blh + states_bytes * st,
                            flops=2 * blh * N * P)
    # the forward's first step: cumulative sums computed inside the chunk-state
    # kernel (reads dt and A, writes dA_cumsum and dt_bhl instead of reading them)
    k["chunk_cumsum_state"] = dict(bytes=in_bytes * blh * P + in_bytes * B * L * G * N + 4 * blh + 4 * H + 2 * 4 * blh
                                   + states_bytes * st, flops=2 * blh * N * P + 2 * blh)
    k["state_passing"] = dict(bytes=states_bytes * st + 4 * B * H * nc + carried_bytes * st + 4 * B * H * N * P,
                              flops=2 * st)
    k["chunk_state_passing"] = dict(bytes=in_bytes * blh * P + in_bytes * B * L * G * N + 2 * 4 * blh
                                    + carried_bytes * st + 4 * B * H * N * P,
                                    flops=2 * blh * N * P + 2 * st)
    k["chunk_scan"] = dict(bytes=in_bytes * blh * P + 2 * in_bytes * B * L * G * N + 2 * 4 * blh + carried_bytes * st
                           + 4 * H + y_bytes * blh * P,
                           flops=2 * blh * N * P + B * nc * H * Q * (Q + 1) * P + B * nc * G * Q * (Q + 1) * N)
    return k


KERNEL_SOURCES = {
    "chunk_cumsum": ["chunk_cumsum.hip"],
    "chunk_cumsum_state": ["chunk_state_hg.hip", "chunk_state.hip", "chunk_cumsum.hip"],
    "chunk_state": ["chunk_state_hg.hip", "chunk_state.hip"],
    "state_passing": ["state_passing.hip"],
    "chunk_state_passing": ["state_fused.hip"],
    "chunk_scan": ["chunk_scan_hg.hip", "chunk_scan.hip"],
}


def kernel_source_hash(kernel):
    """sha256 over the sources that define a kernel (and the shared device header)."""
    import hashlib
    csrc = os.path.join(ROOT, "mamba_ssd_scan_chunk_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["ssd_device.hpp"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when that summary is missing or was taken on a different
    version of the kernel's sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    entry = data.get("kernels", {}).get(kernel)
    if not entry or entry.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return entry.get("bytes_per_launch")


def cpu_model():
    """Host CPU model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(inp, w, target_s=10.0, single_core=("tiny_f32", "mamba2_130m_layer")):
    """The fp64 oracle on a bounded sample of (b, h) pairs, all host cores;
    also one whole pass over the small workloads on ONE core."""
    import numpy as np
    from mamba_ssd_scan_chunk_amd.inputs import WORKLOADS, workload_inputs
    from oracle import oracle as oracle_mod
    o = oracle_mod.get()
    threads = oracle_mod.default_threads()
    total_pairs = w.batch * w.nheads
    t0 = time.perf_counter()
    o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, pairs=[0], nthreads=1)
    t1 = time.perf_counter() - t0
    per_thread = max(1, int(target_s / max(t1, 1e-3)))
    k = int(min(total_pairs, threads * per_thread))
    pairs = np.linspace(0, total_pairs - 1, k).round().astype(np.int64)
    used = min(threads, k)
    # when every pair fits in the time target, whole passes repeat until it is reached
    passes = 0
    t0 = time.perf_counter()
    while True:
        o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, pairs=pairs, nthreads=used)
        passes += 1
        t = time.perf_counter() - t0
        if k < total_pairs or t >= target_s:
            break
    tokens_per_s = passes * w.tokens * (k / total_pairs) / t
    one = {}
    for name in single_core:
        wi = WORKLOADS[name]
        si = workload_inputs(name)
        t0 = time.perf_counter()
        o.recurrence(si.x, si.dt, si.A, si.Bm, si.Cm, si.D, nthreads=1)
        ts = time.perf_counter() - t0
        one[name] = {"s": round(ts, 4), "tokens_per_s": round(wi.tokens / ts, 1),
                     "sample": "every (batch, head) pair over the full sequence, one pass, 1 thread"}
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{k} of {total_pairs} (batch, head) pairs over the full sequence of the {w.name} "
                      f"workload, {passes} pass(es) in {t:.2f} s; tokens/s scaled by the sampled fraction",
            "cpu_model": cpu_model(), "single_core": one}


def spin_cycles(torch, stream, us):
    """Argument of torch.cuda._sleep (a bounded GPU spin) lasting about `us`
    microseconds on this GPU, measured once."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(1_000_000)
    b.record(stream)
    torch.cuda.synchronize()
    return int(1_000_000 * us / max(a.elapsed_time(b) * 1e3, 1.0))


def time_backward(ops, torch, t, sh, steps, fwd_ms=None, modes=("bf16", "f32"), t_alt=None):
    """ssd_backward at the workload (dy in the input dtype, dL/dfinal given),
    `steps` calls per matrix-operand mode after two untimed ones; with t_alt
    the calls alternate between the two batches (each with its own dy)."""
    B, L, H, P = t["x"].shape
    N = t["Bm"].shape[3]
    dev, stream = t["x"].device, torch.cuda.current_stream()
    g = torch.Generator(device=dev).manual_seed(9)
    batches = []
    for tk in (t,) if t_alt is None else (t, t_alt):
        dyb = torch.randn((B, L, H, P), device=dev, generator=g).to(t["x"].dtype)
        dfb = torch.randn((B, H, N, P), device=dev, generator=g)
        batches.append((tk, dyb, dfb))
    wsb = torch.empty(ops.ssd_backward_workspace_bytes(sh), device=dev, dtype=torch.uint8)
    out = {"steps": steps, "workspace_GB": round(wsb.numel() / 1e9, 2)}
    for bm in modes:
        def step_b(k):
            tk, dyb, dfb = batches[k % len(batches)]
            ops.ssd_backward(sh, tk["x"], tk["dt"], tk["A"], tk["Bm"], tk["Cm"], tk["D"], dyb, dfinal=dfb,
                             workspace=wsb, mma=bm)
        for k in range(2):
            step_b(k)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for k in range(steps):
            step_b(k)
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / steps
        out[f"mma_{bm}"] = {"ms": round(bms, 4), "tokens_per_s": round(B * L / (bms * 1e-3), 1)}
        if fwd_ms:
            out[f"mma_{bm}"]["vs_forward_ms"] = round(bms / fwd_ms, 2)
    del batches, wsb
    return out


def time_fp32_path(ops, torch, t, t_alt, sh, w, stream, steps):
    """ssd_forward with fp32 matrix operands (fp32 y) at the workload, steps
    alternating between the batches t and t_alt, and its chunk-state and
    chunk-scan kernels against the fp32 matrix-core peak."""
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = -(-L // Q)
    dev = t["x"].device
    y = torch.empty((B, L, H, P), device=dev, dtype=torch.float32)
    fin = torch.empty((B, H, N, P), device=dev, dtype=torch.float32)
    ws = torch.empty(ops.ssd_workspace_bytes(sh), device=dev, dtype=torch.uint8)
    y_alt = torch.empty_like(y)
    batches = ((t, y), (t_alt, y_alt))

    def fwd(k):
        tk, yk = batches[k & 1]
        ops.ssd_forward(sh, tk["x"], tk["dt"], tk["A"], tk["Bm"], tk["Cm"], tk["D"], y=yk, final_states=fin,
                        workspace=ws, mma="f32")
    dA = torch.empty((B, H, nc, Q), device=dev, dtype=torch.float32)
    dtb = torch.empty_like(dA)
    st = torch.empty((B, nc, H, N, P), device=dev, dtype=torch.float32)
    calls = {
        "chunk_cumsum_state": lambda: ops.ssd_chunk_cumsum_state(sh, t["x"], t["Bm"], t["dt"], t["A"], dA_cumsum=dA,
                                                                 dt_bhl=dtb, states=st, mma="f32"),
        "state_passing": lambda: ops.ssd_state_passing(sh, st, dA, carried=st, final_states=fin),
        "chunk_scan": lambda: ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, st, t["D"], y=y, mma="f32"),
    }
    for k in range(6):
        fwd(k)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(steps):
        fwd(k)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    in_bytes = 2 if w.in_dtype == "bf16" else 4
    costs = algorithmic_costs(w, in_bytes, 4, 4, 4)
    # Per-kernel rows: two untimed passes over the calls first (the first
    # launch of an instance pays for loading its code object), then per timed
    # launch a short GPU spin lets the host queue the events and the call; one
    # launch per event pair; median and min over the pairs.
    for _ in range(2):
        for c in calls.values():
            c()
    torch.cuda.synchronize()
    spin = spin_cycles(torch, stream, 200)
    evs = {k: [] for k in calls}
    for _ in range(max(5, steps // 5)):
        for k, c in calls.items():
            torch.cuda._sleep(spin)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            c()
            e1.record(stream)
            evs[k].append((e0, e1))
    torch.cuda.synchronize()
    out = {"ms": round(ms, 4), "tokens_per_s": round(w.tokens / (ms * 1e-3), 1), "y_dtype": "f32",
           "steps": steps, "mfma_peak_TFLOPs": MFMA_PEAK_TFLOPS["f32"], "kernels": {}}
    for k, pairs in evs.items():
        ts = sorted(1e3 * e0.elapsed_time(e1) for e0, e1 in pairs)
        us = ts[len(ts) // 2]
        c = costs[k]
        tf = c["flops"] / (us * 1e-6) / 1e12
        out["kernels"][k] = {"us_median": round(us, 2), "us_min": round(ts[0], 2), "TFLOPs": round(tf, 2),
                             "mfma_peak_frac": round(tf / MFMA_PEAK_TFLOPS["f32"], 4),
                             "GBps": round(c["bytes"] / (us * 1e-6) / 1e9, 1)}
    del y, y_alt, fin, ws, dA, dtb, st
    return out


def sweep_tuning(ops, torch, names, mma, reps=40):
    """ssd_forward at each workload under every launch choice the tuning table
    holds (the SSD_TUNE override, read by the library at every call): the
    heads per block of the chunk-scan kernel, the state path, and for the
    two-kernel state path the heads per block of the chunk-state kernel.  One
    JSON line per workload: ms per call of every variant and the fastest."""
    from mamba_ssd_scan_chunk_amd.inputs import WORKLOADS, workload_inputs
    stream = torch.cuda.current_stream()
    for name in names:
        w = WORKLOADS[name]
        t = workload_inputs(name).to_torch("cuda")
        sh = ops.shape_of(t, w.chunk)
        y_dtype = w.in_dtype if mma == "bf16" else "f32"
        y = torch.empty(tuple(t["x"].shape), device="cuda",
                        dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32)
        fin = torch.empty((w.batch, w.nheads, w.dstate, w.headdim), device="cuda", dtype=torch.float32)
        ws = torch.empty(ops.ssd_workspace_bytes(sh), device="cuda", dtype=torch.uint8)

        def time_variant(tune):
            os.environ["SSD_TUNE"] = tune
            call = lambda: ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], y=y,
                                           final_states=fin, workspace=ws, mma=mma)
            for _ in range(10):
                call()
            best = None
            for _ in range(3):
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    call()
                b.record(stream)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / reps
                best = ms if best is None else min(best, ms)
            return round(best, 4)

        hpg = w.nheads // w.ngroups
        divs = [k for k in range(1, hpg + 1) if hpg % k == 0]
        out = {"workload": name, "mma": mma, "variants": {}}
        time_variant("")  # clocks and caches warm before the first timed variant
        out["variants"]["rule"] = time_variant("")
        scan = {k: time_variant(f"scan_hg={k}") for k in divs}
        for k, v in scan.items():
            out["variants"][f"scan_hg={k}"] = v
        bs = min(scan, key=scan.get)
        for path in ("fused", "split"):
            out["variants"][f"path={path},scan_hg={bs}"] = time_variant(f"path={path},scan_hg={bs}")
        for k in divs:
            tune = f"path=split,scan_hg={bs},state_hg={k}"
            out["variants"][tune] = time_variant(tune)
        os.environ.pop("SSD_TUNE", None)
        best = min(out["variants"], key=out["variants"].get)
        out["best"] = {"variant": best, "ms": out["variants"][best], "rule_ms": out["variants"]["rule"]}
        print(json.dumps(out), flush=True)
        del t, y, fin, ws
        torch.cuda.empty_cache()


def time_packed(ops, torch, batches, sh, w, fin, steps, nseq_row, mma, stream):
    """ssd_forward_varlen at the workload's shape: each row cut into nseq_row
    sequences at seeded random points, the two input batches alternating;
    10 untimed calls, then `steps` calls between one pair of events."""
    import numpy as np
    B, L = w.batch, w.seqlen
    dev = batches[0][0]["x"].device
    rng = np.random.default_rng(11)
    seq = np.zeros((B, L), np.int32)
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, L), size=nseq_row - 1, replace=False))
        seq[b] = np.searchsorted(cuts, np.arange(L), side="right") + b * nseq_row
    seq_t = torch.from_numpy(seq).to(dev)
    wsv = torch.empty(ops.ssd_workspace_bytes_varlen(sh), device=dev, dtype=torch.uint8)

    def step_v(k):
        tk, yk = batches[k & 1]
        ops.ssd_forward_varlen(sh, tk["x"], tk["dt"], tk["A"], tk["Bm"], tk["Cm"], tk["D"], seq_t, y=yk,
                               final_states=fin, workspace=wsv, mma=mma)
    for k in range(10):
        step_v(k)
    torch.cuda.synchronize()
    v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    v0.record(stream)
    for k in range(steps):
        step_v(k)
    v1.record(stream)
    torch.cuda.synchronize()
    vms = v0.elapsed_time(v1) / steps
    return {"sequences_per_row": nseq_row, "ms": round(vms, 5),
            "tokens_per_s": round(w.tokens / (vms * 1e-3), 1), "call": "ssd_forward_varlen"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="warm-up also lasts at least this long (seconds of back-to-back steps)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--mma", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32-path", action="store_true",
                    help="skip timing the fp32-operand forward beside the bf16 one")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="forwards timed one by one after a 1 GiB cache flush (0: skip)")
    ap.add_argument("--decode-batch", type=int, default=64,
                    help="sequences in the timed single-token decode step (0: skip it)")
    ap.add_argument("--varlen-seqs", type=int, default=16,
                    help="sequences packed per row for the ssd_forward_varlen line (0: skip it)")
    ap.add_argument("--packed-only", action="store_true",
                    help="time only ssd_forward_varlen (--varlen-seqs per row, --steps calls) and print that")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="gradient calls (ssd_backward) timed at the workload (0: skip)")
    ap.add_argument("--backward-only", default=None, choices=["bf16", "f32"],
                    help="time only ssd_backward in this operand mode (--backward-steps calls) and print that")
    ap.add_argument("--no-cumsum-sweep", dest="cumsum_sweep", action="store_false",
                    help="skip the chunk_cumsum bandwidth-vs-length sweep")
    ap.add_argument("--kernel-reps", type=int, default=4,
                    help="back-to-back launches of each call between one pair of events in the per-kernel rows")
    ap.add_argument("--kernel-only", default=None,
                    help="time only this ABI call in the per-kernel loop (for profiling)")
    ap.add_argument("--sweep-tuning", action="store_true",
                    help="time ssd_forward under every launch choice of the per-shape tuning table at each "
                         "workload (or --workload) and print one JSON line per workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode to measure", file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_ssd_scan_chunk_amd import ops
    from mamba_ssd_scan_chunk_amd._lib import LIB_PATH
    from mamba_ssd_scan_chunk_amd.inputs import HEADLINE, WORKLOADS, workload_inputs

    if not os.path.exists(LIB_PATH):
        from mamba_ssd_scan_chunk_amd import build as hip_build
        hip_build.build()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.sweep_tuning:
        names = [args.workload] if args.workload else [n for n in WORKLOADS if WORKLOADS[n].in_dtype == "bf16"]
        sweep_tuning(ops, torch, names, args.mma)
        return

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    inp = workload_inputs(name)
    t = inp.to_torch("cuda")
    t_alt = workload_inputs(name, seed=w.seed + 1).to_torch("cuda")  # the second batch of the timed loop
    sh = ops.shape_of(t, w.chunk)
    dev = t["x"].device
    in_bytes = 2 if w.in_dtype == "bf16" else 4
    y_dtype = w.in_dtype if args.mma == "bf16" else "f32"
    y_bytes = 2 if y_dtype == "bf16" else 4
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = L // Q
    y = torch.empty((B, L, H, P), device=dev, dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32)
    fin = torch.empty((B, H, N, P), device=dev, dtype=torch.float32)
    ws = torch.empty(ops.ssd_workspace_bytes(sh), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    if args.backward_only:
        bwd = time_backward(ops, torch, t, sh, max(args.backward_steps, 1), modes=(args.backward_only,))
        print(json.dumps({"workload": name, "backward": bwd}), flush=True)
        return

    y_alt = torch.empty_like(y)
    batches = ((t, y), (t_alt, y_alt))
    if args.packed_only:
        packed = time_packed(ops, torch, batches, sh, w, fin, args.steps, max(args.varlen_seqs, 1), args.mma, stream)
        print(json.dumps({"workload": name, "forward_packed_sequences": packed}), flush=True)
        return

    def step(k=0):
        tk, yk = batches[k & 1]
        ops.ssd_forward(sh, tk["x"], tk["dt"], tk["A"], tk["Bm"], tk["Cm"], tk["D"], y=yk, final_states=fin,
                        workspace=ws, mma=args.mma)

    # ---- phase 1: whole-path throughput
    warm_run = 0
    warm0 = time.perf_counter()
    while warm_run < args.warmup or time.perf_counter() - warm0 < args.min_warmup_s:
        step(warm_run)
        warm_run += 1
        if warm_run % 16 == 0:
            torch.cuda.synchronize()  # keep the wall clock in step with the GPU
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        step(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    tokens_per_s = w.tokens / (ms_per_step / 1e3)
    # the same number of steps all on the first batch
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(args.steps):
        step(0)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_repeat = r0.elapsed_time(r1) / args.steps
    repeat = {"ms": round(ms_repeat, 5), "tokens_per_s": round(w.tokens / (ms_repeat / 1e3), 1),
              "note": "every step on the same batch: part of its inputs stay in the last-level cache"}

    # Cold-cache forwards (reported beside the line, not as its value): before
    # each timed forward, 1 GiB (four times the last-level cache) is written
    # outside the timed region, so inputs and intermediates come from HBM.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
        cold_ms = []
        for _ in range(args.cold_steps):
            flush.fill_(1.0)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold_ms.append(c0.elapsed_time(c1))
        del flush
        cold_ms.sort()
        med = cold_ms[len(cold_ms) // 2]
        cold = {"steps": args.cold_steps, "ms_median": round(med, 5), "ms_min": round(cold_ms[0], 5),
                "tokens_per_s_median": round(w.tokens / (med / 1e3), 1)}

    # ---- phase 2: per-kernel durations of the calls ssd_forward makes
    # (bf16-operand path: chunk states stored as bf16, carried states written
    # over them as bf16; fp32 path: fp32 in place), events on the launch stream
    dA = torch.empty((B, H, nc, Q), device=dev, dtype=torch.float32)
    dtb = torch.empty_like(dA)
    carried_bytes = states_bytes = 2 if args.mma == "bf16" else 4
    states = torch.empty((B, nc, H, N, P), device=dev,
                         dtype=torch.bfloat16 if states_bytes == 2 else torch.float32)
    carried = states
    # the fused state path writes its bf16 carried states to a buffer of its own
    carried_fused = torch.empty((B, nc, H, N, P), device=dev, dtype=torch.bfloat16) if args.mma == "bf16" else states
    # ssd_forward takes the fused state path (chunk states never stored) where
    # it is supported and has at least two blocks per compute unit; the other
    # state path, where supported, is timed too (reported under "other_path")
    fused_ok = args.mma == "bf16" and N % 64 == 0 and P % 64 == 0 and w.in_dtype == "bf16"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = 128 if (N % 128 == 0 and Q <= 128) else 64  # state rows per block of the fused kernel
    fused = fused_ok and B * H * (N // rows) * (P // 64) >= 2 * cus
    fused_call = lambda: ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, carried=carried_fused,
                                                     final_states=fin, mma=args.mma)
    cumsum_call = lambda: ops.ssd_chunk_cumsum(sh, t["dt"], t["A"], dA_cumsum=dA, dt_bhl=dtb)
    state_call = lambda: ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, states=states, mma=args.mma)
    passing_call = lambda: ops.ssd_state_passing(sh, states, dA, carried=carried, final_states=fin)
    calls = {}
    if fused:
        calls["chunk_cumsum"] = cumsum_call
        calls["chunk_state_passing"] = fused_call
    else:
        # the forward's first step: the cumulative sums inside the chunk-state
        # kernel where that has a head-group instance (else the two launches)
        calls["chunk_cumsum_state"] = lambda: ops.ssd_chunk_cumsum_state(
            sh, t["x"], t["Bm"], t["dt"], t["A"], dA_cumsum=dA, dt_bhl=dtb, states=states, mma=args.mma)
        calls["state_passing"] = passing_call
    scan_carried = carried_fused if fused else carried
    calls["chunk_scan"] = lambda: ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, scan_carried, t["D"],
                                                     y=y, mma=args.mma)
    forward_kernels = list(calls)
    # calls outside this forward, timed beside it: the split first step and
    # the other state path
    if fused:
        calls["chunk_state"] = state_call
        calls["state_passing"] = passing_call
    else:
        calls["chunk_cumsum"] = cumsum_call
        calls["chunk_state"] = state_call
        if fused_ok:
            calls["chunk_state_passing"] = fused_call
    order = list(calls) if args.kernel_only is None else [args.kernel_only]
    for _ in range(2):
        for k in calls:
            calls[k]()
    torch.cuda.synchronize()
    # Each timed step starts with a bounded GPU spin (~1 ms) that keeps the
    # GPU busy while the host queues the step's calls and events, so every
    # event pair brackets GPU time only: no host submission gap inflates the
    # small kernels.  Each pair brackets REPS back-to-back launches of one call
    # (the dispatch gap between a kernel and the event before it would
    # otherwise count against short kernels); the per-launch time is the
    # pair's time over REPS.  The calls outside the forward are timed one
    # launch per pair: repeated, their input rows would stay in the
    # last-level cache between launches, unlike in any forward.
    reps = max(1, args.kernel_reps)
    kreps = {k: (reps if k in forward_kernels else 1) for k in calls}
    spin = spin_cycles(torch, stream, 1000)
    evs = {k: [] for k in order}
    for _ in range(args.steps):
        torch.cuda._sleep(spin)
        for k in calls:
            if k in evs:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _r in range(kreps[k]):
                    calls[k]()
                b.record(stream)
                evs[k].append((a, b))
            else:
                calls[k]()
    torch.cuda.synchronize()
    costs = algorithmic_costs(w, in_bytes, y_bytes, carried_bytes, states_bytes)
    peak_t = MFMA_PEAK_TFLOPS[args.mma]

    def row(k, us):
        c = costs[k]
        gbps = c["bytes"] / (us * 1e-6) / 1e9
        tflops = c["flops"] / (us * 1e-6) / 1e12
        roof_t = min(peak_t, c["flops"] / c["bytes"] * HBM_PEAK_GBPS / 1e3)
        return {"us": round(us, 2), "alg_bytes": c["bytes"], "alg_flops": c["flops"],
                "GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                "TFLOPs": round(tflops, 2), "mfma_peak_frac": round(tflops / peak_t, 4),
                "frac_of_roof": round(tflops / roof_t, 4)}

    kernels = {k: row(k, 1e3 * sum(a.elapsed_time(b) for a, b in pairs) / (len(pairs) * kreps[k]))
               for k, pairs in evs.items()}
    other = {k: kernels.pop(k) for k in list(kernels) if k not in forward_kernels and len(kernels) > 1}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dk["GBps"] / HBM_PEAK_GBPS, 4), "traffic": None}

    # Cold per-kernel rows: before each timed launch 1 GiB (four times the
    # last-level cache) is written, then a short GPU spin lets the host queue
    # the events and the call; one launch per event pair; median and min.
    kernels_cold = None
    if args.cold_steps > 0 and args.kernel_only is None:
        flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
        spin_c = spin_cycles(torch, stream, 200)
        kernels_cold = {}
        for k in forward_kernels:
            ts = []
            for _ in range(args.cold_steps):
                flush.fill_(1.0)
                torch.cuda._sleep(spin_c)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                calls[k]()
                b.record(stream)
                torch.cuda.synchronize()
                ts.append(1e3 * a.elapsed_time(b))
            ts.sort()
            r = row(k, ts[len(ts) // 2])
            kernels_cold[k] = {"us_median": r["us"], "us_min": round(ts[0], 2), "GBps": r["GBps"],
                               "hbm_frac": r["hbm_frac"], "mfma_peak_frac": r["mfma_peak_frac"]}
        del flush

    # The bf16-operand forward with fp32 chunk states (the chunk states stored
    # in fp32, the carried states handed to the chunk scan as bf16).
    fwd_f32_states = None
    if args.mma == "bf16" and not fused and args.kernel_only is None:
        st32 = torch.empty((B, nc, H, N, P), device=dev, dtype=torch.float32)
        hb = torch.empty((B, nc, H, N, P), device=dev, dtype=torch.bfloat16)

        def step32(k):
            tk, yk = batches[k & 1]
            ops.ssd_chunk_cumsum_state(sh, tk["x"], tk["Bm"], tk["dt"], tk["A"], dA_cumsum=dA, dt_bhl=dtb,
                                       states=st32, mma="bf16")
            ops.ssd_state_passing(sh, st32, dA, carried=hb, final_states=fin)
            ops.ssd_chunk_scan(sh, tk["x"], tk["Bm"], tk["Cm"], dtb, dA, hb, tk["D"], y=yk, mma="bf16")
        for k in range(20):
            step32(k)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(args.steps):
            step32(k)
        b.record(stream)
        torch.cuda.synchronize()
        ms32 = a.elapsed_time(b) / args.steps
        fwd_f32_states = {"ms": round(ms32, 5), "tokens_per_s": round(w.tokens / (ms32 * 1e-3), 1),
                          "calls": "ssd_chunk_cumsum_state (fp32 states) -> ssd_state_passing (bf16 carried) "
                                   "-> ssd_chunk_scan"}
        del st32, hb

    # The fp32-operand path (fp32 matrix operands, fp32 chunk and carried
    # states, fp32 y): whole forward and its two contraction kernels against
    # the fp32 matrix-core peak.
    fp32_path = None
    if args.mma == "bf16" and not args.no_fp32_path and args.kernel_only is None:
        fp32_path = time_fp32_path(ops, torch, t, t_alt, sh, w, stream, max(10, args.steps // 2))

    # Packed sequences (ssd_forward_varlen) at the same shape
    varlen = None
    if args.varlen_seqs > 0 and args.kernel_only is None:
        varlen = time_packed(ops, torch, batches, sh, w, fin, args.steps, args.varlen_seqs, args.mma, stream)

    # Single-token decode step at the same layer shape: DECODE_BATCH sequences,
    # one token each, fp32 state advanced in place (8 N P bytes per (b, h)).
    dec = None
    if args.decode_batch > 0:
        DB = args.decode_batch
        g = torch.Generator(device=dev).manual_seed(7)
        io_dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
        xd = torch.randn((DB, H, P), device=dev, generator=g).to(io_dt)
        dtd = torch.nn.functional.softplus(torch.randn((DB, H), device=dev, generator=g) - 2.0)
        Bd = torch.randn((DB, G, N), device=dev, generator=g).to(io_dt)
        Cd = torch.randn((DB, G, N), device=dev, generator=g).to(io_dt)
        sd = torch.randn((DB, H, N, P), device=dev, generator=g)
        yd = torch.empty((DB, H, P), device=dev, dtype=io_dt)
        step_d = lambda: ops.ssd_decode_step(xd, dtd, t["A"], Bd, Cd, t["D"], sd, y=yd)
        for _ in range(20):
            step_d()
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(args.steps):
            step_d()
        d1.record(stream)
        torch.cuda.synchronize()
        dus = 1e3 * d0.elapsed_time(d1) / args.steps
        dbytes = 8 * DB * H * N * P + xd.element_size() * (2 * DB * H * P + 2 * DB * G * N) + 4 * DB * H + 8 * H
        dec = {"batch": DB, "us": round(dus, 2), "tokens_per_s": round(DB / (dus * 1e-6), 1),
               "alg_bytes": dbytes, "GBps": round(dbytes / (dus * 1e-6) / 1e9, 1),
               "hbm_frac": round(dbytes / (dus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        del xd, dtd, Bd, Cd, sd, yd

    # Gradient call at the same workload, reported beside the forward.
    bwd = (time_backward(ops, torch, t, sh, args.backward_steps, ms_per_step, t_alt=t_alt)
           if args.backward_steps > 0 else None)

    # ssd_chunk_cumsum alone against sequence length at the workload's B and H:
    # at the headline (B L H = 1.3 M tokens x heads, 15.7 MB) launch and ramp
    # dominate; the sweep shows where the kernel reaches the HBM roofline.
    sweep = []
    if args.cumsum_sweep:
        for Ls in (L, 4 * L, 16 * L, 64 * L):
            Ls = (Ls // Q) * Q
            shs = ops.SSDShape.make(B, Ls, H, P, N, G, Q)
            dts = torch.rand((B, Ls, H), device=dev) * 0.5
            dAs = torch.empty((B, H, Ls // Q, Q), device=dev)
            dtbs = torch.empty_like(dAs)
            call = lambda: ops.ssd_chunk_cumsum(shs, dts, t["A"], dA_cumsum=dAs, dt_bhl=dtbs)
            for _ in range(10):
                call()
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 50
            torch.cuda._sleep(spin_cycles(torch, stream, 2000))  # the host queues all reps meanwhile
            s0.record(stream)
            for _ in range(reps):
                call()
            s1.record(stream)
            torch.cuda.synchronize()
            sus = 1e3 * s0.elapsed_time(s1) / reps
            sbytes = 12 * B * Ls * H + 4 * H
            sweep.append({"seqlen": Ls, "MB": round(sbytes / 1e6, 1), "us": round(sus, 2),
                          "GBps": round(sbytes / (sus * 1e-6) / 1e9, 1),
                          "hbm_frac": round(sbytes / (sus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
            del dts, dAs, dtbs

    # One elementwise copy of 512 MiB (a single kernel dispatch): its measured
    # rate is the practical HBM ceiling, and under rocprofv3 --pmc its
    # FETCH_SIZE / WRITE_SIZE per dispatch (known to be 512 MiB each)
    # calibrate the same counters read for the SSD kernels.
    src = torch.ones(1 << 27, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        torch.add(src, 0.0, out=dst)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    roofline["traffic"] = measured_traffic(name, dom)

    flops_total = sum(costs[k]["flops"] for k in forward_kernels)
    out = {
        "metric": "Mamba-2 SSD fwd tokens/s (2.7B-layer shape) + % MFMA / HBM roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_run,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mma == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{name}: B={B} L={L} H={H} P={P} N={N} G={G} Q={Q}", "batch": B, "seqlen": L,
                   "nheads": H, "headdim": P, "dstate": N, "ngroups": G, "chunk": Q, "in_dtype": w.in_dtype,
                   "y_dtype": y_dtype, "mma": args.mma, "parallelism": "single GPU"},
        "effective_TFLOPs": round(flops_total / (ms_per_step * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 4),
        "roofline": roofline,
        "kernels": kernels,
        "kernels_cold": kernels_cold,
        "state_path": "fused" if fused else "two-kernel",
        "other_path": other,
        "forward_fp32_chunk_states": fwd_f32_states,
        "fp32_mma_path": fp32_path,
        "copy_GBps": round(copy_gbps, 1),
        "cold_cache": cold,
        "repeat_batch": repeat,
        "decode_step": dec,
        "forward_packed_sequences": varlen,
        "backward": bwd,
        "cumsum_sweep": sweep,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
