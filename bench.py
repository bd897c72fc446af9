#!/usr/bin/env python3
"""Benchmark of the MI355X GDN recurrent decode step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]

Default workload (one "step" = one decode step of every state unit, one
launch): 64 sequences x 48 GDN layers = 3072 independent fp32 states of
48 value heads x 128 x 128 (9.66 GB), vh=48, kh=16, kd=vd=128, seeded
synthetic inputs resident in HBM before timing.  Prints one JSON line with
head-steps/s, the achieved algorithmic HBM bandwidth of the recurrence kernel
against MI355X's 8 TB/s, the measured read+write copy floor, and the CPU
oracle timed on a bounded sample of the same workload.

Other --config values time the other workloads: 0 single sequence x 1 layer
x 64 sequential steps (launch latency), 2 speculative verify (mark + 8-row
step_m + rollback), 3 front end + step, 4 large batch, 5 large batch at
kd=vd=64, 6 speculative verify of one layer with its front end, 7 the
batched decode of workload 1 with the gated RMSNorm fused on the output,
8 and 9 whole layers (projections, front end, gated step) with f32 weights
for 1 and 64 sequences, 10 the whole-layer speculative verify, 11 whole
layers with 4-bit weights and binary16 block scales for 1 sequence, 12 the
whole-layer speculative verify with 4-bit weights.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_deltanet_recurrent_amd as gdn  # noqa: E402
import synth  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
NAMES = ("q", "k", "v", "g", "beta")
METRIC = "GDN head-steps/sec and achieved HBM GB/s (% of MI355X peak), 1 GPU"
KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_recurrent_amd", "csrc", "gdn_kernels.hip")


def frontend_bytes(B, dims, M=1, write_hist=True, dim=5120):
    """Algorithmic HBM bytes of one front-end launch over M rows of B units:
    x and the raw conv inputs per row, Wa and Wb, the conv weights, the
    3-frame history read once (and written once), and the q, k, v, g, beta
    outputs per row."""
    vh, kh, kd, vd = dims
    cd = synth.conv_dim_of(dims)
    return (M * B * dim * 4 + 2 * vh * dim * 4 + M * B * cd * 4
            + (2 if write_hist else 1) * B * 3 * cd * 4 + cd * 16
            + M * B * (2 * kh * kd + vh * vd + 2 * vh) * 4)


def head_step_bytes(dims, rows=1, write_o=True, read_state=True):
    """Algorithmic HBM bytes of one head-step when `rows` steps share one
    state read and one state write (rows=1: a plain step)."""
    vh, kh, kd, vd = dims
    rep = vh // kh
    state = (kd * vd * 4 * (1 if read_state else 0) + kd * vd * 4) / rows
    per_row = vd * 4 + (vd * 4 if write_o else 0) + 8 + 2 * kd * 4 / rep
    return state + per_row


# The parts of the kernel source each measured kernel is built from (the
# shared helpers after the file's header comment, then its own section), so
# that an edit elsewhere in the file does not invalidate its recorded
# counters.
_Q4_SECTION = b"// " + b"-" * 75 + b"\n// Dense layer projections with 4-bit weights"
_RECUR_COMMON = (b"namespace gdn {", b"// ----- wide geometry -")
_RECUR_LAUNCH = (b"// Launches of fewer than kWidemBelow tiles", b"// Streaming copy")
_HEAD = (b"namespace gdn {", b"// Recurrence\n")
HASH_SECTIONS = {
    "recur_wide_kernel": ((b"namespace gdn {", b"// ----- wide geometry, several steps"),
                          _RECUR_LAUNCH),
    "recur_widem_kernel": (_RECUR_COMMON,
                           (b"// ----- wide geometry, several steps", b"// ----- deep geometry"),
                           _RECUR_LAUNCH),
    "recur_deep_kernel": (_RECUR_COMMON, (b"// ----- deep geometry", b"// ----- split geometry"),
                          _RECUR_LAUNCH),
    "recur_split_kernel": (_RECUR_COMMON, (b"// ----- split geometry", _RECUR_LAUNCH[0]),
                           _RECUR_LAUNCH),
    "copy_kernel": (_HEAD, (b"// Streaming copy", b"// Per-unit step counts")),
    "fe_kernel": (_HEAD, (b"// Front end, kernel A", b"// y0[0..n0) = 0")),
    "proj_kernel": ((b"namespace gdn {", b"// Recurrence\n"),
                    (b"// Dense layer projections", _Q4_SECTION), (b"}  // namespace gdn", None)),
    "proj_q4_kernel": ((b"namespace gdn {", b"// Recurrence\n"), (_Q4_SECTION, None)),
}


def kernel_hash(kernel="recur_wide_kernel"):
    """sha256[:16] of the kernel-source sections `kernel` is built from."""
    src = open(KERNEL_SRC, "rb").read()
    h = hashlib.sha256()
    for start, end in HASH_SECTIONS[kernel]:
        a = 0 if start is None else src.find(start)
        b = len(src) if end is None else src.find(end)
        if a < 0 or b < 0:
            raise RuntimeError(f"kernel source layout changed: section marker of {kernel} not found")
        h.update(src[a:b])
    return h.hexdigest()[:16]


def recorded_traffic(workload_key, launches_bytes, kernel="recur_wide_kernel"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_key}_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed(fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3            # seconds


def timed_graph(fn, steps, warmup):
    """fn(0) captured once as a HIP graph, then `steps` replays timed like
    timed(): the launch chain without host gaps (fn must allocate nothing)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn(0)
    return timed(lambda i: graph.replay(), steps, warmup)


def graph_launch_s(fn, steps, per_graph=10):
    """Seconds per call of fn when per_graph calls are captured as one HIP
    graph and replayed: the device-paced launch time, without host gaps."""
    return timed_graph(lambda i: [fn() for _ in range(per_graph)], steps, 1) / (steps * per_graph)


def cpu_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def cpu_info():
    """Online host cores and the CPU model string."""
    online = os.sysconf("SC_NPROCESSORS_ONLN") if hasattr(os, "sysconf") else None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return online, model


def over_ranges(fn, n, chunk, threads):
    """fn(lo, hi) over consecutive ranges of n units on a pool of host threads
    (the oracle releases the GIL); results in range order."""
    from concurrent.futures import ThreadPoolExecutor
    ranges = [(lo, min(lo + chunk, n)) for lo in range(0, n, chunk)]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


class Tol:
    """Elements outside |x - r| <= max(1e-5 |r|, floor) and the pages'
    max|err| / max|ref| ("Kestrel_VLLM #24", section 6), over many ranges."""

    def __init__(self):
        self.bad, self.n, self.max_err, self.max_ref = 0, 0, 0.0, 0.0

    def add(self, x, r, floor=1e-6):
        x = np.asarray(x, np.float64)
        r = np.asarray(r, np.float64)
        err = np.abs(x - r)
        bad = (err > np.maximum(1e-5 * np.abs(r), floor)) | (np.isnan(x) != np.isnan(r))
        self.bad += int(np.count_nonzero(bad))
        self.n += x.size
        if x.size:
            self.max_err = max(self.max_err, float(np.nanmax(err)))
            self.max_ref = max(self.max_ref, float(np.nanmax(np.abs(r))))
        return self

    def merge(self, o):
        self.bad += o.bad
        self.n += o.n
        self.max_err = max(self.max_err, o.max_err)
        self.max_ref = max(self.max_ref, o.max_ref)
        return self

    def rec(self):
        return dict(elements=self.n, out_of_tolerance=self.bad,
                    max_rel_pages=(self.max_err / self.max_ref) if self.max_ref else self.max_err)


def merged(results, k):
    t = Tol()
    for r in results:
        t.merge(r[k])
    return t


def gated_floor(o_ref, z, w, eps):
    """o's absolute floor (1e-6) carried through the gated norm's per-head
    scale s = w silu(z) / sqrt(mean(o^2) + eps)."""
    o64, z64 = o_ref.astype(np.float64), z.astype(np.float64)
    rinv = 1.0 / np.sqrt(np.mean(o64 ** 2, axis=-1, keepdims=True) + eps)
    return 1e-6 * np.abs(rinv * w.astype(np.float64) * z64 / (1.0 + np.exp(-z64)))


def decode_cpu_and_parity(S0, pool, dims, steps, gated=None):
    """The CPU oracle, as it stands, on every unit of the workload for `steps`
    decode steps (inputs cycled from the pool as in the timed loop), timed on
    a pool of host threads, plus a single-thread run of the first 3 steps of
    the first units; then the GPU reruns the same steps from the same initial
    state (one launch over all units per step) and every element of o and of
    the final S is compared with the oracle's.  gated = (z per pool entry,
    norm_w, eps) for the gated-output workload."""
    import oracle
    orc = oracle.load()
    vh, kh, kd, vd = dims
    N = S0.shape[0]
    th = cpu_threads()
    online, model = cpu_info()
    xs = [{n: host(pool[r % len(pool)][n][0]) for n in NAMES} for r in range(steps)]
    # single thread: the first 3 steps of the first units (under a second of work)
    n1 = min(N, 256)
    S1 = host(S0[:n1])
    o1 = np.zeros((n1, vh, vd), np.float32)
    t0 = time.perf_counter()
    for r in range(min(3, steps)):
        orc.gdn_step(S1, *(np.ascontiguousarray(xs[r][n][:n1]) for n in NAMES), o1, dims)
    dt1 = time.perf_counter() - t0
    hs1 = n1 * vh * min(3, steps)
    # every unit, all threads, timed (in place on the host copy)
    S_h = host(S0)
    O_ref = np.zeros((steps, N, vh, vd), np.float32)

    def work(lo, hi):
        for r in range(steps):
            orc.gdn_step(S_h[lo:hi], *(np.ascontiguousarray(xs[r][n][lo:hi]) for n in NAMES),
                         O_ref[r, lo:hi], dims)

    t0 = time.perf_counter()
    over_ranges(work, N, max(1, (N + 4 * th - 1) // (4 * th)), th)
    dt = time.perf_counter() - t0
    hs = N * vh * steps
    cpu = dict(value=hs / dt, unit="head-steps/s", cores=th, kind="oracle",
               sample=f"every unit of the workload ({N} units) x {steps} steps = {hs} head-steps, "
                      f"{dt:.2f} s wall on {th} threads; single thread: the first "
                      f"{min(3, steps)} steps of {n1} units, {dt1:.2f} s",
               threads_used=th, online_cores=online, cpu_model=model,
               single_thread_value=hs1 / dt1, single_thread_sample=f"{n1} units x {min(3, steps)} steps")
    # the GPU on the same steps, then every element against the oracle
    S = S0.clone()
    O = torch.empty((steps, N, vh, vd), device=S0.device)
    for r in range(steps):
        x = pool[r % len(pool)]
        if gated:
            gdn.step_gated(S, *(x[n] for n in NAMES), gated[0][r % len(pool)], gated[1],
                           gated[2], out=O[r:r + 1])
        else:
            gdn.step(S, *(x[n][0] for n in NAMES), o=O[r])
    torch.cuda.synchronize()
    if gated:
        z_h = [host(z) for z in gated[0]]
        w_h = host(gated[1])

    def check(lo, hi):
        to, ts = Tol(), Tol()
        for r in range(steps):
            ref = O_ref[r, lo:hi]
            if gated:
                zz = np.ascontiguousarray(z_h[r % len(pool)][0, lo:hi])
                out = np.zeros_like(ref)
                orc.gated_norm(np.ascontiguousarray(ref), zz, w_h, gated[2], out)
                to.add(host(O[r, lo:hi]), out, gated_floor(ref, zz, w_h, gated[2]))
            else:
                to.add(host(O[r, lo:hi]), ref)
        ts.add(host(S[lo:hi]), S_h[lo:hi])
        return to, ts

    res = over_ranges(check, N, 32, th)
    par = dict(units=N, steps=steps, launch="one launch over all units per step",
               o=merged(res, 0).rec(), S=merged(res, 1).rec())
    if gated:
        par["o_is"] = "the gated output"
    return cpu, par


def host(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def copy_floor(S, reps=5):
    """Read+write floor: stream the state through the same 128-bit access
    pattern and write it back in place."""
    flat = S.view(-1)
    gdn.stream_copy(flat, flat)
    dt = timed(lambda i: gdn.stream_copy(flat, flat), reps, 1)
    return 2 * flat.numel() * 4 * reps / dt / 1e9


def read_floor(S, reps=5):
    """Read-only floor: stream the state with 128-bit non-temporal loads (one
    checksum word per 128 KiB written, 0.003% of the bytes)."""
    flat = S.view(-1)
    words = gdn.stream_read(flat)
    dt = timed(lambda i: gdn.stream_read(flat, words=words), reps, 1)
    return flat.numel() * 4 * reps / dt / 1e9


def bench_decode(cfg, steps, warmup, cpu):
    dims = cfg["dims"]
    vh = dims[0]
    N = cfg["seqs"] * cfg["layers"]
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    pool = [synth.step_inputs(gen, N, dims, M=1, gate=cfg["gate"], device="cuda")
            for _ in range(4)]
    gated = cfg.get("gated", False)
    if gated:
        for x in pool:
            x["z"] = torch.randn((1, N, vh, dims[3]), generator=gen, device="cuda")
        norm_w = 1.0 + 0.1 * torch.randn((dims[3],), generator=gen, device="cuda")
    o = torch.empty((N, vh, dims[3]), device="cuda")
    torch.cuda.synchronize()

    def one(i):
        x = pool[i % 4]
        if gated:
            gdn.step_gated(S, x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], norm_w, 1e-6,
                           out=o.view(1, N, vh, dims[3]))
        else:
            gdn.step(S, x["q"][0], x["k"][0], x["v"][0], x["g"][0], x["beta"][0], o=o)

    dt = timed(one, steps, warmup)
    hs_per_step = N * vh
    bps = head_step_bytes(dims) + (dims[3] * 4 if gated else 0)   # + the gate z
    per_layer = {}
    if not gated and cfg["layers"] > 1:
        # the same step as one launch per layer (each over that layer's
        # seqs units, contiguous), the way a model walks its layers
        L, Bq = cfg["layers"], cfg["seqs"]
        views = [[S[l * Bq:(l + 1) * Bq]] +
                 [[x[n][0][l * Bq:(l + 1) * Bq] for n in NAMES] for x in pool] +
                 [o[l * Bq:(l + 1) * Bq]] for l in range(L)]

        def layers(i):
            for v in views:
                gdn.step(v[0], *v[1 + i % 4], o=v[5])

        dt_l = timed(layers, steps, warmup)
        # the same 48 launches replayed as one graph: what is left of the gap
        # between them is the device's own (one grid drains before the next
        # fills), not the host's launch cost
        dt_lg = timed_graph(layers, steps, warmup)
        per_layer = dict(per_layer_launches=L, per_layer_ms_per_step=round(dt_l / steps * 1e3, 4),
                         per_layer_GBps=round(hs_per_step * bps * steps / dt_l / 1e9, 1),
                         per_layer_graph_ms_per_step=round(dt_lg / steps * 1e3, 4))
    launch_s = dt / steps
    bytes_launch = hs_per_step * bps
    achieved = bytes_launch / launch_s / 1e9
    floor = copy_floor(S)
    rfloor = read_floor(S)
    key = {1: "b64x48", 4: "b512x8", 5: "b512x8_kd64", 7: "b64x48_gated"}.get(
        cfg["id"], f"cfg{cfg['id']}")
    traffic = recorded_traffic(key, bytes_launch)
    res = dict(
        value=hs_per_step * steps / dt, ms_per_step=launch_s * 1e3,
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                      unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4), traffic=traffic),
        extra=dict(copy_floor_GBps=round(floor, 1),
                   frac_of_copy_floor=round(achieved / floor, 4),
                   read_floor_GBps=round(rfloor, 1),
                   algorithmic_bytes_per_launch=int(bytes_launch),
                   bytes_per_head_step=round(bps, 2), head_steps_per_step=hs_per_step,
                   kernel="recur_wide_kernel", kernel_source_sha256_16=kernel_hash(),
                   **per_layer))
    if cpu:
        # outside the timed region, from the state as it now stands
        S0 = S.clone()
        del S
        res["cpu_baseline"], res["extra"]["parity_all_units"] = decode_cpu_and_parity(
            S0, pool, dims, steps=3,
            gated=([x["z"] for x in pool], norm_w, 1e-6) if gated else None)
    return res, dict(workload=cfg["name"], units=N, seqs=cfg["seqs"], layers=cfg["layers"],
                     vh=dims[0], kh=dims[1], kd=dims[2], vd=dims[3],
                     state_GB=round(N * vh * dims[2] * dims[3] * 4 / 1e9, 3),
                     launch="one gdn_step launch over all units per step",
                     inputs="pool of 4 seeded input sets, cycled")


def bench_latency(cfg, steps, warmup, cpu):
    """Single sequence, one layer: T sequential steps, launch-latency bound."""
    dims = cfg["dims"]
    vh = dims[0]
    T = cfg["steps"]
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, 1, dims, device="cuda")
    inp = synth.step_inputs(gen, 1, dims, M=T, device="cuda")
    rows = [{n: inp[n][m] for n in NAMES} for m in range(T)]
    o = torch.empty((1, vh, dims[3]), device="cuda")

    def one(i):
        for x in rows:
            gdn.step(S, x["q"], x["k"], x["v"], x["g"], x["beta"], o=o)

    dt = timed(one, steps, warmup)
    launch_s = dt / (steps * T)
    # the same T-step chain captured once as a HIP graph and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one(0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one(0)
    dt_g = timed(lambda i: graph.replay(), steps, warmup)
    # the kernel's roofline from the graph replay: device-paced launches
    achieved = head_step_bytes(dims) * vh / (dt_g / (steps * T)) / 1e9
    # the same T steps as one gdn_step_m(M=T) call
    o_m = torch.empty((T, 1, vh, dims[3]), device="cuda")
    dt_m = timed(lambda i: gdn.step_m(S, *(inp[n] for n in NAMES), o=o_m), steps, warmup)
    res = dict(value=vh * T * steps / dt, ms_per_step=dt / steps * 1e3,
               roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                             unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                             traffic=recorded_traffic("b1x1", None, kernel="recur_split_kernel")),
               extra=dict(kernel="recur_split_kernel (one gdn_step per launch, graph replay)",
                          algorithmic_bytes_per_launch=int(head_step_bytes(dims) * vh),
                          us_per_call=round(launch_s * 1e6, 3),
                          us_per_step_graph_replay=round(dt_g / (steps * T) * 1e6, 3),
                          us_per_step_step_m=round(dt_m / (steps * T) * 1e6, 3),
                          note="3 MiB state stays in L2/MALL: latency figure, not an HBM claim"))
    if cpu:
        pool1 = [{n: inp[n][m:m + 1] for n in NAMES} for m in range(T)]
        res["cpu_baseline"], res["extra"]["parity_all_units"] = decode_cpu_and_parity(
            S.clone(), pool1, dims, steps=T)
    return res, dict(workload=cfg["name"], units=1, vh=vh, kd=dims[2], steps_per_iteration=T)


def bench_verify(cfg, steps, warmup, cpu, only=None):
    """The speculative cycle.  only = "step_m", "verify_m", "commit" or
    "commit_verify" times that one call alone (the same inputs; every commit
    runs the first set of accepted counts from the current state), so that a
    profiler sees that call's launches only."""
    dims = cfg["dims"]
    vh = dims[0]
    L = cfg["layers"]
    N = cfg["seqs"] * L
    M = cfg["M"]
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    o = torch.empty((M, N, vh, dims[3]), device="cuda")
    slab = gdn.Slab(N, dims)
    rng = np.random.default_rng(cfg["seed"])
    accs = [np.repeat(rng.integers(0, M + 1, cfg["seqs"]), L).astype(np.int32) for _ in range(8)]
    args = [inp[n] for n in NAMES]

    def one(i):
        slab.mark_step_m(S, *args, o=o)          # mark fused into the M-step pass
        slab.rollback(S, accs[i % 8], *args)

    def one_unfused(i):
        slab.mark(S)
        gdn.step_m(S, *args, o=o)
        slab.rollback(S, accs[i % 8], *args)

    acc_dev = [torch.from_numpy(a).to("cuda") for a in accs]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def one_verify_commit(i):                   # no snapshot: verify, then commit in place
        gdn.verify_m(S, *args, o=o)
        gdn.commit(S, acc_dev[i % 8], *args, status=status)

    def one_fused(i):   # steady state: the previous rows' commit and these rows' verify, one pass
        gdn.commit_verify_m(S, acc_dev[i % 8], *args, *args, o=o, status=status)

    if only is not None:
        call = {"step_m": lambda i: gdn.step_m(S, *args, o=o),
                "verify_m": lambda i: gdn.verify_m(S, *args, o=o),
                "commit": lambda i: gdn.commit(S, acc_dev[0], *args, status=status),
                "commit_verify": lambda i: gdn.commit_verify_m(S, acc_dev[0], *args, *args, o=o,
                                                               status=status)}[only]
        dt = timed(call, steps, warmup)
        mean_a = (float(accs[0].mean()) if only in ("commit", "commit_verify")
                  else float(np.mean([a.mean() for a in accs])))
        tile = dims[2] * dims[3] * 4
        rows = N * vh * (M if only != "commit" else mean_a)
        b = N * vh * M * head_step_bytes(dims, rows=M)
        if only == "verify_m":            # no state write
            b -= N * vh * tile
        elif only == "commit":
            # a unit with accepted rows reads and writes its state and reads
            # those rows (no output); a unit with none is not touched
            row = head_step_bytes(dims, rows=1, write_o=False) - 2 * tile
            b = vh * float(((accs[0] > 0) * 2 * tile + accs[0] * row).sum())
        elif only == "commit_verify":
            # every unit reads its state once and writes it back when it
            # accepted rows; it reads those rows, then reads the M draft rows
            # and writes their outputs
            row = head_step_bytes(dims, rows=1, write_o=False) - 2 * tile
            b = vh * float((tile + (accs[0] > 0) * tile + accs[0] * row).sum())
            b += N * vh * M * (head_step_bytes(dims, rows=1) - 2 * tile)
            rows = N * vh * M
        achieved = b / (dt / steps) / 1e9
        res = dict(value=rows * steps / dt, ms_per_step=dt / steps * 1e3,
                   roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                                 unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                                 traffic=None),
                   extra=dict(only=only, algorithmic_bytes_per_launch=int(b),
                              kernel="recur_deep_kernel", mean_accepted=mean_a))
        return res, dict(workload=cfg["name"], units=N, M=M, vh=vh, kd=dims[2], only=only)

    S_start = S.clone() if cpu else None
    dt = timed(one, steps, warmup)
    dt_unfused = timed(one_unfused, steps, 1)
    dt_vc = timed(one_verify_commit, steps, 1)
    dt_fused = timed(one_fused, steps, 1)
    # step_m alone, for the kernel roofline
    dt_m = timed(lambda i: gdn.step_m(S, *args, o=o), steps, 1)
    bytes_m = N * vh * M * head_step_bytes(dims, rows=M)
    achieved = bytes_m / (dt_m / steps) / 1e9
    mean_a = float(np.mean([a.mean() for a in accs]))
    res = dict(value=N * vh * M * steps / dt, ms_per_step=dt / steps * 1e3,
               roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                             unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                             traffic=recorded_traffic("b32x48_m8_step_m", None,
                                                      kernel="recur_deep_kernel")),
               extra=dict(kernel="recur_deep_kernel (gdn_step_m alone)",
                          algorithmic_bytes_per_launch=int(bytes_m),
                          step_m_ms=round(dt_m / steps * 1e3, 4), mean_accepted=mean_a,
                          cycle_ms_separate_mark=round(dt_unfused / steps * 1e3, 4),
                          cycle_ms_verify_commit=round(dt_vc / steps * 1e3, 4),
                          cycle_ms_commit_verify_fused=round(dt_fused / steps * 1e3, 4),
                          value_counts="drafted head-steps per second of the full cycle"))
    if cpu:
        res["extra"]["parity_all_units"] = verify_parity(S_start, inp, dims, accs[0])
    return res, dict(workload=cfg["name"], units=N, M=M, vh=vh, kd=dims[2],
                     cycle="gdn_mark_step_m(M=8) + gdn_rollback(accepted ~ U{0..8})")


def verify_parity(S0, inp, dims, acc):
    """One speculative cycle from S0 in both protocols on the GPU (the fused
    mark + M steps + rollback, and verify + commit), bit-compared with each
    other on the device, and every unit against the oracle's mark, M steps,
    rollback."""
    import oracle
    orc = oracle.load()
    vh, kh, kd, vd = dims
    M, N = inp["q"].shape[:2]
    args = [inp[n] for n in NAMES]
    S = S0.clone()
    slab = gdn.Slab(N, dims)
    o = slab.mark_step_m(S, *args)
    S_m = S.clone()
    slab.rollback(S, acc, *args)
    del slab
    S_b = S0.clone()
    o_b = gdn.verify_m(S_b, *args)
    gdn.commit(S_b, torch.as_tensor(acc, device=S0.device), *args)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.int32), b.view(torch.int32))  # noqa: E731
    protocols_bit_equal = same(o, o_b) and same(S, S_b)
    del S_b, o_b

    def check(lo, hi):
        S_h = host(S0[lo:hi])
        x_h = {n: host(inp[n][:, lo:hi]) for n in NAMES}
        rs = orc.slab(hi - lo, dims)
        rs.mark(S_h)
        o_ref = np.zeros((M, hi - lo, vh, vd), np.float32)
        orc.gdn_step_m(S_h, *(x_h[n] for n in NAMES), o_ref, M, dims)
        to, tm = Tol().add(host(o[:, lo:hi]), o_ref), Tol().add(host(S_m[lo:hi]), S_h)
        rs.rollback(S_h, None, x_h, M, acc[lo:hi])
        return to, tm, Tol().add(host(S[lo:hi]), S_h)

    res = over_ranges(check, N, 16, cpu_threads())
    return dict(units=N, M=M, protocols_bit_equal=bool(protocols_bit_equal),
                o=merged(res, 0).rec(), S_after_step_m=merged(res, 1).rec(),
                S_after_rollback=merged(res, 2).rec())


def bench_frontend(cfg, steps, warmup, cpu):
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    B, T = cfg["seqs"], cfg["steps"]
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=T, device="cuda")
    hist = fe["hist"]
    out = dict(q=torch.empty((B, kh, kd), device="cuda"), k=torch.empty((B, kh, kd), device="cuda"),
               v=torch.empty((B, vh, vd), device="cuda"), g=torch.empty((B, vh), device="cuda"),
               beta=torch.empty((B, vh), device="cuda"))
    o = torch.empty((B, vh, vd), device="cuda")

    def one(i):
        t = i % T
        gdn.frontend(fe["x"][t], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"][t],
                     hist, w["conv_w"], dims, out=out)
        gdn.step(S, out["q"], out["k"], out["v"], out["g"], out["beta"], o=o)

    S_start, hist_start = (S.clone(), hist.clone()) if cpu else (None, None)
    dt = timed(one, steps, warmup)
    cd = synth.conv_dim_of(dims)
    fe_bytes = frontend_bytes(B, dims)
    step_bytes = B * vh * head_step_bytes(dims)
    chain = (step_bytes + fe_bytes) / (dt / steps) / 1e9
    # each kernel alone, device-paced: the step (the dominant kernel) and the front end
    t_step = graph_launch_s(lambda: gdn.step(S, out["q"], out["k"], out["v"], out["g"],
                                             out["beta"], o=o), steps)
    t_fe = graph_launch_s(lambda: gdn.frontend(fe["x"][0], w["Wa"], w["Wb"], w["A_log"],
                                               w["dt_bias"], fe["xc_raw"][0], hist, w["conv_w"],
                                               dims, out=out), steps)
    achieved = step_bytes / t_step / 1e9
    res = dict(value=B * vh * steps / dt, ms_per_step=dt / steps * 1e3,
               roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                             unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                             traffic=recorded_traffic("b128x1", None)),
               extra=dict(kernel="recur_wide_kernel (gdn_step alone, graph replay)",
                          algorithmic_bytes_per_launch=int(step_bytes),
                          step_us=round(t_step * 1e6, 2),
                          frontend_us=round(t_fe * 1e6, 2),
                          frontend_bytes_per_launch=fe_bytes,
                          frontend_GBps=round(fe_bytes / t_fe / 1e9, 1),
                          chain_GBps=round(chain, 1),
                          note="384 MiB state is 1.5x the MALL: partly cache-resident"))
    if cpu:
        res["extra"]["parity_all_units"] = frontend_parity(S_start, hist_start, w, fe, dims, T)
    return res, dict(workload=cfg["name"], units=B, vh=vh, kd=kd, dim=5120, conv_dim=cd)


def frontend_parity(S0, hist0, w, fe, dims, T):
    """T steps of front end + step from the given state and history on the
    GPU, then every row's front-end outputs and o at every step, the final S
    and the history against the oracle's chain (front end, then step on the
    oracle's own outputs)."""
    import oracle
    orc = oracle.load()
    vh, kh, kd, vd = dims
    B = S0.shape[0]
    S, hist = S0.clone(), hist0.clone()
    F = {n: torch.empty((T,) + shp, device=S0.device) for n, shp in
         (("q", (B, kh, kd)), ("k", (B, kh, kd)), ("v", (B, vh, vd)), ("g", (B, vh)),
          ("beta", (B, vh)))}
    O = torch.empty((T, B, vh, vd), device=S0.device)
    for t in range(T):
        out = {n: F[n][t] for n in NAMES}
        gdn.frontend(fe["x"][t], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"][t],
                     hist, w["conv_w"], dims, out=out)
        gdn.step(S, *(out[n] for n in NAMES), o=O[t])
    torch.cuda.synchronize()
    wh = {n: host(t) for n, t in w.items()}

    def check(lo, hi):
        n = hi - lo
        tf, to = Tol(), Tol()
        S_h, h_h = host(S0[lo:hi]), host(hist0[lo:hi])
        for t in range(T):
            ref = dict(q=np.zeros((n, kh, kd), np.float32), k=np.zeros((n, kh, kd), np.float32),
                       v=np.zeros((n, vh, vd), np.float32), g=np.zeros((n, vh), np.float32),
                       beta=np.zeros((n, vh), np.float32))
            orc.gdn_frontend(host(fe["x"][t, lo:hi]), wh["Wa"], wh["Wb"], wh["A_log"],
                             wh["dt_bias"], host(fe["xc_raw"][t, lo:hi]), h_h, wh["conv_w"],
                             ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"], dims)
            for k in NAMES:
                tf.add(host(F[k][t, lo:hi]), ref[k])
            o_ref = np.zeros((n, vh, vd), np.float32)
            orc.gdn_step(S_h, *(ref[k] for k in NAMES), o_ref, dims)
            to.add(host(O[t, lo:hi]), o_ref)
        return tf, to, Tol().add(host(S[lo:hi]), S_h), host(hist[lo:hi]).tobytes() == h_h.tobytes()

    res = over_ranges(check, B, 8, cpu_threads())
    return dict(rows=B, steps=T, frontend=merged(res, 0).rec(), o=merged(res, 1).rec(),
                S=merged(res, 2).rec(), history_bit_exact=all(r[3] for r in res))


def bench_verify_frontend(cfg, steps, warmup, cpu):
    """One layer's speculative verify with its front end: mark(S, hist),
    front end for M draft rows, M-step recurrence, rollback(S, hist)."""
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    B, M = cfg["seqs"], cfg["M"]
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=M, device="cuda")
    hist = fe["hist"]
    slab = gdn.Slab(B, dims, hist_floats_per_unit=3 * cd)
    rows = dict(q=torch.empty((M, B, kh, kd), device="cuda"),
                k=torch.empty((M, B, kh, kd), device="cuda"),
                v=torch.empty((M, B, vh, vd), device="cuda"),
                g=torch.empty((M, B, vh), device="cuda"),
                beta=torch.empty((M, B, vh), device="cuda"))
    o = torch.empty((M, B, vh, vd), device="cuda")
    rng = np.random.default_rng(cfg["seed"])
    accs = [rng.integers(0, M + 1, B).astype(np.int32) for _ in range(8)]
    args = [rows[n] for n in NAMES]

    def one(i):
        slab.mark(S, hist)
        gdn.frontend_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"], hist,
                       w["conv_w"], dims, out=rows)
        gdn.step_m(S, *args, o=o)
        slab.rollback(S, accs[i % 8], *args, hist=hist, xc_raw=fe["xc_raw"])

    acc_dev = [torch.from_numpy(a).to("cuda") for a in accs]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def one_verify_commit(i):
        gdn.frontend_verify_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"],
                              hist, w["conv_w"], dims, out=rows)
        gdn.verify_m(S, *args, o=o)
        gdn.commit(S, acc_dev[i % 8], *args, hist=hist, xc_raw=fe["xc_raw"], status=status)

    dt = timed(one, steps, warmup)
    dt_vc = timed(one_verify_commit, steps, 1)
    # the M-step recurrence and the M-row front end alone, for the rooflines
    t_m = graph_launch_s(lambda: gdn.step_m(S, *args, o=o), steps)
    bytes_m = B * vh * M * head_step_bytes(dims, rows=M)
    achieved = bytes_m / t_m / 1e9
    t_fe = graph_launch_s(lambda: gdn.frontend_m(fe["x"], w["Wa"], w["Wb"], w["A_log"],
                                                 w["dt_bias"], fe["xc_raw"], hist, w["conv_w"],
                                                 dims, out=rows), steps)
    fe_b = frontend_bytes(B, dims, M=M)
    res = dict(value=B * vh * M * steps / dt, ms_per_step=dt / steps * 1e3,
               roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS,
                             unit="GB/s", frac=round(achieved / PEAK_HBM_GBPS, 4),
                             traffic=recorded_traffic("b128x1_m8_step_m", None,
                                                      kernel="recur_deep_kernel")),
               extra=dict(value_counts="drafted head-steps per second of the full cycle",
                          kernel="recur_deep_kernel (gdn_step_m alone, graph replay)",
                          step_m_us=round(t_m * 1e6, 2),
                          algorithmic_bytes_per_launch=int(bytes_m),
                          frontend_m_us=round(t_fe * 1e6, 2),
                          frontend_bytes_per_launch=int(fe_b),
                          frontend_GBps=round(fe_b / t_fe / 1e9, 1),
                          cycle_ms_verify_commit=round(dt_vc / steps * 1e3, 4),
                          note="403 MB state: 1.6x the MALL, partly cache-resident"))
    return res, dict(workload=cfg["name"], units=B, M=M, vh=vh, kd=kd, conv_dim=cd,
                     cycle="gdn_mark(S, hist) + gdn_frontend_m + gdn_step_m + "
                           "gdn_rollback(S, hist)")


PEAK_MFMA_F32_TFLOPS = 157.3


def bench_layer(cfg, steps, warmup, cpu):
    """Whole GDN layers: in_proj_qkv + in_proj_z (one launch), front end,
    recurrence with the gated RMSNorm, out_proj; the output of layer l is the
    input x of layer l + 1.  Weights are f32 (gdn_proj) or, with cfg["q4"],
    4-bit values with binary16 block scales (gdn_proj_q4), packed once before
    timing.  The chain is timed both as launched from the host and as one HIP
    graph replay (no host gaps); the projections alone are timed as graph
    replays of their L launches."""
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    B, L, dim = cfg["seqs"], cfg["layers"], synth.FE_DIM
    q4 = bool(cfg.get("q4"))
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(cfg["seed"], "cuda")
    layers = []
    for _ in range(L):
        if q4:
            pw = synth.proj_weights_q4(gen, dims, dim=dim, device="cuda")
        else:
            pw = synth.proj_weights(gen, dims, dim=dim, device="cuda")
        lw = synth.frontend_weights(gen, dims, dim=dim, device="cuda")
        for n in ("W_qkv", "W_z", "W_out"):
            packed = gdn.proj_q4_pack(*pw[n]) if q4 else gdn.proj_pack(pw[n])
            del pw[n]
            lw[n] = packed
        lw["norm_w"] = pw["norm_w"]
        lw["S"] = synth.state(gen, B, dims, device="cuda")
        lw["hist"] = torch.randn((B, 3, cd), generator=gen, device="cuda")
        layers.append(lw)
    torch.cuda.empty_cache()
    proj = gdn.proj_q4 if q4 else gdn.proj
    x0 = torch.randn((B, dim), generator=gen, device="cuda")
    xs = [torch.empty((B, dim), device="cuda") for _ in range(L)]
    xc = torch.empty((B, cd), device="cuda")
    z = torch.empty((B, vh * vd), device="cuda")
    out = torch.empty((1, B, vh, vd), device="cuda")
    fe = dict(q=torch.empty((B, kh, kd), device="cuda"), k=torch.empty((B, kh, kd), device="cuda"),
              v=torch.empty((B, vh, vd), device="cuda"), g=torch.empty((B, vh), device="cuda"),
              beta=torch.empty((B, vh), device="cuda"))

    def one(i):
        x = x0
        for l, w in enumerate(layers):
            proj(x, w["W_qkv"], w["W_z"], y0=xc, y1=z)
            gdn.frontend(x, w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], xc, w["hist"],
                         w["conv_w"], dims, out=fe)
            gdn.step_gated(w["S"], *(fe[n].unsqueeze(0) for n in NAMES), z.view(1, B, vh, vd),
                           w["norm_w"], 1e-6, out=out)
            proj(out.view(B, vh * vd), w["W_out"], y0=xs[l])
            x = xs[l]

    dt = timed(one, steps, warmup)
    # the same chain captured once as a HIP graph and replayed; it contains
    # no memset node
    dt_g = timed_graph(one, steps, 2)
    # the projections alone, layer after layer, for the kernel roofline
    dt_in = timed_graph(lambda i: [proj(x0, w["W_qkv"], w["W_z"], y0=xc, y1=z) for w in layers],
                        steps, 1)
    h = out.view(B, vh * vd)
    dt_out = timed_graph(lambda i: [proj(h, w["W_out"], y0=xs[0]) for w in layers], steps, 1)
    # read+write floor over one packed weight matrix (also calibrates counters)
    flat = layers[0]["W_qkv"].view(-1)
    floor = copy_floor(layers[0]["W_qkv"].view(torch.float32) if q4 else layers[0]["W_qkv"])
    wbytes = (lambda R, C_: R * C_ * 9 // 16) if q4 else (lambda R, C_: R * C_ * 4)
    w_in = wbytes(cd + vh * vd, dim)
    w_out = wbytes(dim, vh * vd)
    in_bytes = w_in + B * dim * 4 + B * (cd + vh * vd) * 4
    out_bytes = w_out + B * vh * vd * 4 + B * dim * 4
    in_flop = 2 * B * (cd + vh * vd) * dim
    out_flop = 2 * B * dim * vh * vd
    t_in, t_out = dt_in / (steps * L), dt_out / (steps * L)
    kname = "proj_q4_kernel" if q4 else "proj_kernel"
    key = f"layer_q4_b{B}" if q4 else f"layer_b{B}"
    ridge = PEAK_MFMA_F32_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)     # ~19.7 flop/B
    if not q4 and in_flop / in_bytes >= ridge:   # 2B flop per 4-byte weight: from B ~ 40
        roof = dict(bound="mfma", achieved=round(in_flop / t_in / 1e12, 2),
                    peak=PEAK_MFMA_F32_TFLOPS, unit="TFLOP/s",
                    frac=round(in_flop / t_in / 1e12 / PEAK_MFMA_F32_TFLOPS, 4),
                    traffic=recorded_traffic(key, in_bytes, kernel=kname))
    else:
        roof = dict(bound="hbm", achieved=round(in_bytes / t_in / 1e9, 1), peak=PEAK_HBM_GBPS,
                    unit="GB/s", frac=round(in_bytes / t_in / 1e9 / PEAK_HBM_GBPS, 4),
                    traffic=recorded_traffic(key, in_bytes, kernel=kname))
    desc = ("gdn_proj_q4" if q4 else "gdn_proj")
    res = dict(value=B * vh * L * steps / dt_g, ms_per_step=dt_g / steps * 1e3, roofline=roof,
               extra=dict(kernel=f"{kname} (in_proj_qkv + in_proj_z, one launch)",
                          timing="value and ms_per_step: the chain as one HIP graph replay",
                          in_proj_us=round(t_in * 1e6, 2), out_proj_us=round(t_out * 1e6, 2),
                          in_proj_GBps=round(in_bytes / t_in / 1e9, 1),
                          out_proj_GBps=round(out_bytes / t_out / 1e9, 1),
                          in_proj_TFLOPs=round(in_flop / t_in / 1e12, 2),
                          out_proj_TFLOPs=round(out_flop / t_out / 1e12, 2),
                          layer_us_host_launched=round(dt / (steps * L) * 1e6, 2),
                          layer_us_graph_replay=round(dt_g / (steps * L) * 1e6, 2),
                          in_proj_bytes_per_launch=in_bytes, in_proj_flop_per_launch=in_flop,
                          weights_GB=round(L * (w_in + w_out) / 1e9, 3),
                          copy_floor_GBps=round(floor, 1), copy_bytes=flat.numel() * flat.element_size(),
                          kernel_source_sha256_16=kernel_hash(kname)))
    return res, dict(workload=cfg["name"], units=B * L, seqs=B, layers=L, vh=vh, kd=kd,
                     dim=dim, conv_dim=cd, weights="4-bit + binary16 scale per 32" if q4 else "f32",
                     chain=f"{desc}(W_qkv, W_z) + gdn_frontend + gdn_step_gated + "
                           f"{desc}(W_out) per layer")


def bench_layer_verify(cfg, steps, warmup, cpu):
    """Whole GDN layers verifying M draft rows without a snapshot: the input
    projections over all M*B rows, the M-row front end without advancing the
    history, the gated outputs without advancing the state, out_proj over all
    rows, then commit of per-sequence accepted lengths (device array).  The
    output of layer l (its M rows) is the input of layer l + 1.  Weights are
    f32 or, with cfg["q4"], 4-bit with binary16 block scales.  The cycle is
    timed as one HIP graph replay (value; every replay commits the same
    accepted lengths) and as launched from the host (accepted lengths cycled
    over 8 draws)."""
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    B, L, M, dim = cfg["seqs"], cfg["layers"], cfg["M"], synth.FE_DIM
    q4 = bool(cfg.get("q4"))
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(cfg["seed"], "cuda")
    layers = []
    for _ in range(L):
        if q4:
            pw = synth.proj_weights_q4(gen, dims, dim=dim, device="cuda")
        else:
            pw = synth.proj_weights(gen, dims, dim=dim, device="cuda")
        lw = synth.frontend_weights(gen, dims, dim=dim, device="cuda")
        for n in ("W_qkv", "W_z", "W_out"):
            packed = gdn.proj_q4_pack(*pw[n]) if q4 else gdn.proj_pack(pw[n])
            del pw[n]
            lw[n] = packed
        lw["norm_w"] = pw["norm_w"]
        lw["S"] = synth.state(gen, B, dims, device="cuda")
        lw["hist"] = torch.randn((B, 3, cd), generator=gen, device="cuda")
        layers.append(lw)
    torch.cuda.empty_cache()
    rows = M * B
    x0 = torch.randn((M, B, dim), generator=gen, device="cuda")
    xs = [torch.empty((M, B, dim), device="cuda") for _ in range(L)]
    xc = torch.empty((rows, cd), device="cuda")
    z = torch.empty((rows, vh * vd), device="cuda")
    out = torch.empty((M, B, vh, vd), device="cuda")
    fe = dict(q=torch.empty((M, B, kh, kd), device="cuda"),
              k=torch.empty((M, B, kh, kd), device="cuda"),
              v=torch.empty((M, B, vh, vd), device="cuda"), g=torch.empty((M, B, vh), device="cuda"),
              beta=torch.empty((M, B, vh), device="cuda"))
    rng = np.random.default_rng(cfg["seed"])
    accs = [torch.from_numpy(rng.integers(0, M + 1, B).astype(np.int32)).to("cuda")
            for _ in range(8)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows_in = [fe[n] for n in NAMES]

    proj = gdn.proj_q4 if q4 else gdn.proj

    def one(i):
        x = x0
        for l, w in enumerate(layers):
            proj(x.view(rows, dim), w["W_qkv"], w["W_z"], y0=xc, y1=z)
            gdn.frontend_verify_m(x, w["Wa"], w["Wb"], w["A_log"], w["dt_bias"],
                                  xc.view(M, B, cd), w["hist"], w["conv_w"], dims, out=fe)
            gdn.verify_m_gated(w["S"], *rows_in, z.view(M, B, vh, vd), w["norm_w"], 1e-6,
                               out=out)
            proj(out.view(rows, vh * vd), w["W_out"], y0=xs[l].view(rows, dim))
            gdn.commit(w["S"], accs[i % 8], *rows_in, hist=w["hist"],
                       xc_raw=xc.view(M, B, cd), status=status)
            x = xs[l]

    dt = timed(one, steps, warmup)
    dt_g = timed_graph(one, steps, 2)
    dt_in = timed_graph(lambda i: [proj(x0.view(rows, dim), w["W_qkv"], w["W_z"], y0=xc, y1=z)
                                   for w in layers], steps, 1)
    wb = 9 / 16 if q4 else 4
    in_bytes = int((cd + vh * vd) * dim * wb) + rows * dim * 4 + rows * (cd + vh * vd) * 4
    t_in = dt_in / (steps * L)
    kname = "proj_q4_kernel" if q4 else "proj_kernel"
    key = f"layer_q4_verify_b{B}m{M}" if q4 else f"layer_verify_b{B}m{M}"
    roof = dict(bound="hbm", achieved=round(in_bytes / t_in / 1e9, 1), peak=PEAK_HBM_GBPS,
                unit="GB/s", frac=round(in_bytes / t_in / 1e9 / PEAK_HBM_GBPS, 4),
                traffic=recorded_traffic(key, in_bytes, kernel=kname))
    desc = "gdn_proj_q4" if q4 else "gdn_proj"
    res = dict(value=B * vh * M * L * steps / dt_g, ms_per_step=dt_g / steps * 1e3, roofline=roof,
               extra=dict(value_counts="drafted head-steps per second of the full cycle",
                          timing="value and ms_per_step: the cycle as one HIP graph replay",
                          layer_us_graph_replay=round(dt_g / (steps * L) * 1e6, 2),
                          layer_us_host_launched=round(dt / (steps * L) * 1e6, 2),
                          in_proj_us=round(t_in * 1e6, 2),
                          kernel=f"{kname} (in_proj_qkv + in_proj_z over M*B rows)",
                          in_proj_bytes_per_launch=in_bytes,
                          kernel_source_sha256_16=kernel_hash(kname),
                          mean_accepted=float(np.mean([a.float().mean().item() for a in accs]))))
    return res, dict(workload=cfg["name"], units=B * L, seqs=B, layers=L, M=M, vh=vh, kd=kd,
                     dim=dim, conv_dim=cd, weights="4-bit + binary16 scale per 32" if q4 else "f32",
                     chain=f"{desc}(W_qkv, W_z) + gdn_frontend_verify_m + gdn_verify_m_gated + "
                           f"{desc}(W_out) + gdn_commit per layer")


RUNNERS = {0: "bench_latency", 2: "bench_verify", 3: "bench_frontend",
           6: "bench_verify_frontend", 8: "bench_layer", 9: "bench_layer",
           10: "bench_layer_verify", 11: "bench_layer", 12: "bench_layer_verify"}


def runner_of(config):
    return globals()[RUNNERS.get(config, "bench_decode")]


def other_workloads(steps, warmup, skip):
    """Every other workload, timed the same way with fewer steps (no CPU
    baseline, no parity pass), so that one default run measures all of them:
    the result line of each, without its config and cpu fields."""
    out = {}
    for c in sorted(synth.WORKLOADS):
        if c == skip:
            continue
        cfg = dict(synth.WORKLOADS[c])
        cfg["id"] = c
        torch.cuda.synchronize()
        t0 = time.time()
        try:
            res, config = runner_of(c)(cfg, steps, warmup, False)
            torch.cuda.synchronize()
        except Exception as e:  # noqa: BLE001 - recorded; the headline line must still print
            out[str(c)] = dict(workload=cfg["name"], error=f"{type(e).__name__}: {e}")
            print(f"bench.py: workload {c} failed: {out[str(c)]['error']}", file=sys.stderr,
                  flush=True)
            torch.cuda.empty_cache()
            continue
        out[str(c)] = dict(workload=config["workload"], value=round(res["value"], 1),
                           ms_per_step=round(res["ms_per_step"], 5), roofline=res["roofline"],
                           extra={k: v for k, v in res.get("extra", {}).items()
                                  if not isinstance(v, dict)},
                           wall_s=round(time.time() - t0, 2))
        torch.cuda.empty_cache()
        print(f"bench.py: workload {c} done ({out[str(c)]['wall_s']} s)", file=sys.stderr,
              flush=True)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("step_m", "verify_m", "commit", "commit_verify"),
                    help="config 2: time this one call alone (for a profiler)")
    ap.add_argument("--other-steps", type=int, default=20,
                    help="the default workload also times every other workload with this "
                         "many steps (0: skip them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU; --gpus {args.gpus} is not "
              "supported (every state unit is independent, so G GPUs would each run this "
              "same kernel on N/G units with no communication).", file=sys.stderr)
        sys.exit(2)
    if args.only is not None and args.config != 2:
        print("bench.py: --only applies to --config 2", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no HIP device visible", file=sys.stderr)
        sys.exit(1)
    gdn.lib()
    cfg = dict(synth.WORKLOADS[args.config])
    cfg["id"] = args.config
    runner = runner_of(args.config)
    if args.only is not None:
        res, config = bench_verify(cfg, args.steps, args.warmup, False, only=args.only)
    else:
        res, config = runner(cfg, args.steps, args.warmup, not args.no_cpu_baseline)
    line = dict(metric=METRIC, value=round(res["value"], 1), unit="head-steps/s", n_gpus=1,
                steps=args.steps, warmup=args.warmup, ms_per_step=round(res["ms_per_step"], 5),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                data="synthetic", config=config, roofline=res["roofline"])
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    line["extra"] = res.get("extra", {})
    if args.config == 1 and args.only is None and args.other_steps > 0:
        # after the headline measurement, so that it runs on a fresh device
        torch.cuda.empty_cache()
        line["extra"]["workloads"] = other_workloads(args.other_steps, 2, skip=1)
    line["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
