#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet decode step on one MI355X.

Workload (one "step"): B=256 sequences x 36 recurrent layers, one token per
layer: 36 gdn_step calls in layer order on one stream, each on its own
[256][32][128][128] float32 state (512 MiB; 18 GiB in all), with fresh seeded
inputs per layer.  Inputs and states are resident in HBM before timing starts.

Printed: ONE JSON line with the headline metric (state-updates/s, one update =
one 128x128 head state advanced by one token), the roofline of the gdn_step
kernel (algorithmic bytes per launch / mean launch time, i.e. the timed
region's duration from HIP events on the launch stream divided by its 36 x K
launches), the plain C oracle timed on the host on a bounded sample, and
secondary measurements of the other entry points.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import gdn_inputs as gi  # noqa: E402

HV, HK, D = gi.HV, gi.HK, gi.D
# Algorithmic bytes of one state-update of gdn_step: the 64 KiB state read and
# written, v and out (512 B each), half of the shared q and k of the key head
# (512 B), beta and gate (8 B).
STATE_UPDATE_BYTES = 2 * D * D * 4 + 2 * D * 4 + (2 * D * 4) // 2 + 8   # 132616
HBM_PEAK_GBPS = 8000.0
# HBM traffic of one gdn_step launch from hardware counters (FETCH_SIZE and
# WRITE_SIZE, calibrated against a copy of known size); only reported while
# the kernel source is the one the counters were taken on.
TRAFFIC_FILE = os.path.join(HERE, "profiles", "k_step_b256_traffic.json")
KERNEL_SOURCES = [os.path.join(HERE, "gated_deltanet_decode_amd", "csrc", f)
                  for f in ("gdn_device.hpp", "gdn_step.hip")]
METRIC = "GDN state-updates/s (seq·head·token) and achieved HBM GB/s, B=256 decode"
# Algorithmic bytes of gdn_layer_tail at B = 32: per sequence the 2 MiB
# state read and written, x (32 KiB), the 3-slot conv ring read and written
# (2 x 96 KiB), z and y (2 x 16 KiB), beta and gate; shared by all: the conv
# weight (128 KiB) and the norm weight.
TAIL_B32_BYTES = 32 * (2 * HV * D * D * 4 + 8192 * 4 + 2 * 3 * 8192 * 4 + 2 * HV * D * 4
                       + 2 * HV * 4) + 8192 * 4 * 4 + D * 4
# gdn_layer_tail_pair at B = 32: the state read once and written twice, the
# ring read once and written twice, x, z, y, beta and gate for two positions.
TAIL_PAIR_B32_BYTES = 32 * (3 * HV * D * D * 4 + 2 * 8192 * 4 + 3 * 3 * 8192 * 4
                            + 2 * 2 * HV * D * 4 + 2 * 2 * HV * 4) + 8192 * 4 * 4 + D * 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the secondary entry points")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--workload", default="step_b256_x36",
                   choices=["step_b1", "step_b64_x100", "step_b256_x36", "seq_b8_t4096",
                            "seq_b256_t64", "seq_b40_t1024", "tail_b32"],
                   help="step_b256_x36 (default): the headline run; the others run only that "
                        "workload's secondary measurement (for profiling)")
    return p.parse_args()


def setup_step_b256_x36(torch, g):
    c = gi.WORKLOADS["step_b256_x36"]
    B, L, seed = c["B"], c["layers"], c["seed"]
    log(f"[bench] generating {L} x {B} x {HV} x {D}x{D} f32 states (seeded) ...")
    states = torch.empty((L, B, HV, D, D), device="cuda")
    stage = torch.empty((B, HV, D, D), pin_memory=True)
    sn = stage.numpy()
    ins = []
    for l in range(L):
        gi.state_into(sn, seed, l)
        states[l].copy_(stage)
        si = gi.step_inputs(seed, l, B)
        ins.append({n: torch.from_numpy(x).cuda() for n, x in si.items()})
        torch.cuda.synchronize()
    outs = torch.empty((L, B, HV, D), device="cuda")
    return dict(B=B, L=L, states=states, ins=ins, outs=outs)


def measured_traffic():
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        h = hashlib.sha256()
        for path in KERNEL_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != sha:
        return None
    return t.get("traffic_bytes_per_launch")


def inplace_probe(torch, stream, buf, reps=5, staged=True):
    """Rate of an in-place read-modify-write of `buf` with no arithmetic
    (read + write bytes / s; the data is left unchanged): with the staged
    step kernel's memory pattern, or with the tile walk's (staged=False)."""
    import ctypes
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    fn = lib.gdn_probe_inplace_staged if staged else lib.gdn_probe_inplace
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint, ctypes.c_void_p]
    nbytes = buf.numel() * buf.element_size()

    def once():
        assert fn(buf.data_ptr(), nbytes, 0, stream.cuda_stream) == 0
    once()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        once()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return 2 * nbytes / (ms / 1e3) / 1e9


def one_direction_probes(torch, stream, buf, reps=5):
    """Rates (bytes / s) of reading `buf` only and of writing a buffer of the
    same size only, with the tile walk's accesses: what each direction
    reaches alone, against the walk's in-place mix of both."""
    import ctypes
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.gdn_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    lib.gdn_probe_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint,
                                    ctypes.c_void_p]
    nbytes = buf.numel() * buf.element_size()
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    calls = {
        "read": lambda: lib.gdn_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), 4 << 20,
                                           stream.cuda_stream),
        "write": lambda: lib.gdn_probe_write(dst.data_ptr(), nbytes, 0, stream.cuda_stream),
    }
    out = {}
    for name, fn in calls.items():
        assert fn() == 0
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(reps):
            assert fn() == 0
        e.record(stream)
        torch.cuda.synchronize()
        out[name] = nbytes / (s.elapsed_time(e) / reps / 1e3) / 1e9
    del dst
    return out["read"], out["write"]


def small_launch_floors(torch, side, timeit, workgroups, nbytes):
    """Per-launch device time, from a graph of 100 launches, of an empty
    kernel of `workgroups` one-wave workgroups and of the in-place probe over
    `nbytes` with one one-wave workgroup per 4 KiB tile."""
    import ctypes
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.gdn_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gdn_probe_inplace_small.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint,
                                            ctypes.c_void_p]
    buf = torch.zeros(nbytes // 4, device="cuda")
    torch.cuda.synchronize()
    calls = {
        "graph_empty_launch_us": lambda: lib.gdn_probe_empty(workgroups, 64, side.cuda_stream),
        "graph_inplace_probe_us": lambda: lib.gdn_probe_inplace_small(
            buf.data_ptr(), nbytes, 0, side.cuda_stream),
    }
    out = {}
    for name, fn in calls.items():
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            for _ in range(100):
                assert fn() == 0
        torch.cuda.synchronize()
        out[name] = timeit(gr.replay, 10) / 100 * 1e3
    return out


def fma_probe(torch, stream, workgroups, threads, iters=20000, reps=3):
    """Non-packed FP32 FMA rate (TFLOP/s) of independent fmaf chains with no
    memory traffic, at `workgroups` x `threads` threads: the VALU ceiling at
    that number of waves per CU."""
    import ctypes
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    lib.gdn_probe_fma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    n = workgroups * threads
    out = torch.empty(n, device="cuda")

    def once():
        assert lib.gdn_probe_fma(out.data_ptr(), n, workgroups, threads, iters,
                                 stream.cuda_stream) == 0
    once()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        once()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return 2.0 * n * iters * 16 / (ms / 1e3) / 1e12


def copy_probe(torch, stream, nbytes=1 << 30, reps=5, tuned=True):
    """Bandwidth of a device-to-device copy (read + write bytes / s): tuned
    (the tile walk with nontemporal 16-byte accesses, src != dst) or a plain
    grid-stride copy."""
    import ctypes
    from gated_deltanet_decode_amd._build import PROBE_LIBRARY
    lib = ctypes.CDLL(PROBE_LIBRARY)
    fn = lib.gdn_probe_copy_nt if tuned else lib.gdn_probe_copy
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)

    def once():
        assert fn(src.data_ptr(), dst.data_ptr(), nbytes, stream.cuda_stream) == 0
    once()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        once()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * nbytes / (ms / 1e3) / 1e9


def run_step36(g, w, stream, evs=None):
    for l in range(w["L"]):
        t = w["ins"][l]
        if evs is not None:
            evs[l][0].record(stream)
        g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], w["states"][l], w["outs"][l],
               stream=stream)
        if evs is not None:
            evs[l][1].record(stream)


def step_b256_x36_variants(torch, g, w, stream, steps):
    """The same 36-layer step (a) captured once as a HIP graph and replayed,
    and (b) as one gdn_step launch over all layers: the [36][256] layer and
    sequence axes of the contiguous buffers flattened into B = 9216."""
    L, B = w["L"], w["B"]
    res = {}
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=side):
        run_step36(g, w, torch.cuda.current_stream())
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(steps):
        gr.replay()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    res["graph_replay"] = {"ms_per_step": ms, "state_updates_per_s": L * B * HV / (ms / 1e3)}

    cat = {n: torch.cat([w["ins"][l][n] for l in range(L)]) for n in w["ins"][0]}
    flat = w["states"].view(L * B, HV, D, D)
    out = w["outs"].view(L * B, HV, D)

    def one():
        g.step(cat["q"], cat["k"], cat["v"], cat["beta"], cat["gate"], flat, out, stream=stream)
    one()
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(steps):
        one()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    res["flattened_b9216_one_launch"] = {
        "ms_per_step": ms, "state_updates_per_s": L * B * HV / (ms / 1e3),
        "GBps": L * B * HV * STATE_UPDATE_BYTES / (ms / 1e3) / 1e9}
    return res


def host_info():
    info = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["mem_GiB"] = round(int(line.split()[1]) / 2**20, 1)
                    break
    except OSError:
        pass
    return info


def cpu_baseline(seconds):
    """The oracle as it is, on the host cores, over layers of the B=256 x 36-layer decode
    stepped round-robin until `seconds` have passed."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    o = oracle.get()
    c = gi.WORKLOADS["step_b256_x36"]
    B, seed, n_layers = c["B"], c["seed"], 4
    threads = max(1, min(16, os.cpu_count() or 1))
    states = [gi.state(seed, l, B) for l in range(n_layers)]
    ins = [gi.step_inputs(seed, l, B) for l in range(n_layers)]
    bounds = np.linspace(0, B, threads + 1).astype(int)

    def layer(l):
        def part(i):
            a, b = bounds[i], bounds[i + 1]
            si = {n: np.ascontiguousarray(x[a:b]) for n, x in ins[l].items()}
            M = np.ascontiguousarray(states[l][a:b])
            o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
            states[l][a:b] = M
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(part, range(threads)))

    done = 0
    t0 = time.perf_counter()
    while True:
        layer(done % n_layers)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds or done >= 4000:
            break
    updates = done * B * HV

    # one host thread, a smaller slice (32 sequences of layer 0), ~3 s
    si = {n: np.ascontiguousarray(x[:32]) for n, x in ins[0].items()}
    M = np.ascontiguousarray(states[0][:32])
    done1 = 0
    t1 = time.perf_counter()
    while time.perf_counter() - t1 < max(1.0, seconds / 4):
        o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M)
        done1 += 1
    el1 = time.perf_counter() - t1
    other = oracle_other_workloads(o, threads)
    return {"value": updates / el, "unit": "state-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} layer-steps of the B=256 x 36-layer decode (32 heads; layers 0-"
                      f"{n_layers - 1} stepped round-robin), oracle_gdn_step_M split over "
                      f"{threads} host threads by sequence, {el:.1f} s",
            "GBps": updates * STATE_UPDATE_BYTES / el / 1e9,
            "single_thread_value": done1 * 32 * HV / el1,
            "single_thread_sample": f"{done1} steps of 32 sequences x 32 heads, one thread, "
                                    f"{el1:.1f} s",
            "other_workloads": other,
            "host": host_info()}


def _timed(fn, seconds):
    """Calls fn() until `seconds` have passed (at least once); returns (calls, s)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def oracle_other_workloads(o, threads, seconds=1.0):
    """The oracle on the secondary workloads (bounded samples, ~1 s each),
    split over host threads by sequence where there is more than one."""
    from concurrent.futures import ThreadPoolExecutor
    res = {}
    ex = ThreadPoolExecutor(threads)

    def split(B, fn):
        bounds = np.linspace(0, B, min(threads, B) + 1).astype(int)
        list(ex.map(lambda i: fn(bounds[i], bounds[i + 1]), range(len(bounds) - 1)))

    # step_b1: one call, one thread
    si = gi.step_inputs(1000, 0, 1)
    M = gi.state(1000, 0, 1)
    n, el = _timed(lambda: o.step_M(si["q"], si["k"], si["v"], si["beta"], si["gate"], M), seconds)
    res["step_b1"] = {"us_per_call": el / n * 1e6, "state_updates_per_s": n * HV / el, "threads": 1}

    # step_b64_x100: B = 64 calls
    si = gi.step_inputs(1001, 0, 64)
    M = gi.state(1001, 0, 64)

    def b64():
        def part(a, b):
            s_ = {k: np.ascontiguousarray(x[a:b]) for k, x in si.items()}
            m = np.ascontiguousarray(M[a:b])
            o.step_M(s_["q"], s_["k"], s_["v"], s_["beta"], s_["gate"], m)
            M[a:b] = m
        split(64, part)
    n, el = _timed(b64, seconds)
    res["step_b64_x100"] = {"ms_per_100_calls": el / n * 100 * 1e3,
                            "state_updates_per_s": n * 64 * HV / el, "threads": min(threads, 64)}

    # seq_b8_t4096: a 64-token sample of the 8 sequences, one thread per sequence
    T = 64
    ss = gi.step_inputs(1003, 0, 8, T=T)
    Ms = np.zeros((8, HV, D, D), np.float32)

    def seq():
        def part(a, b):
            s_ = {k: np.ascontiguousarray(x[a:b]) for k, x in ss.items()}
            m = np.ascontiguousarray(Ms[a:b])
            o.seq(s_["q"], s_["k"], s_["v"], s_["beta"], s_["gate"], m)
        split(8, part)
    n, el = _timed(seq, seconds)
    rate = n * 8 * T * HV / el
    res["seq_b8_t4096"] = {"state_updates_per_s": rate, "threads": min(threads, 8),
                           "ms_full_run_estimate": 8 * 4096 * HV / rate * 1e3,
                           "sample": f"T={T} of the 4096 tokens"}

    # tail_b32
    ti = gi.tail_inputs(1004, 32)
    Mt = gi.state(1004, 0, 32)

    def tail():
        def part(a, b):
            t_ = {k: (np.ascontiguousarray(x[a:b]) if k not in ("conv_w", "norm_w") else x)
                  for k, x in ti.items()}
            m = np.ascontiguousarray(Mt[a:b])
            o.layer_tail(t_["x"], t_["conv_w"], t_["conv_state"], t_["beta"], t_["gate"], m,
                         t_["z"], t_["norm_w"], HK, D)
        split(32, part)
    n, el = _timed(tail, seconds)
    res["tail_b32"] = {"us_per_call": el / n * 1e6, "state_updates_per_s": n * 32 * HV / el,
                       "threads": min(threads, 32)}
    ex.shutdown()
    return res


def extra_measurements(torch, g, stream, only=None):
    """Secondary entry points, timed with events on the launch stream
    (`only`: run just that configuration)."""
    res = {}
    want = lambda c: only is None or only == c

    def timeit(fn, reps):
        # warm up for at least 30 ms of GPU work: after the host has spent
        # time generating inputs the GPU clock ramps up over ~20 ms of load
        t_end = time.perf_counter() + 0.03
        n = 0
        while n < 2 or time.perf_counter() < t_end:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    # step_b1: B=1 single step (latency-bound)
    if want("step_b1"):
        si = {n: torch.from_numpy(x).cuda() for n, x in gi.step_inputs(1000, 0, 1).items()}
        M = torch.from_numpy(gi.state(1000, 0, 1)).cuda()
        o = torch.empty((1, HV, D), device="cuda")
        ms = timeit(lambda: g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o,
                                   stream=stream), 1000)
        res["step_b1"] = {"us_per_call": ms * 1e3, "state_updates_per_s": 32 / (ms / 1e3)}
        # the prepared call (tensors checked once, converted arguments reused)
        call = g.bind_step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o, stream=stream)
        ms = timeit(call, 1000)
        res["step_b1"]["prepared_us_per_call"] = ms * 1e3
        call = g.bind_step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o, stream=stream,
                           cached=True)
        ms = timeit(call, 1000)
        res["step_b1"]["prepared_cached_us_per_call"] = ms * 1e3
        # the same call replayed from a captured graph of 100 calls (no host
        # launch path in the loop: device-side time per call)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=side):
            for _ in range(100):
                g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o)
        torch.cuda.synchronize()
        ms = timeit(gr.replay, 10) / 100
        res["step_b1"]["graph_us_per_call"] = ms * 1e3
        gr2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr2, stream=side):
            for _ in range(100):
                g.step(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o, cached=True)
        torch.cuda.synchronize()
        ms = timeit(gr2.replay, 10) / 100
        res["step_b1"]["graph_cached_us_per_call"] = ms * 1e3
        # floors of this launch, replayed the same way: an empty kernel of the
        # step's shape at B = 1 (512 one-wave workgroups) and the in-place
        # probe over 2 MiB with that shape (the state's bytes, no arithmetic)
        res["step_b1"].update(small_launch_floors(torch, side, timeit, 512, 2 << 20))

    # step_b64_x100: B=64 decode, 100 calls with fresh inputs
    if want("step_b64_x100"):
        c1 = gi.WORKLOADS["step_b64_x100"]
        M = torch.from_numpy(gi.state(c1["seed"], 0, 64)).cuda()
        ins = [{n: torch.from_numpy(x).cuda() for n, x in gi.step_inputs(c1["seed"], i, 64).items()}
               for i in range(100)]
        o = torch.empty((64, HV, D), device="cuda")

        def c1run():
            for t in ins:
                g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], M, o, stream=stream)
        ms = timeit(c1run, 3)
        upd = 100 * 64 * HV

        def c1cached():
            for t in ins:
                g.step(t["q"], t["k"], t["v"], t["beta"], t["gate"], M, o, stream=stream,
                       cached=True)
        ms_c = min(timeit(c1cached, 3) for _ in range(3))
        ms = min(ms, min(timeit(c1run, 3) for _ in range(2)))
        res["step_b64_x100"] = {"ms": ms, "state_updates_per_s": upd / (ms / 1e3),
                                "GBps": upd * STATE_UPDATE_BYTES / (ms / 1e3) / 1e9,
                                "cached_ms": ms_c,
                                "cached_state_updates_per_s": upd / (ms_c / 1e3),
                                "cached_GBps": upd * STATE_UPDATE_BYTES / (ms_c / 1e3) / 1e9,
                                "note": "the 128 MiB state fits the 256 MB Infinity Cache; "
                                        "cached_*: gdn_step_ex with GDN_STATE_CACHED"}

    # gdn_pair: B=256, one layer, two positions (state read once, written twice)
    if only is None:
        c2 = gi.WORKLOADS["step_b256_x36"]
        si = {n: torch.from_numpy(x).cuda() for n, x in gi.step_inputs(c2["seed"], 0, 256, T=2).items()}
        M = torch.from_numpy(gi.state(c2["seed"], 0, 256)).cuda()
        Mn = torch.empty_like(M)
        o = torch.empty((256, 2, HV, D), device="cuda")
        ms = timeit(lambda: g.pair(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, Mn, o,
                                   stream=stream), 10)
        pair_bytes = 256 * HV * (3 * D * D * 4 + 2 * (STATE_UPDATE_BYTES - 2 * D * D * 4))
        res["pair_b256"] = {"us_per_call": ms * 1e3, "state_updates_per_s": 2 * 256 * HV / (ms / 1e3),
                            "GBps": pair_bytes / (ms / 1e3) / 1e9,
                            "bytes_per_call": pair_bytes}
        del M, Mn

    # seq_b8_t4096: gdn_seq B=8 x T=4096 from a zero state
    if want("seq_b8_t4096"):
        c3 = gi.WORKLOADS["seq_b8_t4096"]
        si = {n: torch.from_numpy(x).cuda() for n, x in gi.step_inputs(c3["seed"], 0, 8, T=4096).items()}
        M = torch.zeros((8, HV, D, D), device="cuda")
        o = torch.empty((8, 4096, HV, D), device="cuda")
        # gdn_seq, and gdn_seq_exact (the decay multiplied into the state on
        # every token): timed in alternation after a joint warmup, best of 3
        # rounds of 5 calls each (the clock ramps up over the first ~10 calls
        # after the GPU has idled while the host generated the inputs)
        run = lambda exact: g.seq(si["q"], si["k"], si["v"], si["beta"], si["gate"], M, o,
                                  stream=stream, exact=exact)
        for _ in range(5):
            run(False)
            run(True)
        ms, ms_exact = float("inf"), float("inf")
        for _ in range(3):
            ms = min(ms, timeit(lambda: run(False), 5))
            ms_exact = min(ms_exact, timeit(lambda: run(True), 5))
        upd = 8 * 4096 * HV
        # The method's work is 7 flop per state element and token: the
        # decay multiply and three FMA (the rank-1 update and the two dot
        # products).  gdn_seq executes 6 of them: it carries a qualifying
        # 16-token group's decay as one scale instead of multiplying every
        # element.
        tf = upd * D * D * 7 / (ms / 1e3) / 1e12
        tf6 = upd * D * D * 6 / (ms / 1e3) / 1e12
        # the VALU ceiling measured at the kernel's own occupancy (one 8-wave
        # workgroup per CU, as this launch) and at 16 waves per CU
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        probe8 = fma_probe(torch, stream, cus, 512)
        probe16 = fma_probe(torch, stream, 4 * cus, 256)
        res["seq_b8_t4096"] = {"ms": ms, "state_updates_per_s": upd / (ms / 1e3),
                               "TFLOPs": tf, "flop_per_element": 7,
                               "frac_fp32_vector_nonpacked_78.6": tf / 78.6,
                               "frac_fp32_vector_157.3": tf / 157.3,
                               "executed_TFLOPs_6_flop_per_element": tf6,
                               "executed_frac_fp32_vector_nonpacked_78.6": tf6 / 78.6,
                               "fma_probe_TFLOPs_8_waves_per_cu": probe8,
                               "fma_probe_TFLOPs_16_waves_per_cu": probe16,
                               "executed_frac_of_fma_probe_same_occupancy": tf6 / probe8,
                               "exact_ms": ms_exact,
                               "exact_TFLOPs": upd * D * D * 7 / (ms_exact / 1e3) / 1e12}

    # seq_b256_t64: gdn_seq with many heads and a short sequence (B=256 x
    # T=64 from a seeded state, 4 states in rotation), and seq_b40_t1024:
    # more heads than CUs and a longer sequence (B=40 x T=1024); both take
    # the half-head route with 16-token chunks, 3 workgroups per CU
    for name in ("seq_b256_t64", "seq_b40_t1024"):
        if not want(name):
            continue
        c5 = gi.WORKLOADS[name]
        B, T = c5["B"], c5["T"]
        si = {n: torch.from_numpy(x).cuda() for n, x in gi.step_inputs(c5["seed"], 0, B, T=T).items()}
        sts = [torch.from_numpy(gi.state(c5["seed"], s_, B)).cuda() for s_ in range(4)]
        o = torch.empty((B, T, HV, D), device="cuda")
        k = [0]

        def rot(exact):
            i = k[0] % 4
            k[0] += 1
            g.seq(si["q"], si["k"], si["v"], si["beta"], si["gate"], sts[i], o, stream=stream,
                  exact=exact)
        reps = 8 if T <= 64 else 3
        ms = min(timeit(lambda: rot(False), reps) for _ in range(3))
        ms_x = min(timeit(lambda: rot(True), reps) for _ in range(3))
        upd = B * T * HV
        tf = upd * D * D * 7 / (ms / 1e3) / 1e12
        res[name] = {"ms": ms, "state_updates_per_s": upd / (ms / 1e3),
                     "TFLOPs": tf, "flop_per_element": 7,
                     "frac_fp32_vector_nonpacked_78.6": tf / 78.6,
                     # executed with the scaled decay: 6 flop per element
                     "executed_TFLOPs_6_flop_per_element": tf * 6 / 7,
                     "executed_frac_fp32_vector_nonpacked_78.6": tf * 6 / 7 / 78.6,
                     "state_GBps": B * HV * 2 * D * D * 4 / (ms / 1e3) / 1e9,
                     "exact_ms": ms_x,
                     "exact_TFLOPs": upd * D * D * 7 / (ms_x / 1e3) / 1e12}
        del sts, si, o

    # tail_b32: layer tail B=32
    if want("tail_b32"):
        c4 = gi.WORKLOADS["tail_b32"]
        ti = {n: torch.from_numpy(x).cuda() for n, x in gi.tail_inputs(c4["seed"], 32).items()}
        M = torch.from_numpy(gi.state(c4["seed"], 0, 32)).cuda()
        y = torch.empty((32, HV * D), device="cuda")
        ws = torch.empty(g.layer_tail_workspace_bytes(32), dtype=torch.uint8, device="cuda")
        ms = timeit(lambda: g.layer_tail(ti["x"], ti["conv_w"], ti["conv_state"], ti["beta"],
                                         ti["gate"], M, ti["z"], ti["norm_w"], y, workspace=ws,
                                         stream=stream), 200)
        res["tail_b32"] = {"us_per_call": ms * 1e3,
                                         "state_updates_per_s": 32 * HV / (ms / 1e3)}
        three = g.TailParams(4, 128, 1e-6, 1)
        ms = timeit(lambda: g.layer_tail(ti["x"], ti["conv_w"], ti["conv_state"], ti["beta"],
                                         ti["gate"], M, ti["z"], ti["norm_w"], y, workspace=ws,
                                         params=three, stream=stream), 200)
        res["tail_b32"]["three_launch_us_per_call"] = ms * 1e3
        # the same call over 6 state sets in rotation (768 MiB of state, more
        # than the 256 MB Infinity Cache holds): an HBM-streaming figure
        sets = [torch.from_numpy(gi.state(c4["seed"], s_, 32)).cuda() for s_ in range(6)]
        css = [ti["conv_state"].clone() for _ in range(6)]
        k = [0]

        def rot():
            i = k[0] % 6
            k[0] += 1
            g.layer_tail(ti["x"], ti["conv_w"], css[i], ti["beta"], ti["gate"], sets[i], ti["z"],
                         ti["norm_w"], y, workspace=ws, stream=stream)
        ms = timeit(rot, 120)
        res["tail_b32"]["rotating_6_states_us_per_call"] = ms * 1e3
        res["tail_b32"]["rotating_GBps"] = TAIL_B32_BYTES / (ms / 1e3) / 1e9
        res["tail_b32"]["rotating_frac_of_8TBps"] = TAIL_B32_BYTES / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS
        # gdn_layer_tail_pair over the same rotating states: both positions,
        # ring and state read once and written twice
        t2 = {n: torch.from_numpy(x).cuda() for n, x in gi.tail_inputs(c4["seed"], 32, slot=1).items()}
        pr = {n: torch.stack([ti[n], t2[n]], dim=1).contiguous() for n in ("x", "beta", "gate", "z")}
        nxt = [torch.empty_like(sets[0]), torch.empty_like(css[0])]
        y2 = torch.empty((32, 2, HV * D), device="cuda")

        def rot_pair():
            i = k[0] % 6
            k[0] += 1
            g.layer_tail_pair(pr["x"], ti["conv_w"], css[i], nxt[1], pr["beta"], pr["gate"],
                              sets[i], nxt[0], pr["z"], ti["norm_w"], y2, stream=stream)
        ms = timeit(rot_pair, 120)
        res["tail_b32"]["pair_rotating_us_per_call"] = ms * 1e3
        res["tail_b32"]["pair_bytes_per_call"] = TAIL_PAIR_B32_BYTES
        res["tail_b32"]["pair_rotating_GBps"] = TAIL_PAIR_B32_BYTES / (ms / 1e3) / 1e9
        del sets, css, nxt
        # the same tail starting from the raw beta/alpha logits (gdn_layer_tail_ba)
        gin = {n: torch.from_numpy(x).cuda() for n, x in gi.gate_inputs(c4["seed"], 32).items()}
        wsb = torch.empty(g.layer_tail_ba_workspace_bytes(32), dtype=torch.uint8, device="cuda")
        ms = timeit(lambda: g.layer_tail_ba(ti["x"], ti["conv_w"], ti["conv_state"], gin["ba"],
                                            gin["a_log"], gin["dt_bias"], M, ti["z"], ti["norm_w"],
                                            y, workspace=wsb, stream=stream), 200)
        res["tail_b32"]["raw_gates_us_per_call"] = ms * 1e3
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the decode step has no cross-GPU exchange and shards by sequence", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_deltanet_decode_amd as g
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    stream = torch.cuda.current_stream()
    if args.workload != "step_b256_x36":
        res = extra_measurements(torch, g, stream, only=args.workload)
        print(json.dumps({"workload": args.workload, "extra": res}), flush=True)
        return
    copy_gbps = copy_probe(torch, stream)
    plain_copy_gbps = copy_probe(torch, stream, tuned=False)
    log(f"[bench] copy probes: tuned {copy_gbps:.0f} GB/s, plain {plain_copy_gbps:.0f} GB/s")
    w = setup_step_b256_x36(torch, g)
    L, B = w["L"], w["B"]
    inplace_gbps = inplace_probe(torch, stream, w["states"][0])
    walk_gbps = inplace_probe(torch, stream, w["states"][0], staged=False)
    log(f"[bench] in-place probes (no arithmetic): the step's staged pattern {inplace_gbps:.0f} "
        f"GB/s, the tile walk {walk_gbps:.0f} GB/s")
    read_gbps, write_gbps = one_direction_probes(torch, stream, w["states"][0])
    log(f"[bench] the same walk one way: read only {read_gbps:.0f} GB/s, write only "
        f"{write_gbps:.0f} GB/s")
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        run_step36(g, w, stream)
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps x {L} gdn_step launches")
    # The timed region holds nothing but the K x 36 launches; its duration
    # from HIP events on the launch stream, divided by the launches, is the
    # mean launch duration (gaps between back-to-back launches included).
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        run_step36(g, w, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)

    updates_per_step = L * B * HV
    ms_per_step = ms_total / args.steps
    value = updates_per_step / (ms_per_step / 1e3)
    bytes_per_launch = B * HV * STATE_UPDATE_BYTES
    avg_launch_ms = ms_per_step / L
    achieved = bytes_per_launch / (avg_launch_ms / 1e3) / 1e9
    # A separate pass, outside the timed region: each launch of 3 more steps
    # bracketed by its own pair of events (the event records between kernels
    # slow those steps slightly; context only).
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(L)] for _ in range(3)]
    for s in range(3):
        run_step36(g, w, stream, evs[s])
    torch.cuda.synchronize()
    launch_ms = [evs[s][l][0].elapsed_time(evs[s][l][1]) for s in range(3) for l in range(L)]
    log(f"[bench] {ms_per_step:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}), "
        f"{avg_launch_ms * 1e3:.1f} us per launch; {achieved:.0f} GB/s; event-bracketed "
        f"launches: mean {np.mean(launch_ms) * 1e3:.1f} us min {min(launch_ms) * 1e3:.1f} "
        f"max {max(launch_ms) * 1e3:.1f}")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gdn_step decode, B=256 sequences x 36 layers (one 512 MiB "
                               "state per layer, 18 GiB), 32 value / 16 key heads, d=128, "
                               "one token per layer",
                   "global_batch": B, "layers": L, "launches_per_step": L,
                   "seed": gi.WORKLOADS["step_b256_x36"]["seed"]},
        "achieved_GBps_step": updates_per_step * STATE_UPDATE_BYTES / (ms_per_step / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "k_step_staged (gdn_step)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(),
                     "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": avg_launch_ms * 1e3,
                     "launches_timed": L * args.steps,
                     "copy_probe_GBps": copy_gbps,
                     "frac_of_copy_probe": achieved / copy_gbps,
                     "plain_copy_probe_GBps": plain_copy_gbps,
                     "inplace_probe_GBps": inplace_gbps,
                     "frac_of_inplace_probe": achieved / inplace_gbps,
                     "walk_inplace_probe_GBps": walk_gbps,
                     "read_only_probe_GBps": read_gbps,
                     "write_only_probe_GBps": write_gbps,
                     "event_bracketed_launch_us": float(np.mean(launch_ms)) * 1e3,
                     "event_bracketed_launches": len(launch_ms)},
    }
    if not args.no_extra:
        log("[bench] graph replay and flattened single launch of the 36 layers")
        line["extra_step_b256_x36"] = step_b256_x36_variants(torch, g, w, stream, args.steps)
        log("[bench] secondary entry points")
        del w
        torch.cuda.empty_cache()
        line["extra"] = extra_measurements(torch, g, stream)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
