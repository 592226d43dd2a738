#!/usr/bin/env python3
"""Benchmark of the latent-MoE output tail on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

One step = one lt_latent_tail call at every token count of the sweep
T = 1, 2, 4, ..., 8192 (L=1024, H=7168, full column window n=7168, one
partial, RMSNorm on, eps=1e-6): every step of the tail runs in every call
(partial sum, bf16 round trip, RMSNorm, projection, beta-add), the small
token counts on the weight-streaming kernel and the large ones on the
sum+RMSNorm kernel followed by the MFMA GEMM.

Inputs are seeded synthetic bf16 data (latent_moe_output_amd.synth, decode
recipe at T=8192, the smaller T take its first rows), resident in HBM before
the timed region.  To measure HBM rather than the 256 MB Infinity Cache,
every call reads a different copy of W (a pool of 48 copies, 704 MB) and
rotates through enough copies of its partials/out to cycle >= 512 MB.

Printed: ONE JSON line on stdout.  `value` is the whole-job throughput:
algorithmic flops of the K timed steps / wall-clock time between two device
synchronisations.  The timed steps run as HIP graphs of ten sweeps (each
call on its own W copy and rotation set, so a replay cycles the whole W pool)
replayed back to back right after the W warmup sweeps, the way a serving loop
launches them; `value_direct_launch` is the same K steps launched call by call
from Python just before, from a GPU that was idle while the graphs were
captured (and so starts at its idle clocks).  Per-T figures come from a separate
instrumented pass: HIP events recorded on the benchmark stream around each
call and, through lt_set_kernel_events, around its projection kernel, each
call queued behind a short GPU spin so that host launch time stays outside
the events; `graph_call_us` is each T on its own: its rotation sets captured
into one graph (each call on its own W copy) and replayed, elapsed time per
call (its `w_stream_gbps` is the W window over that time).  `roofline` is
for the dominant kernel (k_gemm_ring at T=8192); `roofline_skinny` for the
weight-streaming kernel at T <= 16, whose W-window rate is the top-level
`w_stream_gbps`; `context.single_launch_floor` times a probe launch of the
same shape that only streams the W window (and an empty one).  `configs`
times the column-shard workloads (T=256 with 8 partials, T=8191 with 4
partials, with and without the norm, 896-column windows) and `attn_res` the
AttnRes zero-block call (hidden 7168, every switch on) against their
rooflines.  `cpu_baseline` times the fp64 CPU oracle (median of three runs)
on a bounded sample of the T=8192 call on this host's cores.
`roofline.traffic` is the GEMM's HBM bytes per launch from the committed
rocprofv3 counter summary under profiles/, or null once the GEMM sources
differ from the ones those counters were taken on.

    python bench.py --workload NAME --steps K

times one workload alone (decodeN, shard, ragged, ragged_nonorm, prefill,
attn_resN) and prints one JSON line; it is what the profiles under
profiles/ run.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "latent-tail TFLOP/s + W-stream GB/s vs roofline, T=1..8192, L=1024, H=7168"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, MI355X dense bf16
T_SWEEP = [1 << i for i in range(14)]
L, H, P, EPS = 1024, 7168, 1, 1e-6
N_WPOOL = 48
SPIN_CYCLES = 200_000   # GPU spin (about 0.1 ms) queued ahead of an event-timed call
ROTATE_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_of(T, n=H, L_=L):
    return 2 * T * L_ * n


def bytes_of(T, n=H, L_=L, P_=P, norm=True):
    """Algorithmic HBM bytes of one call: W window once, every partial once,
    the norm weight, a read and a write of the out window."""
    return 2 * n * L_ + 2 * P_ * T * L_ + 4 * T * n + (2 * L_ if norm else 0)


class Hip:
    """The few HIP runtime calls the benchmark needs (events), via ctypes."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed: %d" % rc)
        return ev.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_by_workload.md")
GEMM_SOURCES = [os.path.join(ROOT, "latent_moe_output_amd", "csrc", f)
                for f in ("k_gemm.hip", "lt_device.h")]


def gemm_traffic_bytes():
    """HBM bytes per launch of the T=8192 GEMM from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled against a plain copy), or None
    when the GEMM sources changed since the counters were taken."""
    import hashlib

    try:
        text = open(TRAFFIC_FILE).read()
        src = b"".join(open(f, "rb").read() for f in GEMM_SOURCES)
    except OSError:
        return None
    sha = hashlib.sha256(src).hexdigest()
    for line in text.splitlines():
        if line.startswith("traffic_k_gemm_T8192 "):
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("sources_sha256") == sha:
                return int(kv["bytes"])
    return None


RES_T = [1, 16, 1024, 8192]


def context_pass(binding, hip, stream, sh, sets, wpool, norm_w, reps=20):
    """Context for the roofline fractions, not part of `value`: the copy
    bandwidth this GPU reaches on a W-sized buffer (PyTorch device copy), and
    warm timings (the same W, partials and out every call, so W stays in the
    256 MB Infinity Cache) next to the cold ones."""
    import numpy as np
    import torch

    ctx = {}
    with torch.cuda.stream(stream):
        a, b = hip.event(), hip.event()
        big = [torch.empty(64 << 20, dtype=torch.int16, device="cuda") for _ in range(2)]
        for _ in range(3):
            big[1].copy_(big[0])
        hip.record(a, sh)
        for i in range(reps):
            big[(i + 1) % 2].copy_(big[i % 2])
        hip.record(b, sh)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(a, b) * 1e3 / reps
        ctx["copy_128MiB"] = {"us": round(us, 2),
                              "gbps_read_plus_write": round(2 * big[0].numel() * 2 / us / 1e3, 1)}
        del big
        warm = {}
        for T in (1, 8192):
            p, o = sets[T][0]
            W = wpool[0]
            for _ in range(3):
                binding.check(binding.lt_latent_tail(p, P, T, L, norm_w, EPS, W, H, 0, H, o, H, sh))
            hip.record(a, sh)
            for _ in range(reps):
                binding.check(binding.lt_latent_tail(p, P, T, L, norm_w, EPS, W, H, 0, H, o, H, sh))
            hip.record(b, sh)
            torch.cuda.synchronize()
            warm[str(T)] = {"call_us": round(hip.elapsed_ms(a, b) * 1e3 / reps, 3),
                            "timing": "%d back-to-back calls" % reps}
        ctx["warm_same_buffers"] = warm
        hip.destroy(a)
        hip.destroy(b)
    ctx["single_launch_floor"] = launch_floor(hip, stream, sh, wpool)
    ctx["clocks"] = gpu_clocks()
    ctx["power_under_load"] = power_under_load(binding, stream, sh, sets, wpool, norm_w)
    return ctx


def under_profiler():
    return "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ)


def power_under_load(binding, stream, sh, sets, wpool, norm_w, seconds=3.0, samples=3):
    """Socket power and per-XCD shader clocks (`amd-smi metric -p -c`) while
    the T = 8192 call (norm + GEMM, own W copy per call) runs back to back
    for a few seconds, next to the package power cap (`rocm-smi
    --showmaxpower`): whether the GEMM runs at the nominal clock the MFMA
    peak assumes or at a power-limited one.  None under a profiler or where
    the tools are missing."""
    import re
    import subprocess
    import threading
    import time
    import torch

    if under_profiler():
        return None

    def sample():
        try:
            r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                               timeout=30)
        except (OSError, subprocess.SubprocessError):
            return None
        watts = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
        gfx = re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", r.stdout)
        if not watts or not gfx:
            return None
        return {"socket_power_w": float(watts[0]),
                "gfx_clk_mhz": [float(x) for x in gfx]}

    T = 8192
    p, _ = sets[T][0]
    o = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    R = 8
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(R):
            binding.check(binding.lt_latent_tail(p, P, T, L, norm_w, EPS, wpool[i % len(wpool)], H,
                                                 0, H, o, H, sh))
    reps = int(seconds / (R * 125e-6))

    def work():
        with torch.cuda.stream(stream):
            for _ in range(reps):
                g.replay()

    th = threading.Thread(target=work)
    th.start()
    time.sleep(1.2)
    got = []
    for _ in range(samples):
        x = sample()
        if x is not None:
            got.append(x)
        time.sleep(0.2)
    th.join()
    torch.cuda.synchronize()
    del g, o
    cap = None
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True, timeout=20)
        m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", r.stdout)
        cap = float(m.group(1)) if m else None
    except (OSError, subprocess.SubprocessError):
        pass
    if not got:
        return None
    clk = [sum(x["gfx_clk_mhz"]) / len(x["gfx_clk_mhz"]) for x in got]
    return {"socket_power_w": [x["socket_power_w"] for x in got],
            "gfx_clk_mhz_mean_over_xcds": [round(c, 1) for c in clk],
            "power_cap_w": cap,
            "workload": "T=8192 call (norm + GEMM, n=7168) back to back for about %.1f s, "
                        "sampled %d times after 1.2 s" % (seconds, len(got))}


def launch_floor(hip, stream, sh, wpool, reps=10):
    """What one launch at the weight-streaming kernel's shape (256 workgroups
    of 512 threads, one 57,344-byte share of the W window each) costs back to
    back when it does nothing but stream the W window into LDS (probe kernel
    of libltprobe.so, each launch on its own W copy), and when its body is
    empty.  The decode call cannot be faster than the stream probe."""
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "latent_moe_output_amd", "probe", "libltprobe.so"))
    lib.ltp_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                               ctypes.c_void_p]
    lib.ltp_empty.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
    nwg, nthr = 256, 512
    share = 2 * H * L // nwg                         # 57,344 bytes: 28 W rows
    res = {}
    for name, one in (("stream_w_window", lambda i: lib.ltp_stream(wpool[i % len(wpool)].data_ptr(),
                                                                    share, nwg, nthr, sh)),
                      ("empty", lambda i: lib.ltp_empty(nwg, nthr, sh))):
        R = len(wpool)
        for i in range(R):
            assert one(i) == 0
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(R):
                assert one(i) == 0
        with torch.cuda.stream(stream):
            g.replay()
            a, b = hip.event(), hip.event()
            hip.record(a, sh)
            for _ in range(reps):
                g.replay()
            hip.record(b, sh)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(a, b) * 1e3 / (reps * R)
        hip.destroy(a)
        hip.destroy(b)
        res[name] = {"us_per_launch": round(us, 3)}
        del g
    w = 2 * H * L
    res["stream_w_window"]["gbps"] = round(w / res["stream_w_window"]["us_per_launch"] / 1e3, 1)
    res["stream_w_window"]["frac_of_hbm_roofline"] = round(
        w / HBM_PEAK / (res["stream_w_window"]["us_per_launch"] * 1e-6), 4)
    res["shape"] = "%d workgroups x %d threads, %d bytes each, back to back in a graph of %d " \
                   "launches (own W copy each)" % (nwg, nthr, share, len(wpool))
    return res


def gpu_clocks():
    """The clock lines `rocm-smi --showclocks` prints for the first card
    (current levels right after the timed work), or None where the tool is
    missing or fails, and under a profiler: its preloaded library would start
    the GPU in the child before rocm-smi's launcher hands over to python."""
    import subprocess

    if under_profiler():
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        cards = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    if not isinstance(cards, dict) or not cards:
        return None
    first = cards[sorted(cards)[0]]
    if not isinstance(first, dict):
        return None
    return {k: v for k, v in first.items() if "clock" in k.lower() or "clk" in k.lower()}


def residual_pass(binding, hip, stream, sh, sets, wpool, norm_w, call_kern, reps=20):
    """The residual form (the tail plus the decoder layer's prefix-sum update,
    fused into the epilogue) against the unfused pair: the tail, then a
    separate bf16 add of prefix + out (PyTorch's elementwise kernel on the
    same stream).  Kernel times from HIP events around each launch."""
    import numpy as np
    import torch

    res = {}
    with torch.cuda.stream(stream):
        for T in RES_T:
            pre = [torch.randn(T, H, device="cuda").to(torch.bfloat16) for _ in range(2)]
            rsd = [torch.empty_like(p) for p in pre]
            ev = [(hip.event(), hip.event(), hip.event(), hip.event()) for _ in range(reps)]
            for i in range(reps + 2):
                p, o = sets[T][i % len(sets[T])]
                W = wpool[(7 * i) % len(wpool)]
                e = ev[i - 2] if i >= 2 else None
                torch.cuda._sleep(SPIN_CYCLES)   # host enqueue time off the timed span
                if e:
                    binding.lt_set_kernel_events(e[0], e[1])
                binding.check(binding.lt_latent_tail_residual(
                    p, P, T, L, norm_w, EPS, W, H, 0, H, o, H, pre[i % 2], H, rsd[i % 2], H, sh))
                binding.lt_set_kernel_events(None, None)
                torch.cuda._sleep(SPIN_CYCLES)
                if e:
                    hip.record(e[2], sh)
                torch.add(pre[i % 2], o.view(torch.bfloat16), out=rsd[i % 2])
                if e:
                    hip.record(e[3], sh)
            torch.cuda.synchronize()
            fused = float(np.mean([hip.elapsed_ms(e[0], e[1]) * 1e3 for e in ev]))
            add = float(np.mean([hip.elapsed_ms(e[2], e[3]) * 1e3 for e in ev]))
            for e in ev:
                for x in e:
                    hip.destroy(x)
            res[str(T)] = {
                "fused_kernel_us": round(fused, 3),
                "tail_kernel_us": round(call_kern[T], 3),
                "separate_add_us": round(add, 3),
                "unfused_us": round(call_kern[T] + add, 3),
                "extra_bytes": 4 * T * H,
            }
            del pre, rsd
    return res


CONFIG_RUNS = ("shard", "ragged", "ragged_nonorm")


def tail_workload(name):
    """A workload of synth.WORKLOADS by name; `decodeN` is the decode shape at
    T = N."""
    from latent_moe_output_amd import synth

    if name.startswith("decode") and name[6:].isdigit():
        return synth.WORKLOADS["decode"].with_T(int(name[6:]))
    return synth.WORKLOADS[name]


def time_workload(binding, hip, stream, sh, wl, wpool, reps=10):
    """One tail workload at its real shape: inputs drawn on the device (same
    distributions as the host generator; the ragged workload's +-1e4 outliers
    are left out, they do not change the work), each call on its own W copy
    and a rotated partials/out set, R calls captured into one graph and
    replayed `reps` times; back-to-back time per call."""
    import torch

    from latent_moe_output_amd import synth

    per = 2 * wl.P * wl.T * wl.L + 2 * wl.T * wl.ld_out
    R = int(min(16, max(2, math.ceil(ROTATE_BYTES / per))))
    with torch.cuda.stream(stream):
        sets = [synth.generate_device(wl, seed=s) for s in range(R)]
    torch.cuda.synchronize()
    nw = sets[0]["norm_w"]
    binding.check(binding.lt_reserve(wl.T, wl.L, sh))

    def one(i):
        d = sets[i % R]
        return binding.lt_latent_tail(d["partials"], wl.P, wl.T, wl.L, nw, wl.eps,
                                      wpool[(5 * i) % len(wpool)], wl.H, wl.c0, wl.n,
                                      d["out"], wl.ld_out, sh)

    for i in range(R):
        binding.check(one(i))
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(R):
            binding.check(one(i))
    with torch.cuda.stream(stream):
        g.replay()
        a, b = hip.event(), hip.event()
        hip.record(a, sh)
        for _ in range(reps):
            g.replay()
        hip.record(b, sh)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(a, b) * 1e3 / (reps * R)
    hip.destroy(a)
    hip.destroy(b)
    del sets, g
    torch.cuda.synchronize()
    f = 2 * wl.T * wl.L * wl.n
    byt = 2 * wl.n * wl.L + 2 * wl.P * wl.T * wl.L + 4 * wl.T * wl.n + (2 * wl.L if wl.norm else 0)
    roof_us = max(byt / HBM_PEAK, f / MFMA_BF16_PEAK) * 1e6
    return {
        "T": wl.T, "n_partials": wl.P, "c0": wl.c0, "n": wl.n, "ld_out": wl.ld_out,
        "norm": wl.norm,
        "path": ("skinny" if binding.lt_path_for(wl.T, wl.n) == 1 else
                 ("sum+norm, gemm" if wl.norm else "sum, gemm" if wl.P > 1 else "gemm")),
        "call_us": round(us, 3),
        "tflops": round(f / us / 1e6, 2),
        "alg_gbps": round(byt / us / 1e3, 1),
        "alg_bytes": byt,
        "roofline_us": round(roof_us, 3),
        "bound": "hbm" if byt / HBM_PEAK > f / MFMA_BF16_PEAK else "mfma",
        "frac_of_roofline": round(roof_us / us, 3),
        "timing": "graph of %d calls (own W copy and input set each) replayed %d times"
                  % (R, reps),
    }


def configs_pass(binding, hip, stream, sh, wpool, reps=10):
    """The column-shard workloads at their real shapes (not part of `value`):
    the 8-partial shard (T=256, window of 896 columns) and the ragged prefill
    shard (T=8191, 4 partials, window of 896 columns) with and without the
    norm."""
    return {name: time_workload(binding, hip, stream, sh, tail_workload(name), wpool, reps)
            for name in CONFIG_RUNS}


ATTN_RES_T = (1, 3, 7, 17, 320)
ATTN_RES_H = 7168
ATTN_RES_SLOTS = 9


def attn_res_bytes(T, H=ATTN_RES_H):
    """Algorithmic bytes of one AttnRes zero-block call with every switch on:
    prefix and delta read, prefix, block slot and output written, the norm
    weight read once."""
    return 10 * T * H + 2 * H


def time_attn_res(binding, hip, stream, sh, T, H=ATTN_RES_H, reps=20):
    """lt_attn_res_zero_block with the delta, the block write and the output
    norm, on rotated input sets (>= 256 MB for T >= 320), R calls captured
    into one graph and replayed; back-to-back time per call."""
    import torch

    per = 2 * T * H * (3 + ATTN_RES_SLOTS)
    R = int(min(64, max(2, math.ceil((256 << 20) / per))))
    with torch.cuda.stream(stream):
        g0 = torch.Generator(device="cuda")
        g0.manual_seed(T)

        def draw(shape, std=1.0, mean=0.0):
            x = torch.randn(shape, generator=g0, device="cuda") * std + mean
            return x.to(torch.bfloat16).view(torch.int16)

        sets = [dict(p=draw((T, H)), d=draw((T, H), 0.1), b=draw((T, ATTN_RES_SLOTS, H)),
                     o=torch.empty((T, H), dtype=torch.int16, device="cuda"))
                for _ in range(R)]
        w = draw((H,), 0.1, 1.0)
    torch.cuda.synchronize()

    def one(i):
        d = sets[i % R]
        return binding.lt_attn_res_zero_block(d["p"], d["d"], T, H, d["b"], ATTN_RES_SLOTS,
                                              i % ATTN_RES_SLOTS, w, EPS, d["o"], sh)

    for i in range(R):
        binding.check(one(i))
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(R):
            binding.check(one(i))
    with torch.cuda.stream(stream):
        g.replay()
        a, b = hip.event(), hip.event()
        hip.record(a, sh)
        for _ in range(reps):
            g.replay()
        hip.record(b, sh)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(a, b) * 1e3 / (reps * R)
    hip.destroy(a)
    hip.destroy(b)
    del sets, g
    torch.cuda.synchronize()
    byt = attn_res_bytes(T, H)
    return {"T": T, "H": H, "call_us": round(us, 3), "alg_bytes": byt,
            "alg_gbps": round(byt / us / 1e3, 1), "roofline_us": round(byt / HBM_PEAK * 1e6, 3),
            "frac_of_roofline": round(byt / HBM_PEAK / (us * 1e-6), 4), "bound": "hbm",
            "timing": "graph of %d calls (own input set each) replayed %d times" % (R, reps)}


def attn_res_pass(binding, hip, stream, sh):
    """The AttnRes zero-block path at the pages' contract token counts
    (hidden 7168, every switch on)."""
    return {str(T): time_attn_res(binding, hip, stream, sh, T) for T in ATTN_RES_T}


def single_workload(name, steps):
    """Time one workload alone (for profilers): `decodeN`, `shard`, `ragged`,
    `ragged_nonorm`, `prefill` or `attn_resN` (AttnRes zero-block path at
    T = N, hidden 7168).  Prints one JSON line."""
    import torch

    from latent_moe_output_amd import binding

    binding.load()
    binding.lt_set_skinny_max_tokens(-1)
    hip = Hip()
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    reps = max(1, steps)
    if name.startswith("attn_res"):
        res = time_attn_res(binding, hip, stream, sh, int(name[8:] or 320), reps=reps)
    else:
        wl = tail_workload(name)
        nw = int(min(48, max(2, math.ceil(ROTATE_BYTES / (2 * wl.n * wl.L)))))
        with torch.cuda.stream(stream):
            g0 = torch.Generator(device="cuda")
            g0.manual_seed(0)
            W0 = (torch.randn((wl.H, wl.L), generator=g0, device="cuda") * wl.w_std).to(
                torch.bfloat16).view(torch.int16)
            wpool = [W0] + [W0.clone() for _ in range(nw - 1)]
        torch.cuda.synchronize()
        res = time_workload(binding, hip, stream, sh, wl, wpool, reps=reps)
    print(json.dumps(dict(workload=name, **res)), flush=True)


def cpu_baseline(d, target_s=4.0):
    """The fp64 oracle as it stands on this host's cores, on the first S tokens
    of the T=8192 call (S sized for ~target_s seconds of work), timed three
    times (the median is reported)."""
    from oracle import oracle

    oracle.build(force=False)
    threads = oracle.max_threads()
    cal_T = 16
    t0 = time.perf_counter()
    oracle.latent_tail(d["partials"][:, :cal_T], d["norm_w"], EPS, d["W"], 0, H,
                       d["out"][:cal_T])
    cal = time.perf_counter() - t0
    S = int(max(cal_T, min(8192, cal_T * target_s / max(cal, 1e-6))))
    S = max(cal_T, (S // 16) * 16)
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.latent_tail(d["partials"][:, :S], d["norm_w"], EPS, d["W"], 0, H, d["out"][:S])
        runs.append(time.perf_counter() - t0)
    dt = sorted(runs)[1]
    # the same oracle on one thread, on a sample a sixteenth the size
    S1 = max(16, (S // 16) // 16 * 16)
    t0 = time.perf_counter()
    oracle.latent_tail(d["partials"][:, :S1], d["norm_w"], EPS, d["W"], 0, H, d["out"][:S1],
                       nthreads=1)
    dt1 = time.perf_counter() - t0
    oracle.latent_tail(d["partials"][:, :16], d["norm_w"], EPS, d["W"], 0, H, d["out"][:16],
                       nthreads=threads)                       # restore the thread count
    return {
        "value": flops_of(S) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d of the 8192 tokens of the T=8192 call (L=1024, n=7168, one "
                  "partial, RMSNorm on), fp64 C oracle, %d OpenMP threads, median of 3 runs "
                  "(%.2f s)" % (S, threads, dt),
        "seconds": dt,
        "seconds_runs": [round(x, 3) for x in runs],
        "tokens": S,
        "cpu_model": cpu_model(),
        "single_thread": {"value": flops_of(S1) / dt1 / 1e12, "unit": "TFLOP/s",
                          "tokens": S1, "seconds": dt1},
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=4.0)
    ap.add_argument("--workload", default=None,
                    help="time one workload alone and exit (decodeN, shard, ragged, "
                         "ragged_nonorm, prefill, attn_resN); for profilers")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the tail on one GPU only: the kernel works on one GPU's "
              "share at its real shape and nothing here talks to a second GPU "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.workload:
        single_workload(args.workload, args.steps)
        return

    import numpy as np
    import torch

    from latent_moe_output_amd import binding, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    binding.lt_set_skinny_max_tokens(-1)
    hip = Hip()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    sh = stream.cuda_stream

    wl = synth.WORKLOADS["decode"].with_T(max(T_SWEEP))
    log("generating inputs ...")
    d = synth.generate(wl, seed=0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).to(dev)

    with torch.cuda.stream(stream):
        W0 = to_dev(d["W"])
        wpool = [W0] + [W0.clone() for _ in range(N_WPOOL - 1)]
        norm_w = to_dev(d["norm_w"])
        part_all = to_dev(d["partials"])
        out_all = to_dev(d["out"])
        sets = {}
        for T in T_SWEEP:
            per = 2 * P * T * L + 2 * T * H
            R = int(min(48, max(2, math.ceil(ROTATE_BYTES / per))))
            sets[T] = [(part_all[:, :T].clone(), out_all[:T].clone()) for _ in range(R)]
    del part_all, out_all
    st = binding.lt_reserve(max(T_SWEEP), L, sh)
    binding.check(st)
    torch.cuda.synchronize()
    log("inputs resident: W pool %d x %.1f MB, rotation sets %s" % (
        N_WPOOL, 2 * H * L / 1e6, {T: len(v) for T, v in sets.items()}))

    counter = [0]

    def call(T, step):
        p, o = sets[T][step % len(sets[T])]
        W = wpool[counter[0] % N_WPOOL]
        counter[0] += 1
        return binding.lt_latent_tail(p, P, T, L, norm_w, EPS, W, H, 0, H, o, H, sh)

    # ---- graphs: the sweep captured into HIP graphs of G = 10 steps (every
    # call reads its own W copy and rotation set, so one replay cycles the
    # whole 705 MB W pool and leaves nothing in the 256 MB Infinity Cache for
    # the next), one of K mod G steps, and one of the W warmup steps.  The
    # graph is how a serving loop launches these calls; replay removes the
    # Python launch overhead from the measurement, not any GPU work.
    K = args.steps
    nT = len(T_SWEEP)
    G = min(10, K)

    def capture(nsweeps, first):
        if nsweeps <= 0:
            return None
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for s_ in range(first, first + nsweeps):
                for T in T_SWEEP:
                    binding.check(call(T, s_))
        return g

    g_warm = capture(args.warmup, 0)
    graph = capture(G, args.warmup)
    g_rem = capture(K % G, args.warmup + G)
    torch.cuda.synchronize()

    # ---- the same K steps launched call by call from Python, for reference.
    # It runs first, from a GPU that sat idle while the graphs were captured:
    # after an idle spell the sweep runs about 10 % slower for its first few
    # milliseconds, however it is launched, and the timed region below must
    # not start in that state (at K = 20 it lasts 8 ms; with only the W
    # warmup sweeps before it the graph read 0.393 ms per step, and 0.353
    # on a GPU kept busy).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for T in T_SWEEP:
            binding.check(call(T, s))
    torch.cuda.synchronize()
    wall_direct = time.perf_counter() - t0

    # ---- warmup: the W warmup sweeps, replayed right before the timed region
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    t0 = time.perf_counter()
    for _ in range(K // G):
        graph.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    # ---- instrumented pass (not part of `value`): HIP events around every
    # call and, through lt_set_kernel_events, around its projection kernel
    KI = min(K, 50)
    ev = [[[hip.event() for _ in range(4)] for _ in range(nT)] for _ in range(KI)]
    torch.cuda.synchronize()
    for s in range(KI):
        for i, T in enumerate(T_SWEEP):
            e = ev[s][i]
            # a short spin kernel ahead of each call keeps the GPU busy while
            # the host enqueues the events and the call, so the host's launch
            # time does not land between the events
            with torch.cuda.stream(stream):
                torch.cuda._sleep(SPIN_CYCLES)
            hip.record(e[0], sh)
            binding.lt_set_kernel_events(e[1], e[2])
            st = call(T, s)
            binding.lt_set_kernel_events(None, None)
            hip.record(e[3], sh)
            if st != binding.LT_OK:
                raise binding.LtError(st)
    torch.cuda.synchronize()
    del graph

    # ---- per-T back-to-back time: for each T its R rotation sets (each call
    # on its own W copy) captured into one graph, replayed; per-call time =
    # elapsed / (replays x R), gaps between launches included
    graph_us = {}
    for T in T_SWEEP:
        R = len(sets[T])
        gT = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(gT, stream=stream):
            for s in range(R):
                binding.check(call(T, s))
        reps = max(3, min(20, int(4000 / R / max(1.0, T / 256))))
        with torch.cuda.stream(stream):
            gT.replay()                                  # untimed
            a, b = hip.event(), hip.event()
            hip.record(a, sh)
            for _ in range(reps):
                gT.replay()
            hip.record(b, sh)
        torch.cuda.synchronize()
        graph_us[T] = hip.elapsed_ms(a, b) * 1e3 / (reps * R)
        hip.destroy(a)
        hip.destroy(b)
        del gT

    per_T = []
    call_us = {}
    kern_us = {}
    for i, T in enumerate(T_SWEEP):
        c = [hip.elapsed_ms(ev[s][i][0], ev[s][i][3]) * 1e3 for s in range(KI)]
        k = [hip.elapsed_ms(ev[s][i][1], ev[s][i][2]) * 1e3 for s in range(KI)]
        call_us[T] = float(np.mean(c))
        kern_us[T] = float(np.mean(k))
        f, b = flops_of(T), bytes_of(T)
        roof_us = max(b / HBM_PEAK, f / MFMA_BF16_PEAK) * 1e6
        per_T.append({
            "T": T,
            "path": "skinny" if binding.lt_path_for(T, H) == 1 else "norm+gemm",
            "call_us": round(call_us[T], 3),
            "kernel_us": round(kern_us[T], 3),
            "call_us_median": round(float(np.median(c)), 3),
            "tflops": round(f / call_us[T] / 1e6, 2),
            "w_stream_gbps": round(2 * H * L / graph_us[T] / 1e3, 1),
            "alg_gbps": round(b / call_us[T] / 1e3, 1),
            "roofline_us": round(roof_us, 3),
            "bound": "hbm" if b / HBM_PEAK > f / MFMA_BF16_PEAK else "mfma",
            "frac_of_roofline": round(roof_us / call_us[T], 3),
            "graph_call_us": round(graph_us[T], 3),
            "graph_frac_of_roofline": round(roof_us / graph_us[T], 3),
        })
    for row in ev:
        for e4 in row:
            for e in e4:
                hip.destroy(e)

    residual = residual_pass(binding, hip, stream, sh, sets, wpool, norm_w, call_kern=kern_us)
    context = context_pass(binding, hip, stream, sh, sets, wpool, norm_w)

    total_flops = K * sum(flops_of(T) for T in T_SWEEP)
    value = total_flops / wall / 1e12

    Tg = max(T_SWEEP)
    g_ach = flops_of(Tg) / (kern_us[Tg] * 1e-6)
    roofline = {
        "bound": "mfma",
        "achieved": round(g_ach / 1e12, 2),
        "peak": MFMA_BF16_PEAK / 1e12,
        "unit": "TFLOP/s",
        "frac": round(g_ach / MFMA_BF16_PEAK, 4),
        "traffic": gemm_traffic_bytes(),
        "kernel": "k_gemm_ring, 256x256 tiles, 8 waves (T=8192, L=1024, n=7168)",
        "avg_launch_us": round(kern_us[Tg], 3),
        "flops_per_launch": flops_of(Tg),
    }
    # The peak assumes the 2.4 GHz nominal shader clock; under a sustained
    # load of this call the package sits at its power cap with lower XCD
    # clocks (context.power_under_load).  The same achieved rate against the
    # peak scaled to the mean of those clock readings:
    pul = context.get("power_under_load") or {}
    clk = pul.get("gfx_clk_mhz_mean_over_xcds")
    if clk:
        mhz = sum(clk) / len(clk)
        roofline["frac_at_loaded_clock"] = round(g_ach / (MFMA_BF16_PEAK * mhz / 2400.0), 4)
        roofline["loaded_clock_mhz"] = round(mhz, 1)
    # decode kernel: back-to-back launches (each on its own W copy) between two
    # events, so the events' own cost does not land on a 6 us kernel.  A spin
    # kernel queued first keeps the GPU busy while the host enqueues all of
    # them, so the host's launch rate cannot leave gaps between the kernels.
    sk = [T for T in T_SWEEP if T <= 16]
    NB = 48
    e0, e1 = hip.event(), hip.event()
    for s_ in range(2):
        with torch.cuda.stream(stream):
            torch.cuda._sleep(4_000_000)
        hip.record(e0, sh)
        for i in range(NB):
            binding.check(call(sk[i % len(sk)], i))
        hip.record(e1, sh)
        torch.cuda.synchronize()
    sk_us = hip.elapsed_ms(e0, e1) * 1e3 / NB
    hip.destroy(e0)
    hip.destroy(e1)
    sk_bytes = sum(bytes_of(sk[i % len(sk)]) for i in range(NB)) / NB
    roofline_skinny = {
        "bound": "hbm",
        "achieved": round(sk_bytes / (sk_us * 1e-6) / 1e9, 1),
        "peak": HBM_PEAK / 1e9,
        "unit": "GB/s",
        "frac": round(sk_bytes / (sk_us * 1e-6) / HBM_PEAK, 4),
        "traffic": None,
        "kernel": "k_skinny, one 16-token tile (T=1,2,4,8,16 in turn; L=1024, n=7168)",
        "avg_launch_us": round(sk_us, 3),
        "bytes_per_launch_avg": int(sk_bytes),
        "timing": "%d back-to-back launches between two HIP events, all enqueued "
                  "behind a spin kernel before the first event (includes the GPU's gaps "
                  "between launches)" % NB,
    }

    configs = configs_pass(binding, hip, stream, sh, wpool)
    attn_res = attn_res_pass(binding, hip, stream, sh)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16, decode recipe; W pool of 48 copies + rotated "
                "partials/out so every call reads HBM, not the Infinity Cache)",
        "config": {
            "workload": "latent-MoE tail, T sweep 1..8192 (powers of 2), L=1024, H=7168, "
                        "full window c0=0 n=7168, 1 partial, RMSNorm on, eps=1e-6",
            "T_sweep": T_SWEEP, "L": L, "H": H, "n": H, "c0": 0, "n_partials": P,
            "skinny_max": binding.lt_get_skinny_max_tokens(),
        },
        "w_stream_gbps": round(roofline_skinny["achieved"] * (2 * H * L)
                               / roofline_skinny["bytes_per_launch_avg"], 1),
        "w_stream_note": "W-window bytes (2*n*L) per decode launch (T <= 16) / its back-to-back "
                         "time; roofline_skinny has the same launches against all their bytes",
        "launch": "HIP graph of %d sweeps (%d calls) replayed %d times%s, right after the %d "
                  "warmup sweeps (also a graph), which follow the direct-launch pass" % (
                      G, G * nT, K // G, " + one of %d sweeps" % (K % G) if K % G else "",
                      args.warmup),
        "value_direct_launch": round(total_flops / wall_direct / 1e12, 2),
        "ms_per_step_direct_launch": round(wall_direct / K * 1e3, 4),
        "per_T": per_T,
        "roofline": roofline,
        "roofline_skinny": roofline_skinny,
        "residual": residual,
        "configs": configs,
        "attn_res": attn_res,
        "context": context,
    }
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
