"""Benchmark of the biased multi-query attention hot path on one MI355X.

One step = the full-context workload: 9 independent seeded layers (one per
transformer block), each = pair-bias projection ([512,512,128] bf16 ->
8 heads of 512 x 512 cells) + biased soft-capped MQA forward (B=1, S=8192,
8 query heads, 1 K/V head, d=128, bf16 inputs, fp32 accumulation), back to
back on one stream with every input already resident in HBM.

Two routes compute a layer: the pair form (the default), one
kernel that projects the bias cells it uses inside the attention and never
writes a bias tensor; and two kernels, the projection writing the compact
fp32 bias and the attention reading it.  The route not timed is measured
after it, for comparison.

Before each route's W warmup steps it runs untimed steps for --settle-ms
(300 ms): under sustained load the clock takes tens of milliseconds to
settle, and a route timed before that reads slow.

Prints ONE JSON line: attention TFLOP/s over the whole step (FLOPs =
2*B*Hq*S^2*(Dk + Dv) per layer, non-causal QK^T + PV), the roofline of the dominant
kernel from HIP events on its own stream, and the CPU oracle timed on a
bounded sample (3 of the 9 layers by default) on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--cpu-layers N]
                    [--dv 128|192] [--workload full|mid|shard] [--kv-splits N|auto]
                    [--path pair|two] [--settle-ms T] [--copy-mib N]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

#: MI355X published dense peaks used for the roofline.
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "biased_mqa_fwd_full_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(B, S, H=8, Dk=128, Dv=128, Sq=None):
    """QK^T + PV multiply-adds, non-causal: 2 B H Sq S (Dk + Dv) (Sq = S unless
    only a block of query positions is computed)."""
    return 2.0 * B * H * (S if Sq is None else Sq) * S * (Dk + Dv)


def proj_bytes(P, C, H=8, elem=2):
    return P * P * C * elem + C * H * elem + H * P * P * 4


def proj_flops(P, C, H=8):
    return 2.0 * P * P * C * H


def source_digest():
    """First 16 hex digits of the sha256 of the attention kernel's source and
    its launch header with // comments and runs of white space removed: an
    edit of the comments keeps counters taken on the kernel, any change of
    the code drops them."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("biased_mqa_fwd.hip", "abg_internal.h"):
        with open(os.path.join(ROOT, "long_context_biased_amd", "csrc", f)) as fh:
            code = re.sub(r"//[^\n]*", "", fh.read())
        h.update(re.sub(r"\s+", " ", code).encode())
    return h.hexdigest()[:16]


def load_counters(path):
    """HBM bytes and MFMA counters per launch of the timed kernel (the pair
    form, or the attention of the two-kernel route) from the committed
    rocprofv3 summary, if it was taken on the current kernel source and
    route; else None."""
    try:
        kv = {}
        with open(COUNTERS_FILE) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_digest") != source_digest() or kv.get("path", "two") != path:
            return None
        return {"hbm_bytes_per_launch": float(kv["hbm_bytes_per_launch"]),
                "mfma_flops_per_launch": float(kv["mfma_flops_per_launch"]),
                "mfma_busy_frac": float(kv["mfma_busy_frac"]),
                "cycles_per_launch": float(kv["cycles_per_launch"]) if "cycles_per_launch" in kv
                else None}
    except (OSError, KeyError, ValueError):
        return None


def environment(torch, dev):
    """Versions and device figures recorded with each result."""
    p = torch.cuda.get_device_properties(dev)
    env = {"device": p.name, "gcn_arch": getattr(p, "gcnArchName", None),
           "compute_units": p.multi_processor_count, "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None)}
    clk = getattr(p, "clock_rate", None)
    if clk:
        env["max_clock_mhz"] = round(clk / 1000.0)
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    return env


def host_cpu():
    """This host's CPU model, the cores this process may run on and the
    logical CPUs of the machine."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = os.cpu_count()
    return {"cpu_model": model, "cores": affinity, "logical_cpus": os.cpu_count()}


def cpu_baseline(host_layers):
    """The oracle (unchanged) on a bounded sample of the workload: the first
    layers (projection + all 8192 x 8 output rows each), timed on this host's
    cores.  numpy's elementwise steps run on one thread and its matrix
    products on the BLAS pool; ``cores`` is what the process may use, and
    ``blas_threads`` the pool's size."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    t0 = time.perf_counter()
    for layer in host_layers:
        bias = oracle.project_pair_bias(layer.pair, layer.weight)
        oracle.attention(layer.q, layer.k, layer.v, bias, scale=layer.scale, cap=layer.cap)
    dt = time.perf_counter() - t0
    L0 = host_layers[0]
    fl = attn_flops(L0.B, L0.S, Dv=L0.v.shape[-1]) * len(host_layers)
    hc = host_cpu()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": hc["cores"],
            "kind": "oracle", "cpu_model": hc["cpu_model"], "logical_cpus": hc["logical_cpus"],
            "blas_threads": blas, "wall_s": round(dt, 2),
            "sample": (f"{len(host_layers)} of the 9 layers (projection + all {L0.S} positions x "
                       f"8 heads each), float64 numpy, {dt:.1f} s wall; elementwise steps on one "
                       f"thread, matrix products on {blas} BLAS threads")}


class ClockSampler:
    """Reads the GPU's shader clock and power from sysfs (hwmon of the amdgpu
    device) every few milliseconds while a timed region runs, in a host
    thread that makes no GPU call.  Figures are None where the files are not
    readable."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.period = period_s
        self.freq, self.power = [], []
        self.cap_w = None
        self.files = {}
        for hw in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
            try:
                with open(os.path.join(hw, "name")) as f:
                    if f.read().strip() != "amdgpu":
                        continue
            except OSError:
                continue
            for key, name in (("freq", "freq1_input"), ("power", "power1_average"),
                              ("power_in", "power1_input"), ("cap", "power1_cap")):
                fn = os.path.join(hw, name)
                if os.access(fn, os.R_OK):
                    self.files.setdefault(key, fn)
            # without a clock input in hwmon: the device's shader clock
            # levels, the current one marked with '*'
            dpm = os.path.join(os.path.dirname(os.path.dirname(hw)), "pp_dpm_sclk")
            if "freq" not in self.files and os.access(dpm, os.R_OK):
                self.files["freq_dpm"] = dpm
            if self.files:
                break
        if "cap" in self.files:
            v = self._read("cap")
            self.cap_w = v / 1e6 if v is not None else None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, key):
        fn = self.files.get(key)
        if fn is None:
            return None
        try:
            with open(fn) as f:
                return float(f.read().strip())
        except (OSError, ValueError):
            return None

    def _read_dpm(self):
        fn = self.files.get("freq_dpm")
        if fn is None:
            return None
        try:
            with open(fn) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        mhz = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                        return float(mhz.replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            fq = self._read("freq")
            if fq is not None:
                self.freq.append(fq / 1e6)
            else:
                mhz = self._read_dpm()
                if mhz is not None:
                    self.freq.append(mhz)
            pw = self._read("power") if "power" in self.files else self._read("power_in")
            if pw is not None:
                self.power.append(pw / 1e6)
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        def med(x):
            return round(float(np.median(x)), 1) if x else None
        return {"sclk_mhz_median": med(self.freq), "sclk_samples": len(self.freq),
                "power_w_median": med(self.power), "power_cap_w": self.cap_w,
                "source": ("sysfs hwmon (amdgpu)" + (", clock from pp_dpm_sclk" if "freq_dpm" in self.files
                                                      else "") + ", sampled during the timed region")
                          if self.files else "not readable on this host"}


def attention_only(args, torch, dev, biased_mqa_fwd, workloads):
    """One attention kernel, B = 1, S = --seq-len, a random compact bias:
    K launches back to back between two events after the clock settles.
    Prints one JSON line (not the headline metric)."""
    dt, cap = args.attention_only.split(":")
    cap = float(cap)
    S = args.seq_len
    L = workloads.make_custom(B=1, S=S, dtype=dt, C=8, seed=S, qkv_std=1.0, bias_std=2.0)

    def g(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = g(L.q), g(L.k), g(L.v)
    P = -(-S // 16)
    bias = torch.randn(8, P, P, device=dev, generator=torch.Generator(device=dev).manual_seed(S))
    out = torch.empty_like(q)
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        biased_mqa_fwd(q, k, v, bias, out, softcap=cap)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        biased_mqa_fwd(q, k, v, bias, out, softcap=cap)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        biased_mqa_fwd(q, k, v, bias, out, softcap=cap)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    fl = attn_flops(1, S)
    tf = fl / (us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_FP32_MATRIX_TFLOPS
    kernel = ("biased_mqa_fwd_kernel (generic, float32)" if dt != "bf16" else
              "biased_mqa_fwd_bf16_capped_kernel" if cap > 0 else "biased_mqa_fwd_bf16_uncapped_kernel")
    log(f"attention only, {dt}, cap {cap:g}, S={S}: {us:.1f} us per launch = {tf:.1f} TFLOP/s")
    print(json.dumps({"metric": f"attention kernel TFLOP/s, {dt}, cap {cap:g}, S={S}, 8 heads, "
                                f"d=128", "value": round(tf, 2), "unit": "TFLOP/s",
                      "avg_launch_us": round(us, 2), "steps": args.steps,
                      "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak,
                                   "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                                   "kernel": kernel, "flops_per_launch": fl}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers per step (default 9 for full, mid and shard; 1 for variant and "
                         "stress, whose step is one call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=3,
                    help="layers in the oracle's timed sample (about 4-5 s each on 16 cores)")
    ap.add_argument("--dv", type=int, default=128, choices=(128, 192),
                    help="value width (192 is the released checkpoint's; the headline "
                         "workload uses 128)")
    ap.add_argument("--workload", default="full",
                    choices=("full", "mid", "shard", "variant", "stress"),
                    help="full: the full-context layers (the headline); mid: S=2048 layers; "
                         "shard: one GPU's share of a full-context layer under sequence "
                         "parallelism over 8 GPUs (1024 query positions at offset 3072, all "
                         "8192 keys); variant: one call on 8 items of S=8192 (4 ref/alt pairs, "
                         "one pair representation per pair); stress: one call at S=16384")
    ap.add_argument("--kv-splits", default=None,
                    help="key ranges per attention call (an integer or 'auto'; default: 1 for "
                         "full, auto otherwise)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before each route's warmup steps, run untimed steps for this long: "
                         "the clock takes tens of ms of sustained load to settle, and a route "
                         "timed while it still moves reads up to 30%% slow")
    ap.add_argument("--path", default=None, choices=("pair", "two"),
                    help="pair (default): the projection inside the attention kernel; two: "
                         "projection kernel + attention kernel")
    ap.add_argument("--attention-only", default=None,
                    choices=("bf16:5", "bf16:0", "f32:5", "f32:0"),
                    help="instead of the headline step, time the attention kernel alone for "
                         "this dtype and cap (0 = uncapped: the generic kernel) on one layer "
                         "of --seq-len positions, against the matching matrix-core peak")
    ap.add_argument("--seq-len", type=int, default=8192,
                    help="sequence length for --attention-only")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the measurement, run 3 plain device-to-device copies of this "
                         "many MiB (a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    path = args.path or "pair"

    import torch
    from long_context_biased_amd import (biased_mqa_fwd, pair_bias_project, pair_biased_mqa_fwd,
                                         workloads)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wl = args.workload
    n_layers = args.layers if args.layers is not None else (
        1 if wl in ("variant", "stress") else 9)
    if args.attention_only:
        attention_only(args, torch, dev, biased_mqa_fwd, workloads)
        return

    def to_gpu(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    from long_context_biased_amd import auto_kv_splits, workspace_bytes
    if wl != "full":
        args.no_cpu_baseline = True
    t0 = time.perf_counter()
    layers, host = [], []
    for li in range(n_layers):
        L = workloads.make_layer({"mid": "mid", "variant": "variant", "stress": "stress"}.get(
            wl, "full"), layer=li, Dv=args.dv)
        if li < max(1, args.cpu_layers):
            host.append(L)
        t = {n: to_gpu(getattr(L, n)) for n in ("q", "k", "v", "pair", "weight")}
        P = -(-L.S // 16)
        q_off, Sq = (3072, 1024) if wl == "shard" else (0, L.S)
        t["q"] = t["q"][:, q_off:q_off + Sq].contiguous()
        n_pairs = L.pair.shape[0]
        t["group"] = L.bias_group
        t["bias"] = torch.empty((n_pairs, 8, P, P), dtype=torch.float32, device=dev)
        t["out"] = torch.empty((L.B, Sq, 8, args.dv), dtype=t["q"].dtype, device=dev)
        ks = args.kv_splits if args.kv_splits is not None else ("1" if wl == "full" else "auto")
        z = auto_kv_splits(L.B, Sq, L.S) if ks == "auto" else int(ks)
        t["z"], t["q_off"], t["Sq"] = z, q_off, Sq
        nws = workspace_bytes(L.B, Sq, 8, args.dv, z)
        t["ws"] = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev) if nws > 0 else None
        layers.append(t)
    torch.cuda.synchronize()
    log(f"inputs: {n_layers} layers generated and uploaded in {time.perf_counter() - t0:.1f} s")
    host0 = host[0]
    S = host0.S
    Bw = host0.B
    n_pairs = host0.pair.shape[0]
    P = -(-S // 16)
    scale = host0.scale
    cap = host0.cap

    stream = torch.cuda.current_stream(dev)

    def step_two(events=None):
        for li, t in enumerate(layers):
            if events is not None:
                events[li][0].record(stream)
            pair_bias_project(t["pair"], t["weight"], out=t["bias"])
            if events is not None:
                events[li][1].record(stream)
            biased_mqa_fwd(t["q"], t["k"], t["v"], t["bias"], out=t["out"], scale=scale,
                           softcap=cap, bias_group=t["group"], q_offset=t["q_off"],
                           kv_splits=t["z"], workspace=t["ws"])
            if events is not None:
                events[li][2].record(stream)

    def step_pair(events=None):
        for li, t in enumerate(layers):
            if events is not None:
                events[li][0].record(stream)
            pair_biased_mqa_fwd(t["q"], t["k"], t["v"], t["pair"], t["weight"], out=t["out"],
                                scale=scale, softcap=cap, pair_group=t["group"],
                                q_offset=t["q_off"], kv_splits=t["z"], workspace=t["ws"])
            if events is not None:
                events[li][1].record(stream)
                events[li][2].record(stream)

    clocks = {}

    def measure(step):
        """ms per step over K timed steps (after W warmups), then per-kernel
        averages from the same steps run again with events around each
        launch: (ms_per_step, first-kernel ms list, second-kernel ms list)."""
        with ClockSampler() as clk:  # the clock and power under this load
            t_end = time.perf_counter() + args.settle_ms * 1e-3
            while time.perf_counter() < t_end:  # clock settle, untimed
                step()
                torch.cuda.synchronize()
            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            # Timed region: K steps between two events, no per-kernel events inside.
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(args.steps):
                step()
            end.record(stream)
            torch.cuda.synchronize()
        clocks[step.__name__] = clk.summary()
        ms = start.elapsed_time(end) / args.steps
        ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_layers)]
              for _ in range(args.steps)]
        for st in range(args.steps):
            step(ev[st])
        torch.cuda.synchronize()
        k1 = [e[0].elapsed_time(e[1]) for st in ev for e in st]
        k2 = [e[1].elapsed_time(e[2]) for st in ev for e in st]
        return ms, k1, k2

    Sq = layers[0]["Sq"]
    fl_layer = attn_flops(Bw, S, Dv=args.dv, Sq=Sq)
    pb = proj_bytes(P, 128) * n_pairs
    pf = proj_flops(P, 128) * n_pairs
    if path == "pair":
        ms_per_step, fused_ms, _ = measure(step_pair)
        kern_ms = fused_ms
        kern_fl = fl_layer + pf  # the kernel also projects the bias cells it uses
        ms_two, proj_ms, attn_ms = measure(step_two)
    else:
        ms_per_step, proj_ms, attn_ms = measure(step_two)
        kern_ms = attn_ms
        kern_fl = fl_layer
        ms_pair = measure(step_pair)[0]
    # The pair form is the only kernel of its step, so its average launch
    # time is the timed region itself over its launches (no per-kernel
    # events inside it; events around every launch add their own gap).  In
    # the two-kernel route the attention shares the step with the projection,
    # so its average comes from the event-bracketed steps.
    kern_event_avg = float(np.mean(kern_ms))
    kern_avg = ms_per_step / n_layers if path == "pair" else kern_event_avg
    attn_avg = float(np.mean(attn_ms))
    proj_interval = float(np.mean(proj_ms))

    # The projection kernel on its own, launches back to back over the
    # layers (their pair representations, 64 MiB each, do not fit the
    # last-level cache together): its per-launch time without the event
    # and launch gaps that separate it from the attention kernel in the
    # two-kernel route.
    for _ in range(args.warmup):
        for t in layers:
            pair_bias_project(t["pair"], t["weight"], out=t["bias"])
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(args.steps):
        for t in layers:
            pair_bias_project(t["pair"], t["weight"], out=t["bias"])
    p1.record(stream)
    torch.cuda.synchronize()
    proj_avg = p0.elapsed_time(p1) / (args.steps * n_layers)

    # The attainable rate beside it: a plain device-to-device copy that moves
    # as many bytes per launch (half read, half written), back to back over
    # as many distinct buffers as there are layers.
    half = pb // 2
    csrc = [torch.ones(half, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    cdst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(n_layers)]
    for _ in range(args.warmup):
        for a, b in zip(csrc, cdst):
            b.copy_(a)
    torch.cuda.synchronize()
    p0.record(stream)
    for _ in range(args.steps):
        for a, b in zip(csrc, cdst):
            b.copy_(a)
    p1.record(stream)
    torch.cuda.synchronize()
    copy_avg = p0.elapsed_time(p1) / (args.steps * n_layers)
    del csrc, cdst

    value = n_layers * fl_layer / (ms_per_step * 1e-3) / 1e12
    achieved = kern_fl / (kern_avg * 1e-3) / 1e12
    counters = load_counters(path) if (args.dv == 128 and wl == "full") else None
    log(f"{path}: step {ms_per_step:.3f} ms; kernel avg {kern_avg * 1e3:.1f} us "
        f"(event-bracketed: avg {kern_event_avg * 1e3:.1f}, median "
        f"{np.median(kern_ms) * 1e3:.1f}, p95 {np.percentile(kern_ms, 95) * 1e3:.1f}) "
        f"= {achieved:.1f} TFLOP/s")
    log(f"two kernels: attention avg {attn_avg * 1e3:.1f} us, projection interval "
        f"{proj_interval * 1e3:.1f} us; projection alone {proj_avg * 1e3:.1f} us = "
        f"{pb / (proj_avg * 1e-3) / 1e9:.0f} GB/s; a copy of as many bytes {copy_avg * 1e3:.1f} us")

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {args.copy_mib} MiB")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {len(host)} layer(s) ...")
        cpu = cpu_baseline(host[:max(1, args.cpu_layers)])
        log(f"cpu baseline: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    rec = {
        "metric": ("biased-MQA fwd TFLOP/s at S=8192, H=8, d=128 bf16; % MFMA peak"
                   if (args.dv == 128 and wl == "full") else
                   f"biased-MQA fwd TFLOP/s at B={Bw}, S={S}, Sq={Sq}, H=8, dk=128, dv={args.dv} "
                   f"bf16; % MFMA peak"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(128) q,k,v; N(0,1) pair rep; W var 1/128)",
        "config": {"workload": {"full": "full-context: 9 independent layers, each pair-bias "
                                        "projection + biased soft-capped MQA fwd",
                                "mid": "mid: independent S=2048 layers, each pair-bias projection "
                                       "+ biased soft-capped MQA fwd",
                                "shard": "one GPU's share of full-context layers (queries "
                                         "3072..4095 of 8192, all keys; full projection)",
                                "variant": "variant batch: one call on 8 items of S=8192, 4 "
                                           "ref/alt pairs (alt = ref + noise on rows "
                                           "4090..4101), one pair representation per pair",
                                "stress": "stress: one call at S=16384 (P=1024), pair-bias "
                                          "projection + biased soft-capped MQA fwd"}[wl],
                   "route": {"pair": "pair form: projection inside the attention kernel",
                             "two": "projection kernel + attention kernel"}[path],
                   "B": Bw, "S": S, "Sq": Sq, "kv_splits": layers[0]["z"], "P": P, "q_heads": 8,
                   "kv_heads": 1, "d": 128, "dv": args.dv,
                   "pair_channels": 128, "layers": n_layers, "softcap": cap,
                   "global_batch": Bw, "seq_len": S, "parallelism": "none (1 GPU)"},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counters["hbm_bytes_per_launch"] if counters else None,
                     "mfma_flops_counter": counters["mfma_flops_per_launch"] if counters else None,
                     "mfma_busy_frac_counter": counters["mfma_busy_frac"] if counters else None,
                     # GPU cycles per launch from the counters (GRBM_GUI_ACTIVE per XCD) and
                     # the clock they imply with this run's launch time: the frac on any box
                     # is flops * clock / (cycles * peak)
                     "cycles_per_launch_counter": counters.get("cycles_per_launch")
                     if counters else None,
                     "implied_clock_mhz": round(counters["cycles_per_launch"] / (kern_avg * 1e3), 1)
                     if counters and counters.get("cycles_per_launch") else None,
                     "kernel": "biased_mqa_fwd_bf16_capped_kernel" +
                               (" (pair form)" if path == "pair" else ""),
                     "flops_per_launch": kern_fl,
                     "avg_launch_us": round(kern_avg * 1e3, 2),
                     "avg_launch_from": ("timed region / launches" if path == "pair" else
                                         "event-bracketed steps"),
                     "event_avg_launch_us": round(kern_event_avg * 1e3, 2),
                     "median_launch_us": round(float(np.median(kern_ms)) * 1e3, 2),
                     "p95_launch_us": round(float(np.percentile(kern_ms, 95)) * 1e3, 2)},
        "other_route": ({"route": "projection kernel + attention kernel",
                         "ms_per_step": round(ms_two, 4),
                         "attention_avg_launch_us": round(attn_avg * 1e3, 2)}
                        if path == "pair" else
                        {"route": "pair form", "ms_per_step": round(ms_pair, 4)}
                        if ms_pair is not None else None),
        "projection": {"bound": "hbm", "route": "projection kernel of the two-kernel route, "
                                                "timed back to back over the layers",
                       "avg_launch_us": round(proj_avg * 1e3, 2),
                       "in_route_interval_us": round(proj_interval * 1e3, 2),
                       "bytes_per_launch": pb,
                       "achieved_GBs": round(pb / (proj_avg * 1e-3) / 1e9, 1),
                       "peak_GBs": PEAK_HBM_GBS,
                       "frac": round(pb / (proj_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "copy_same_bytes": {"avg_launch_us": round(copy_avg * 1e3, 2),
                                           "achieved_GBs": round(2 * half / (copy_avg * 1e-3) / 1e9, 1)},
                       "frac_of_copy": round(copy_avg / proj_avg, 4)},
        "cpu_baseline": cpu,
        "env": {**environment(torch, dev), "host": host_cpu(),
                "gpu_clock_power": clocks.get("step_pair" if path == "pair" else "step_two")},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
