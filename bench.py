"""Benchmark of the routed MoE layer on one MI355X.

Default workload: the pages' per-device prefill share (2048 tokens, hidden
8192, intermediate 2048, 8 local experts, top-2, per-channel fp8 weights,
plus the shared expert 8192 -> 2048 -> 8192 on every token).  One step is one
moe_forward (route, quantise + permute, gate-up GEMM with SiLU*gate, down
GEMM, combine) on resident device inputs.  Weight sets are rotated across steps
(--copies, default 3) so that the 256 MB last-level cache cannot hold them.

Prints ONE JSON line: metric / value (fp8 TFLOP/s of the whole layer,
6*H*I flops per routed row and per shared-expert token), the roofline of the
dominant kernel (the down GEMM, the layer's longest; the gate-up GEMM's
beside it), each timed by events its own dispatch stamps, the decode-share
weight-stream rate, and the CPU oracle timed on a bounded sample (reported
baseline only).

`roofline.traffic` (HBM bytes per launch) comes from the FETCH_SIZE /
WRITE_SIZE counter summary under profiles/; it is reported only while the
kernel sources still hash to the value recorded there, and is null
otherwise.  `--copy-kernel MIB` runs only a plain device copy of that
size (the counters' calibration) and exits.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
LAYER_METRIC = "MoE layer µs & fp8 TFLOP/s (% MFMA peak); decode weight-stream GB/s (% HBM)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="prefill")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-share measurement")
    ap.add_argument("--no-latent", action="store_true", help="skip the LatentMoE block measurement")
    ap.add_argument("--no-block", action="store_true", help="skip the per-block fp8 measurement")
    ap.add_argument("--no-block-decode", action="store_true",
                    help="per-block fp8: time the prefill share only (for kernel traces of one workload)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill (headline) measurement: for profiling the other workloads alone")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny (launch-latency) workload")
    ap.add_argument("--no-skewed", action="store_true", help="skip the skewed 256-expert whole layer")
    ap.add_argument("--no-latent-core", action="store_true", help="skip the LatentMoE expert core alone")
    ap.add_argument("--no-sclk", action="store_true", help="skip sampling the shader clock under load")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens in the CPU oracle's sample (FFN + combine of each)")
    ap.add_argument("--copy-kernel", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_layer_prefill_hbm_traffic.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_layer_decode_hbm_traffic.txt")
LATENT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "latent_block_hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_ffn_softmax_amd", "csrc", f)
                  for f in ("gemm.hip", "device_common.h", "internal.h")]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(which, path=TRAFFIC_FILE):
    """HBM bytes per launch of GEMM `which` ("gemm1" / "gemm2") from the
    committed counter summary `path`, or None when the summary is absent or
    the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields[f"{which}_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_kernel(mib):
    """A plain elementwise device copy (negation) of `mib` MiB, five times:
    reads and writes exactly mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy kernel: 5 launches of {mib} MiB read + {mib} MiB written")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Device inputs of one workload with `copies` weight sets and a workspace."""

    def __init__(self, name, copies):
        import torch

        import mixture_experts_ffn_softmax_amd as moe
        import moe_synth

        self.inp = moe_synth.make_inputs(name, device="cuda")
        c = self.cfg = self.inp["cfg"]
        self.T, self.H, self.I, self.E, self.k = c["T"], c["H"], c["I"], c["E"], c["k"]
        sets = [self.inp["routed"]] + [{n: t.clone() for n, t in self.inp["routed"].items()}
                                       for _ in range(copies - 1)]
        self.routed = [moe.Weights(s, c["fmt"]) for s in sets]
        self.shared = None
        if self.inp["shared"] is not None:
            sh = [self.inp["shared"]] + [{n: t.clone() for n, t in self.inp["shared"].items()}
                                         for _ in range(copies - 1)]
            self.shared = [moe.Weights(s, "fp8") for s in sh]
        self.out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device="cuda")
        nbytes = moe.forward_workspace_size(self.T, self.k, self.routed[0], self.shared is not None)
        self.ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
        self.moe = moe

    def step(self, i, events=None, gemm_events=None, layer_events=None):
        j = i % len(self.routed)
        g = gemm_events or (None, None)
        self.moe.moe_forward(self.inp["x"], self.inp["logits"], self.k, self.routed[j],
                             None if self.shared is None else self.shared[j], self.inp["gamma"],
                             self.inp["eps"], out=self.out, ws=self.ws, events=events,
                             gemm1_events=g[0], gemm2_events=g[1], layer_events=layer_events)

    def flops(self):
        rows = self.T * self.k + (self.T if self.shared is not None else 0)
        return 6.0 * self.H * self.I * rows, 4.0 * self.H * self.I * rows

    def weight_bytes_touched(self):
        import torch

        import moe_synth
        ids = torch.topk(self.inp["logits"], self.k, dim=1).indices
        touched = int(torch.unique(ids).numel())
        per = moe_synth.weight_bytes_per_expert(self.H, self.I, self.cfg["fmt"])
        scales = {"fp8": 4 * (2 * self.I + self.H),
                  "fp8_block": 4 * 3 * (self.H // 128) * (self.I // 128)}.get(self.cfg["fmt"], 0)
        # (MXFP4: the per-expert figure already holds the e8m0 scales)
        total = touched * (per + scales)
        if self.shared is not None:
            total += 3 * self.H * self.I + 4 * (2 * self.I + self.H)
        io = self.T * self.H * 2 * 2 + self.T * self.E * 4
        return total, io, touched

    def gemm_bytes(self):
        """Algorithmic HBM bytes of one gate-up and one down GEMM launch:
        the touched experts' weights (and scales) read once, the quantised
        token rows read once, h written and read once (bf16), the fp32
        expert output rows written once."""
        total, _, touched = self.weight_bytes_touched()
        if self.cfg["fmt"] != "fp8":
            return None, None
        rows = self.T * self.k + (self.T if self.shared is not None else 0)
        experts = touched + (1 if self.shared is not None else 0)
        w13 = experts * (2 * self.H * self.I + 4 * 2 * self.I)
        w2 = experts * (self.H * self.I + 4 * self.H)
        g1 = w13 + self.T * (self.H + 4) + rows * self.I * 2
        g2 = w2 + rows * self.I * 2 + rows * self.H * 4
        return g1, g2


class LatentBlock:
    """The LatentMoE block (hidden 7168 -> latent 3584 -> 896 MXFP4 experts
    top-16 + RMSNorm -> 7168, bf16 shared experts 7168 -> 6144 -> 7168) on
    512 tokens.  Its 15.7 GB of expert weights are far beyond the last-level
    cache, so one weight copy suffices."""

    def __init__(self):
        import torch

        import mixture_experts_ffn_softmax_amd as moe
        import moe_synth
        self.moe = moe
        self.blk = b = moe_synth.latent_block_inputs(**moe_synth.LATENT_BLOCK, device="cuda")
        c = self.cfg = b["cfg"]
        self.lw = moe.LatentWeights(b["down"], b["up"], b["shared"])
        self.routed = moe.Weights(b["routed"], "mxfp4")
        self.out = torch.empty((c["T"], c["Hm"]), dtype=torch.bfloat16, device="cuda")
        n = moe.latent_forward_workspace_size(c["T"], c["k"], self.lw, self.routed)
        self.ws = torch.empty((n,), dtype=torch.uint8, device="cuda")

    def step(self, i, events=None, gemm_events=None, layer_events=None):
        b, c = self.blk, self.cfg
        g = gemm_events or (None, None)
        self.moe.moe_latent_forward(b["x"], b["logits"], c["k"], self.lw, self.routed, b["gamma"], b["eps"],
                                    out=self.out, ws=self.ws, layer_events=layer_events, gemm1_events=g[0],
                                    gemm2_events=g[1])

    def accounting(self):
        """(algorithmic bytes, flops, routed gate-up weight bytes) of one block."""
        import torch

        import moe_synth
        c = self.cfg
        T, Hm, L, I, E, k, Is = (c[n] for n in ("T", "Hm", "L", "I", "E", "k", "Is"))
        touched = int(torch.unique(torch.topk(self.blk["logits"], k, dim=1).indices).numel())
        expert = moe_synth.weight_bytes_per_expert(L, I, "mxfp4")
        proj = 2 * (Hm * L // 2 + Hm * L // 32)
        shared = 3 * Hm * Is * 2
        io = T * Hm * 2 * 2 + T * E * 4
        flops = 6.0 * L * I * T * k + 4.0 * T * Hm * L + 6.0 * T * Hm * Is
        gate_up = touched * 2 * (L * I // 2 + L * I // 32)
        return touched * expert + proj + shared + io, flops, gate_up, touched


def dense_rates(block, reps=20):
    """Standalone TFLOP/s of the block's projections and of the shared
    experts' down GEMM (moe_linear, back-to-back launches between two events)."""
    import torch
    moe, b, c = block.moe, block.blk, block.cfg
    T = c["T"]
    cases = {"down_proj_mxfp4": (b["x"], block.lw.down),
             "up_proj_mxfp4": (torch.zeros((T, c["L"]), dtype=torch.bfloat16, device="cuda"), block.lw.up),
             "shared_down_bf16": (torch.zeros((T, c["Is"]), dtype=torch.bfloat16, device="cuda"),
                                  moe.Linear(b["shared"]["w2"]))}
    res = {}
    for name, (a, w) in cases.items():
        out = torch.empty((T, w.c.n_out), dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            moe.moe_linear(a, w, out=out)
        ev = make_events(2)
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            moe.moe_linear(a, w, out=out)
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / reps * 1e3
        flops = 2.0 * T * w.c.n_out * w.c.n_in
        res[name] = {"us": round(us, 2), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                     "frac_bf16_peak": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return res


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def sample_sclk(layer, seconds=3.0):
    """The shader clock while the layer runs back to back: rocm-smi (a child
    process) reads the clocks once the GPU has been busy for a second.
    Returns the reported SCLK string, or None."""
    import subprocess
    import threading

    import torch
    box = {}

    def probe():
        time.sleep(1.0)
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
            box["out"] = r.stdout
        except Exception as e:  # noqa: BLE001 (best effort: the tool may be absent)
            box["err"] = str(e)

    th = threading.Thread(target=probe)
    th.start()
    t0, i = time.perf_counter(), 0
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        layer.step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > 30:
                break
    torch.cuda.synchronize()
    th.join()
    try:
        data = json.loads(box.get("out", ""))
        for card in data.values():
            for key, val in card.items():
                if "sclk" in key.lower():
                    return str(val)
    except ValueError:
        pass
    return None


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()          # creates the underlying HIP event
    return evs


def time_layer(layer, steps, warmup):
    """Times `steps` steps after `warmup` untimed ones.  Returns a dict: ms per
    step by the host clock between synchronisations (`ms`) and by GPU events
    around the whole region (`gpu_ms`), both over plain steps with nothing
    stamped inside the layers; then, in passes of their own over the same
    steps, the per-layer durations (`layer_ms`, a list) from the start/stop
    events the layer's own first and last dispatches stamp, and the average
    GEMM1 / GEMM2 launch ms (`g1_ms`, `g2_ms`) from the events their
    dispatches stamp.  A dispatch that stamps an event runs a few
    microseconds longer (about 8 us per decode layer), so no stamped pass is
    the timed one, and no layer carries two kinds of event."""
    import torch
    for i in range(warmup):
        layer.step(i)
    torch.cuda.synchronize()
    ge = [(make_events(2), make_events(2), make_events(2)) for _ in range(steps)]
    region = make_events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record()
    for i in range(steps):
        layer.step(i)
    region[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        layer.step(i, layer_events=ge[i][2])
    torch.cuda.synchronize()
    for i in range(steps):
        layer.step(i, gemm_events=ge[i][:2])
    torch.cuda.synchronize()
    return dict(ms=(t1 - t0) * 1e3 / steps, gpu_ms=region[0].elapsed_time(region[1]) / steps,
                layer_ms=[c[0].elapsed_time(c[1]) for _, _, c in ge],
                g1_ms=sum(a.elapsed_time(b) for (a, b), _, _ in ge) / steps,
                g2_ms=sum(a.elapsed_time(b) for _, (a, b), _ in ge) / steps)


def percentiles_us(ms_list):
    """Median, p10 and p90 of per-layer durations, in microseconds."""
    import numpy as np
    a = np.asarray(ms_list) * 1e3
    return {"median": round(float(np.median(a)), 1), "p10": round(float(np.percentile(a, 10)), 1),
            "p90": round(float(np.percentile(a, 90)), 1)}


def stage_times(layer, steps):
    """Per-stage averages from events recorded at the stage boundaries, in a
    separate untimed pass (each record adds a few microseconds of its own)."""
    import torch

    from mixture_experts_ffn_softmax_amd import MOE_N_STAGES, STAGE_NAMES
    evs = [make_events(MOE_N_STAGES + 1) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        layer.step(i, events=evs[i])
    torch.cuda.synchronize()
    stage = {n: 0.0 for n in STAGE_NAMES}
    for e in evs:
        for s, n in enumerate(STAGE_NAMES):
            stage[n] += e[s].elapsed_time(e[s + 1]) / steps
    return stage


def cpu_baseline(layer, n_tokens, min_seconds=10.0):
    """The oracle, as it stands, on a bounded sample: routing of all tokens
    plus quantise / FFN / combine of n_tokens sampled tokens, repeated until
    at least min_seconds of host time have been spent."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from oracle.moe import ExpertWeights

    def host(d):
        return None if d is None else ExpertWeights(
            layer.cfg["fmt"] if d is layer.inp["routed"] else "fp8",
            *(d[n].cpu().numpy() for n in ("w1", "w3", "w2", "s1", "s3", "s2")))

    x = layer.inp["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    logits = layer.inp["logits"].cpu().numpy()
    Wr, Ws = host(layer.inp["routed"]), host(layer.inp["shared"])
    n_tokens = min(n_tokens, layer.T)
    tokens = np.sort(np.random.default_rng(0).choice(layer.T, n_tokens, replace=False))
    gamma = None if layer.inp["gamma"] is None else layer.inp["gamma"].cpu().numpy()
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.moe.forward_sampled(x, logits, layer.k, Wr, tokens, shared=Ws, norm_gamma=gamma,
                                   norm_eps=layer.inp["eps"])
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    rows = n_tokens * layer.k + (n_tokens if Ws is not None else 0)
    flops = 6.0 * layer.H * layer.I * rows * passes
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{passes} passes of: routing of all {layer.T} tokens + quantise/permute/FFN/combine "
                       f"of {n_tokens} sampled tokens (float64 NumPy); {dt:.1f} s wall in total")


def measure_prefill(args):
    """The headline line: the prefill share's layer, its rooflines and stages."""
    import torch
    log(f"[bench] workload {args.config}: generating inputs ({args.copies} weight copies)")
    layer = Layer(args.config, args.copies)
    c = layer.cfg
    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up")
    tl = time_layer(layer, args.steps, args.warmup)
    ms, gpu_ms, g1_ms, g2_ms = tl["ms"], tl["gpu_ms"], tl["g1_ms"], tl["g2_ms"]
    stage = stage_times(layer, min(args.steps, 20))
    flops, flops_g1 = layer.flops()
    flops_g2 = flops - flops_g1
    value = flops / (ms * 1e-3) / 1e12
    achieved_g1 = flops_g1 / (g1_ms * 1e-3) / 1e12
    achieved_g2 = flops_g2 / (g2_ms * 1e-3) / 1e12
    wbytes, io, touched = layer.weight_bytes_touched()
    log(f"[bench] {ms * 1e3:.1f} us/layer ({gpu_ms * 1e3:.1f} by GPU events), {value:.1f} TFLOP/s; "
        f"gemm1 {g1_ms * 1e3:.1f} us, gemm2 {g2_ms * 1e3:.1f} us; stages with events (us): "
        + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in stage.items()))
    result = {
        "metric": LAYER_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "us_per_layer": round(ms * 1e3, 1),
        "us_per_layer_gpu_events": round(gpu_ms * 1e3, 1),
        "us_per_layer_dispatch_events": percentiles_us(tl["layer_ms"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x e4m3 (gate-up) and bf16 x bf16 (down) MFMA, fp32 accumulate",
        "data": "synthetic (seeded; shapes of the pages' per-device prefill share)",
        "config": {"workload": f"{args.config}: T={c['T']} H={c['H']} I={c['I']} E={c['E']} top_k={c['k']} "
                               f"{c['fmt']}{' +shared expert' if c['shared'] else ''}",
                   "tokens": c["T"], "routed_rows": c["T"] * c["k"], "weight_copies": args.copies,
                   "flops_per_step": flops, "touched_experts": touched},
        "stage_us_with_events": {n: round(v * 1e3, 2) for n, v in stage.items()},
        "frac_fp8_peak_layer": round(value / PEAK_FP8_TFLOPS, 4),
        "roofline": {"kernel": "gemm2 (down grouped GEMM, bf16 h x W2 widened to bf16): the layer's longest kernel",
                     "bound": "mfma", "achieved": round(achieved_g2, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_g2 / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("gemm2"), "flops_per_launch": flops_g2,
                     "avg_launch_us": round(g2_ms * 1e3, 2)},
        "roofline_gemm1": {"kernel": "gemm1 (gate-up grouped GEMM + SiLU*gate, fp8)", "bound": "mfma",
                           "achieved": round(achieved_g1, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved_g1 / PEAK_FP8_TFLOPS, 4), "traffic": measured_traffic("gemm1"),
                           "flops_per_launch": flops_g1, "avg_launch_us": round(g1_ms * 1e3, 2)},
    }
    del layer
    return result


def measure_small(name, steps, warmup):
    """The tiny workload: launch-latency bound, so only microseconds."""
    import torch
    layer = Layer(name, 1)
    c = layer.cfg
    tl = time_layer(layer, steps, warmup)
    res = {"workload": f"{name}: T={c['T']} H={c['H']} I={c['I']} E={c['E']} top_k={c['k']} {c['fmt']}",
           "us_per_layer": round(tl["ms"] * 1e3, 2), "us_per_layer_gpu_events": round(tl["gpu_ms"] * 1e3, 2),
           "us_per_layer_dispatch_events": percentiles_us(tl["layer_ms"]),
           "gemm_us": {"gemm1": round(tl["g1_ms"] * 1e3, 2), "gemm2": round(tl["g2_ms"] * 1e3, 2)},
           "bound": "launch latency (fractions of a roofline are not meaningful at this size)"}
    del layer
    torch.cuda.empty_cache()
    return res


def measure_skewed(steps, warmup):
    """The skewed whole layer (16384 tokens, 256 experts, top-8, Zipf-biased
    router, hottest expert ~5x the mean): fp8 MFMA bound."""
    import torch
    layer = Layer("skewed", 1)
    c = layer.cfg
    tl = time_layer(layer, steps, warmup)
    flops, flops_g1 = layer.flops()
    wb, io, touched = layer.weight_bytes_touched()
    ms = tl["ms"]
    ids = torch.topk(layer.inp["logits"], layer.k, dim=1).indices
    counts = torch.bincount(ids.flatten(), minlength=layer.E).float()
    g1, g2 = tl["g1_ms"], tl["g2_ms"]
    res = {"workload": f"skewed: T={c['T']} H={c['H']} I={c['I']} E={c['E']} top_k={c['k']} fp8, "
                       f"Zipf-biased router (alpha {c['alpha']:.4f})",
           "us_per_layer": round(ms * 1e3, 1), "us_per_layer_gpu_events": round(tl["gpu_ms"] * 1e3, 1),
           "us_per_layer_dispatch_events": percentiles_us(tl["layer_ms"]),
           "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_fp8_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
           "GB_per_s": round((wb + io) / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round((wb + io) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "algorithmic_bytes": wb + io, "flops_per_layer": flops, "touched_experts": touched,
           "alpha": c["alpha"], "hottest_over_mean": round(float(counts.max() / counts.mean()), 3),
           "gemm_us": {"gemm1": round(g1 * 1e3, 1), "gemm2": round(g2 * 1e3, 1)},
           "gemm_frac": {"gemm1_fp8": round(flops_g1 / (g1 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                         "gemm2_bf16": round((flops - flops_g1) / (g2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}}
    del layer
    torch.cuda.empty_cache()
    return res


def measure_latent_core(steps, warmup):
    """The LatentMoE expert core alone (512 tokens of latent 3584, 896 MXFP4
    experts 3584 -> 3072 -> 3584, top-16, RMSNorm): HBM bound on the touched
    experts' weights."""
    import torch
    layer = Layer("latent", 1)
    c = layer.cfg
    tl = time_layer(layer, steps, warmup)
    flops, _ = layer.flops()
    wb, io, touched = layer.weight_bytes_touched()
    ms = tl["ms"]
    # the routed gate-up GEMM streams the touched experts' W1 and W3 (codes and scales) once
    gate_up = touched * 2 * (c["H"] * c["I"] // 2 + c["H"] * c["I"] // 32)
    g1_us = tl["g1_ms"] * 1e3
    res = {"workload": f"latent core: T={c['T']} H={c['H']} I={c['I']} E={c['E']} top_k={c['k']} mxfp4 +RMSNorm",
           "us_per_layer": round(ms * 1e3, 1), "us_per_layer_gpu_events": round(tl["gpu_ms"] * 1e3, 1),
           "us_per_layer_dispatch_events": percentiles_us(tl["layer_ms"]),
           "GB_per_s": round((wb + io) / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round((wb + io) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
           "algorithmic_bytes": wb + io, "touched_experts": touched,
           "gemm_us": {"gemm1": round(tl["g1_ms"] * 1e3, 1), "gemm2": round(tl["g2_ms"] * 1e3, 1)},
           "roofline": {"kernel": "routed gate-up GEMM (MXFP4 weights streamed once)", "bound": "hbm",
                        "achieved": round(gate_up / (g1_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gate_up / (g1_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic("gemm1", LATENT_TRAFFIC_FILE), "avg_launch_us": round(g1_us, 2),
                        "bytes_per_launch": gate_up}}
    del layer
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the layer is "
              "measured on one device's share (the expert-parallel path across GPUs is not "
              "implemented).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_kernel:
        copy_kernel(args.copy_kernel)
        return

    result = {"metric": LAYER_METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": True}
    if not args.no_prefill:
        result = measure_prefill(args)
        torch.cuda.empty_cache()
    result["rocm_version"] = rocm_version()
    result["torch_hip"] = torch.version.hip
    if not args.no_sclk and not args.no_prefill:
        log("[bench] shader clock under load (rocm-smi while the prefill layer runs)")
        sl = Layer(args.config, 1)
        result["sclk_under_load"] = sample_sclk(sl)
        del sl
        torch.cuda.empty_cache()

    if not args.no_tiny:
        log("[bench] tiny workload (launch latency)")
        result["tiny"] = measure_small("tiny", max(args.steps, 200), args.warmup)

    if not args.no_skewed:
        log("[bench] skewed whole layer (16384 tokens, 256 experts top-8)")
        result["skewed"] = measure_skewed(min(args.steps, 20), min(args.warmup, 3))

    if not args.no_latent_core:
        log("[bench] LatentMoE expert core alone (512 tokens, 896 MXFP4 experts top-16, RMSNorm)")
        result["latent_core"] = measure_latent_core(min(args.steps, 20), min(args.warmup, 3))

    if not args.no_decode:
        log("[bench] decode share (weight-stream bound)")
        dl = Layer("decode", args.copies)
        dtl = time_layer(dl, max(args.steps, 50), args.warmup)
        dms, dgpu_ms = dtl["ms"], dtl["gpu_ms"]
        dstage = stage_times(dl, 20)
        dbytes, dio, dtouched = dl.weight_bytes_touched()
        gbs = (dbytes + dio) / (dms * 1e-3) / 1e9
        g1b, g2b = dl.gemm_bytes()
        groof = {}
        for name, nbytes, ms, what in (("gemm1", g1b, dtl["g1_ms"], "gate-up grouped GEMM (fp8 weights streamed once)"),
                                       ("gemm2", g2b, dtl["g2_ms"], "down grouped GEMM (fp8 weights streamed once)")):
            gb = nbytes / (ms * 1e-3) / 1e9
            groof[name] = {"kernel": what, "bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(gb / PEAK_HBM_GBS, 4),
                           "traffic": measured_traffic(name, DECODE_TRAFFIC_FILE),
                           "avg_launch_us": round(ms * 1e3, 2), "bytes_per_launch": nbytes}
        result["decode"] = {"workload": "decode: T=64 H=8192 I=2048 E=8 top_k=2 fp8",
                            "us_per_layer": round(dms * 1e3, 1), "us_per_layer_gpu_events": round(dgpu_ms * 1e3, 1),
                            "us_per_layer_dispatch_events": percentiles_us(dtl["layer_ms"]),
                            "GB_per_s": round(gbs, 1),
                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": dbytes + dio,
                            "roofline_gemm1": groof["gemm1"], "roofline_gemm2": groof["gemm2"],
                            "stage_us_with_events": {n: round(v * 1e3, 2) for n, v in dstage.items()}}
        del dl
        torch.cuda.empty_cache()

    if not args.no_block:
        log("[bench] per-block fp8 routed weights (128 x 128 tiles): prefill and decode shares")
        blk = {}
        for name in ("prefill_block",) + (() if args.no_block_decode else ("decode_block",)):
            bl = Layer(name, args.copies)
            btl = time_layer(bl, 20, 3)
            bus = percentiles_us(btl["layer_ms"])
            fl, _ = bl.flops()
            wb, io, _ = bl.weight_bytes_touched()
            bms = btl["ms"] * 1e-3
            blk[name] = {"us_per_layer": round(bms * 1e6, 1), "us_per_layer_dispatch_events": bus,
                         "TFLOP/s": round(fl / bms / 1e12, 1),
                         "GB_per_s": round((wb + io) / bms / 1e9, 1),
                         "gemm_us": {"gemm1": round(btl["g1_ms"] * 1e3, 2), "gemm2": round(btl["g2_ms"] * 1e3, 2)}}
            del bl
            torch.cuda.empty_cache()
        result["fp8_block"] = blk

    if not args.no_latent:
        log("[bench] LatentMoE block (512 tokens, hidden 7168, latent 3584, 896 MXFP4 experts top-16, "
            "bf16 shared experts 7168->6144->7168)")
        lb = LatentBlock()
        ltl = time_layer(lb, 10, 2)
        lbytes, lflops, gate_up_bytes, ltouched = lb.accounting()
        lus = percentiles_us(ltl["layer_ms"])
        g1_us = ltl["g1_ms"] * 1e3
        result["latent_block"] = {
            "workload": "LatentMoE block: T=512 hidden=7168 latent=3584 I=3072 E=896 top_k=16 mxfp4, "
                        "shared 7168->6144->7168 bf16",
            "us_per_block_dispatch_events": lus, "us_per_block": round(ltl["ms"] * 1e3, 1),
            "algorithmic_bytes": lbytes, "touched_experts": ltouched,
            "GB_per_s": round(lbytes / (ltl["ms"] * 1e-3) / 1e9, 1),
            "frac_hbm": round(lbytes / (ltl["ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "TFLOP/s": round(lflops / (ltl["ms"] * 1e-3) / 1e12, 1),
            "roofline": {"kernel": "routed gate-up GEMM (MXFP4 weights streamed once)", "bound": "hbm",
                         "achieved": round(gate_up_bytes / (g1_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gate_up_bytes / (g1_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("gemm1", LATENT_TRAFFIC_FILE), "avg_launch_us": round(g1_us, 2),
                         "bytes_per_launch": gate_up_bytes},
            "core_gemm_us": {"gemm1": round(g1_us, 2), "gemm2": round(ltl["g2_ms"] * 1e3, 2)},
            "dense": dense_rates(lb),
        }
        del lb
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_tokens} sampled tokens")
        layer = Layer(args.config, 1)
        result["cpu_baseline"] = cpu_baseline(layer, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
