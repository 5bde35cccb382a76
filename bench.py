"""Benchmark of the DiT self-attention hot path on one MI355X.

A step is one full layer: dense attention over the whole token grid for all heads
(or, for a block-sparse workload, route + block-sparse attention).  Inputs are
seeded synthetic bf16 tensors already resident in HBM when the timed region
starts.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W]
                    [--workload v5|image|v5s|v10s|v10d|v5h7|v5w|v5sw|v5o|v5so|v5d128|v5s128|j_edit2|b_v5]
                    [--no-cpu-baseline] [--calib-copy]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/layer + TFLOP/s (frac of bf16 MFMA peak), 124,992 tokens, 56 heads d=96"
PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
DESCR = {
    "v5": "dense attention, 5 s 1344x768 video token grid 31x48x84 = 124,992 tokens, 56 heads x 96",
    "image": "dense attention, image token grid 1x256x256 = 65,536 tokens, 56 heads x 96",
    "v5s": "route + block-sparse attention (sparsity 0.75, 128-token blocks), 124,992 tokens, 56 heads x 96",
    "v10s": "route + block-sparse attention (sparsity 0.80, 128-token blocks), 245,952 tokens, 56 heads x 96",
    "v10d": "dense attention, 10 s video token grid 61x48x84 = 245,952 tokens, 56 heads x 96",
    "v5h7": ("dense attention, 124,992 tokens, 7 heads x 96: one GPU's head share when the 56-head layer is "
             "split by head over 8 GPUs"),
    "j_edit2": ("joint attention, image edit with 2 reference images: 65,536 target queries against "
                "197,120 keys (512 text + 2 x 65,536 reference + 65,536 target tokens), 56 heads x 96"),
    "v5d128": ("dense attention at head dim 128, 124,992 tokens, 42 heads x 128 (the same 5376 hidden width; "
               "RoPE chunks 44/42/42)"),
    "v5s128": ("route + block-sparse attention (sparsity 0.75) at head dim 128, 124,992 tokens, 42 heads x 128"),
    "v5w": ("dense attention, 124,992 tokens, 56 heads x 96, norm weights 1.75(1+0.1N(0,1)): logit bound 59.6, "
            "past what exp2 takes unshifted, so the static softmax subtracts a constant shift"),
    "v5sw": ("route + block-sparse attention (sparsity 0.75), 124,992 tokens, 56 heads x 96, norm weights "
             "1.75(1+0.1N(0,1)) (static softmax with a constant shift)"),
    "v5o": ("dense attention, 124,992 tokens, 56 heads x 96, w_q channel 0 at 6: logit bound 89.9, past the "
            "static limit of 80, so the running-maximum softmax runs"),
    "v5so": ("route + block-sparse attention (sparsity 0.75), 124,992 tokens, 56 heads x 96, w_q channel 0 at 6 "
             "(running-maximum softmax)"),
    "s4": "dense attention, small grid 5x24x40 = 4,800 tokens, 2 heads x 96 (contract checks)",
    "s4s": "route + block-sparse attention (sparsity 0.75), small grid 5x24x40, 2 heads x 96 (contract checks)",
    "j_small": ("joint attention, 768 target queries against 1,314 keys (50 text + 2 reference images + target), "
                "3 heads x 96 (contract checks)"),
    "b_mid": "operators around attention on 1,000 tokens, hidden 5376, FFN 14336 (contract checks)",
    "b_v5": ("operators around attention at 124,992 tokens, hidden 5376, FFN 14336: AdaLN update, gated "
             "residual + AdaLN update, SwiGLU, gated residual"),
}
BLOCK_METRIC = "GB/s of HBM (frac of 8 TB/s), AdaLN / gated residual / SwiGLU, 124,992 tokens, hidden 5376, FFN 14336"


KERNEL_SRC = os.path.join(ROOT, "image_diffusion_transformer_amd", "csrc", "attn_fwd.hip")
BLOCK_SRC = os.path.join(ROOT, "image_diffusion_transformer_amd", "csrc", "block_ops.hip")


def kernel_source_sha256(path: str = KERNEL_SRC) -> str:
    """SHA-256 of a kernel source's code: comments removed and whitespace runs collapsed, so that the stored
    HBM-traffic figures stay valid across comment edits and lapse with any change to the code itself."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    code = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    return hashlib.sha256(" ".join(code.split()).encode()).hexdigest()


def logit_bound(wq: np.ndarray, wk: np.ndarray, d: int) -> float:
    """log2(e) sqrt(d) max_i u_i v_i times a 2% margin, u_i, v_i being the larger |weight| of channel pair i
    in w_q, w_k: the bound on |logit| in base 2 that QK-RMSNorm and RoPE guarantee."""
    u = np.maximum(np.abs(wq[0::2]), np.abs(wq[1::2])).astype(np.float64)
    v = np.maximum(np.abs(wk[0::2]), np.abs(wk[1::2])).astype(np.float64)
    return math.log2(math.e) * math.sqrt(d) * float(np.max(u * v)) * 1.02


def softmax_mode(wq: np.ndarray, wk: np.ndarray, d: int) -> str:
    """Which attention kernel does the work for these norm weights: "static" (exp2 of the logits, less the
    constant max(0, bound - 48)) when the logit bound is at most 80, else "online" (running maximum).  Used to
    name the kernel."""
    return "static" if logit_bound(wq, wk, d) <= 80.0 else "online"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class ClockSampler:
    """Samples the GPU's graphics clock while the timed steps run, in a background thread: the current level of
    pp_dpm_sclk in sysfs (the power firmware's clock, refreshed every few milliseconds), else the mean of the
    XCDs' current clocks from amdsmi's GPU metrics (refreshed about once a second).  Reports the mean, median,
    min and max over the samples (MHz), or None where neither source is readable."""

    def __init__(self, period_s: float = 0.01):
        import threading
        self.period = period_s
        self.samples = []
        self.source = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._read = self._open()

    def _open(self):
        import glob
        for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            def read(path=path):
                for line in open(path).read().splitlines():
                    if line.rstrip().endswith("*"):
                        return float(re.findall(r"(\d+)\s*[Mm]hz", line)[0])
                return None
            try:
                if read() is not None:
                    self.source = f"sysfs {path} (current level)"
                    return read
            except Exception:
                continue
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                c = [int(v) for v in amdsmi.amdsmi_get_gpu_metrics_info(h)["current_gfxclks"]
                     if isinstance(v, (int, float)) and 0 < v < 10000]
                return sum(c) / len(c) if c else None
            if read() is not None:
                self.source = "amdsmi gpu metrics: mean of the XCDs' current_gfxclks"
                return read
        except Exception:
            pass
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None:
                    self.samples.append(v)
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._read is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.array(self.samples)
        return {"mean_mhz": round(float(a.mean()), 1), "median_mhz": round(float(np.median(a)), 1),
                "min_mhz": round(float(a.min()), 1), "max_mhz": round(float(a.max()), 1), "samples": int(a.size),
                "source": self.source}


def timing_summary(ms):
    """Mean, median and min of per-step event timings (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4)}


def sample_blocks(nb: int, count: int = 8, seed: int = 1234):
    """Query blocks the oracle checks: first, last (ragged), middle and seeded random ones."""
    rng = np.random.default_rng(seed)
    fixed = sorted(set([0, nb - 1, nb // 2]))
    others = np.setdiff1d(np.arange(nb), fixed)
    rest = [int(b) for b in rng.choice(others, size=min(len(others), max(0, count - len(fixed))), replace=False)]
    return sorted(set(fixed + rest))[:count]


def executed_flops(mask: np.ndarray, N: int, block: int = 128, d: int = 96) -> float:
    """4 d sum over kept (i, j) block pairs of |B_i| |B_j|."""
    nb = mask.shape[1]
    sizes = np.full(nb, block, dtype=np.float64)
    sizes[-1] = N - (nb - 1) * block
    per_head = np.einsum("hij,i,j->h", mask.astype(np.float64), sizes, sizes)
    return float(4.0 * d * per_head.sum())


def bench_joint(args, torch, dit):
    """Joint attention (explicit positions, queries = target tokens, keys = the whole sequence)."""
    from synth import make_joint_inputs
    x = make_joint_inputs(args.workload)
    wl = x.workload
    dev = torch.device("cuda:0")

    def up(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(x.q), up(x.k), up(x.v)
    wq, wk = torch.from_numpy(x.wq).to(dev), torch.from_numpy(x.wk).to(dev)
    qp = torch.from_numpy(x.q_pos).to(dev)
    kp = torch.from_numpy(x.k_pos).to(dev)
    o = torch.empty_like(q)
    ws = torch.empty(dit.dit_attn_joint_workspace_bytes(wl.Nq, wl.Nkv, wl.heads, wl.head_dim, x.max_pos), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def call():
        dit.dit_attn_joint(q, k, v, wq, wk, qp, kp, x.max_pos, wl.theta, wl.eps, o=o, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            events[i][0].record(stream)
            call()
            events[i][1].record(stream)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    call_ms = [e[0].elapsed_time(e[1]) for e in events]
    ms_call = float(np.mean(call_ms))
    flops = 4.0 * wl.Nq * wl.Nkv * wl.head_dim * wl.heads
    tflops = flops / (ms_step * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 Q/K/V; norm weights 1+0.1N(0,1))",
        "config": {"workload": f"{wl.name}: {DESCR[wl.name]}", "queries": wl.Nq, "keys": wl.Nkv, "heads": wl.heads,
                   "head_dim": wl.head_dim, "mode": "joint"},
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(flops / (ms_call * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flops / (ms_call * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": f"attn_static_kernel<{wl.head_dim}, false, false>", "kernel_ms": round(ms_call, 3),
                     "timed": "whole call: K^/V fragment prepass + attention kernels", "flops_per_launch": flops},
        "call_ms": timing_summary(call_ms),
        "sclk": clk.summary(),
    }
    # parity on sampled query rows of four heads, and the CPU baseline: the fp64 oracle on the same rows
    heads = sorted(set([0, wl.heads // 3, (2 * wl.heads) // 3, wl.heads - 1]))
    nqb = -(-wl.Nq // 128)
    blocks = sample_blocks(nqb)
    rows = np.concatenate([np.arange(b * 128, min(wl.Nq, (b + 1) * 128)) for b in blocks])
    o_np = o[torch.from_numpy(rows).to(dev)][:, heads].float().cpu().numpy()
    if not args.no_cpu_baseline:
        from oracle import attention as A
        cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        ref = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps, heads=heads, rows=rows)
        t_cpu = time.perf_counter() - t0
        err = np.abs(o_np.astype(np.float64) - ref)
        frac = (len(rows) * len(heads)) / (wl.Nq * wl.heads)
        result["parity"] = {"rows": int(len(rows)), "heads": heads, "blocks": blocks, "max_abs": float(err.max()),
                            "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(ref))}
        result["cpu_baseline"] = {
            "value": round(flops * frac / t_cpu / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads() or cores,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle on {len(blocks)} query blocks x {len(heads)} heads ({len(rows)} rows each, "
                       f"all {wl.Nkv} keys): {t_cpu:.1f} s for {frac:.5f} of the layer; full layer extrapolated to "
                       f"{t_cpu / frac:.0f} s"),
            "host_cores": cores}
    print(json.dumps(result), flush=True)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return None


def bench_block(args, torch, dit):
    """The fused operators around attention, each timed on its own; a step runs all four once."""
    from synth import BLOCK_WORKLOADS, make_block_inputs
    wl = BLOCK_WORKLOADS[args.workload]
    t0 = time.time()
    x = make_block_inputs(wl)
    log(f"inputs {wl.name}: {wl.tokens} tokens, hidden {wl.hidden}, ffn {wl.ffn} in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")

    def up(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    X, Y, GU = up(x.x), up(x.y), up(x.gate_up)
    gate, shift, scale = (torch.from_numpy(v).to(dev) for v in (x.gate, x.shift, x.scale))
    h1, h2, xo, xo2 = (torch.empty_like(X) for _ in range(4))
    out = torch.empty((wl.tokens, wl.ffn), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    act = wl.tokens * wl.hidden * 2
    ops = [  # name, call, algorithmic HBM bytes (activations; the fp32 vectors stay in cache)
        ("adaln_modulate", lambda: dit.dit_adaln_modulate(X, shift, scale, wl.eps, h=h1), 2 * act),
        ("gated_residual+adaln", lambda: dit.dit_gated_residual(X, Y, gate, shift, scale, wl.eps, x_out=xo, h=h2),
         4 * act),
        ("swiglu", lambda: dit.dit_swiglu(GU, out=out), 3 * wl.tokens * wl.ffn * 2),
        ("gated_residual", lambda: dit.dit_gated_residual(xo, Y, gate, x_out=xo2, modulate=False), 3 * act),
    ]
    for _ in range(args.warmup):
        for _, f, _ in ops:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            for j, (_, f, _) in enumerate(ops):
                f()
                ev[i][j + 1].record(stream)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j, (name, _, _) in enumerate(ops)}
    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    total = sum(b for _, _, b in ops)
    gbs = total / (ms_step * 1e-3) / 1e9
    dom = "swiglu"
    dom_bytes = dict((n, b) for n, _, b in ops)[dom]
    dom_gbs = dom_bytes / (per[dom] * 1e-3) / 1e9
    traffic = None
    tp = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(tp):
        with open(tp) as f:
            tr = json.load(f)
        if tr.get("workload") == wl.name and tr.get("source_sha256") == kernel_source_sha256(BLOCK_SRC):
            traffic = tr.get("bytes_per_launch")
    result = {
        "metric": BLOCK_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded: residual stream N(0,1) with per-channel offsets and wide channels, branch N(0,1), "
                "gate/up 2N(0,1), modulation vectors 0.5N(0,1))",
        "config": {"workload": f"{wl.name}: {DESCR[wl.name]}", "tokens": wl.tokens, "hidden": wl.hidden,
                   "ffn": wl.ffn},
        "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "per_op_ms": {n: round(v, 4) for n, v in per.items()},
        "per_op_gbs": {n: round(b / (per[n] * 1e-3) / 1e9, 1) for n, _, b in ops},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": f"swiglu_kernel<{min(8, -(-wl.ffn // 8 // 256))}>",
                     "kernel_ms": round(per[dom], 4), "bytes_per_launch": dom_bytes},
        "call_ms": {n: timing_summary([e[j].elapsed_time(e[j + 1]) for e in ev]) for j, (n, _, _) in enumerate(ops)},
        "sclk": clk.summary(),
    }
    if not args.no_cpu_baseline:
        from oracle import block_ops as O
        rows = np.arange(0, wl.tokens, max(1, wl.tokens // 256))[:256]
        cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        xs, ys, gus = x.x[rows].astype(np.float64), x.y[rows].astype(np.float64), x.gate_up[rows].astype(np.float64)
        O.adaln_modulate(xs, x.shift, x.scale, wl.eps)
        r, _ = O.gated_residual_adaln(xs, ys, x.gate, x.shift, x.scale, wl.eps)
        O.swiglu(gus)
        O.gated_residual(r, ys, x.gate)
        t_cpu = time.perf_counter() - t0
        frac = len(rows) / wl.tokens
        result["cpu_baseline"] = {
            "value": round(total * frac / t_cpu / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle of the four operators on {len(rows)} evenly spaced rows: {t_cpu:.2f} s "
                      f"for {frac:.5f} of the step (same algorithmic bytes per row)"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="v5", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--traffic", default=None,
                    help="HBM counter summary for the attention kernel (default: profiles/traffic_<workload>.json)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU mode (heads would shard "
              "across GPUs with one all-to-all each way; not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import image_diffusion_transformer_amd as dit
    from synth import WORKLOADS, make_inputs

    if args.workload.startswith("j_"):
        return bench_joint(args, torch, dit)
    if args.workload.startswith("b_"):
        return bench_block(args, torch, dit)

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = make_inputs(wl)
    log(f"inputs {wl.name}: N={wl.N} heads={wl.heads} generated in {time.time() - t0:.1f}s")

    def up(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = up(x.q), up(x.k), up(x.v)
    wq, wk = torch.from_numpy(x.wq).to(dev), torch.from_numpy(x.wk).to(dev)
    g = (wl.T, wl.H, wl.W)
    o = torch.empty_like(q)
    ws = dit.workspace_for(q, g)
    sparse = wl.mode == "sparse"
    mask = torch.empty((wl.heads, wl.nb, wl.nb), dtype=torch.uint8, device=dev) if sparse else None
    stream = torch.cuda.current_stream()
    N, H, d = wl.N, wl.heads, wl.head_dim
    dense_flops = 4.0 * N * N * d * H

    def step(ev=None):
        if sparse:
            if ev is not None:
                ev[0].record(stream)
            dit.dit_attn_route(q, k, wq, wk, g, wl.sparsity, wl.theta, wl.eps, mask=mask, workspace=ws)
            if ev is not None:
                ev[1].record(stream)
            dit.dit_attn_block_sparse(q, k, v, wq, wk, g, mask, wl.theta, wl.eps, o=o, workspace=ws)
            if ev is not None:
                ev[2].record(stream)
        else:
            if ev is not None:
                ev[0].record(stream)
            dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps, o=o, workspace=ws)
            if ev is not None:
                ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = 3 if sparse else 2
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t_start = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    if sparse:
        route_ms = [e[0].elapsed_time(e[1]) for e in events]
        attn_ms = [e[1].elapsed_time(e[2]) for e in events]
    else:
        route_ms = []
        attn_ms = [e[0].elapsed_time(e[1]) for e in events]
    ms_attn = float(np.mean(attn_ms))
    ms_route = float(np.mean(route_ms)) if route_ms else 0.0
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step (events: attn {ms_attn:.2f} ms, route {ms_route:.2f} ms)")

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if sparse:
        mask_np = mask.cpu().numpy()
        flops = executed_flops(mask_np, N, d=d)
    else:
        mask_np = None
        flops = dense_flops
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12

    traffic = None
    traffic_path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(traffic_path):
        with open(traffic_path) as f:
            tr = json.load(f)
        # counters taken on another version of the kernel source say nothing about this one
        if tr.get("workload") == wl.name and tr.get("source_sha256") == kernel_source_sha256():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded N(0,1) bf16 Q/K/V, video grids plus smooth sinusoid component; norm weights "
                 + ("1+0.1N(0,1)" if wl.weight_scale == 1.0 else f"{wl.weight_scale:g}(1+0.1N(0,1))")
                 + (f", w_q channel 0 at {wl.wq_spike:g})" if wl.wq_spike else ")")),
        "config": {"workload": f"{wl.name}: {DESCR[wl.name]}", "tokens": N, "heads": H, "head_dim": d,
                   "grid": [wl.T, wl.H, wl.W], "mode": wl.mode, "sparsity": wl.sparsity if sparse else None},
        "ms_per_layer": round(ms_step, 3),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": f"attn_{softmax_mode(x.wq, x.wk, d)}_kernel<{d}, " + ("true, false>" if sparse else "false, false>"),
                     "timed": "whole call: K^/V fragment prepass + attention kernels",
                     "kernel_ms": round(ms_attn, 3), "flops_per_launch": flops},
        # per-step event timings of the attention call (and of the router call for sparse workloads)
        "call_ms": timing_summary(attn_ms),
        "sclk": clk.summary(),
    }
    if sparse:
        result["dense_equivalent_tflops"] = round(dense_flops / (ms_step * 1e-3) / 1e12, 2)
        result["route_ms"] = round(ms_route, 3)
        result["route_call_ms"] = timing_summary(route_ms)
        result["kept_fraction"] = round(float(mask_np.mean()), 4)

    # ---- parity on sampled query blocks and the CPU baseline (fp64 oracle on host cores)
    blocks = sample_blocks(wl.nb)
    heads = sorted(set([0, H // 3, (2 * H) // 3, H - 1]))
    rows = np.concatenate([np.arange(b * 128, min(N, (b + 1) * 128)) for b in blocks])
    o_np = o[torch.from_numpy(rows).to(dev)][:, heads].float().cpu().numpy()
    if not args.no_cpu_baseline:
        from oracle import attention as A
        cores = len(os.sched_getaffinity(0))
        oracle_mask = mask_np
        mask_check = None
        if sparse:
            # the router's mask of head 0 against the oracle's (fp32 specification, every row), and O of head 0
            # evaluated on the oracle's mask; the other sampled heads on the router's
            from oracle import router as R
            t0 = time.perf_counter()
            m0 = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, wl.sparsity, wl.theta, wl.eps, heads=[0])[0]
            t_route = time.perf_counter() - t0
            bad = int(np.any(m0 != mask_np[0], axis=1).sum())
            oracle_mask = mask_np.copy()
            oracle_mask[0] = m0
            mask_check = {"head": 0, "rows": int(wl.nb), "rows_mismatched": bad, "oracle_s": round(t_route, 2)}
        t0 = time.perf_counter()
        ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, heads=heads, rows=rows,
                          mask=oracle_mask)
        t_cpu = time.perf_counter() - t0
        frac_rows = (len(rows) * len(heads)) / (N * H)
        if sparse:
            sizes = np.full(wl.nb, 128.0)
            sizes[-1] = N - (wl.nb - 1) * 128
            sample_flops = 4.0 * d * sum(float(sizes[b] * (mask_np[h, b] * sizes).sum())
                                         for h in heads for b in blocks)
        else:
            sample_flops = 4.0 * d * N * len(rows) * len(heads)
        cpu_tflops = sample_flops / t_cpu / 1e12
        err = np.abs(o_np.astype(np.float64) - ref)
        result["parity"] = {"rows": int(len(rows)), "heads": heads, "blocks": blocks,
                            "max_abs": float(err.max()), "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(ref)),
                            "mask_source": ("oracle router for head 0, gpu router for the others" if sparse
                                            else None),
                            "router_mask_vs_oracle": mask_check}
        result["cpu_baseline"] = {
            "value": round(cpu_tflops, 5), "unit": "TFLOP/s", "cores": blas_threads() or cores, "kind": "oracle",
            "sample": (f"fp64 numpy oracle on {len(blocks)} query blocks x {len(heads)} heads "
                       f"({len(rows)} rows each, all keys): {t_cpu:.1f} s for {frac_rows:.5f} of the layer; "
                       f"full layer extrapolated to {t_cpu / frac_rows:.0f} s"),
            "host_cores": cores,
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
