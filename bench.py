#!/usr/bin/env python3
"""Throughput of the Mixtral-shaped sparse mixture-of-experts layer on one MI355X.

One step = one moe_forward call (route -> permute -> grouped expert GEMMs -> combine) over one
batch of seeded synthetic tokens that are already resident in HBM. The default workload is the
decode step (T=32 tokens, d=4096, F=14336, E=8, K=2, bf16): HBM-bound, every expert's weights
stream once. Other workloads (--workload) are reported the same way.

Prints ONE JSON line: tokens/s for the whole step, the roofline of the dominant kernel (timed
live with HIP events recorded by the library around that kernel inside the timed region) and
the CPU oracle timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import signal
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + TFLOP/s or HBM GB/s vs peak (E=8,K=2,d=4096,F=14336)"
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3         # fp32 MFMA/vector


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_T32")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="bounded CPU-oracle sample time")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="decode workload only: skip the prefill and tiny-layer objects of the default run")
    p.add_argument("--probe", choices=["copy"], help="plain copy of known size (counter calibration)")
    p.add_argument("--pass", dest="pass_", choices=["forward", "backward", "train", "block"], default="forward",
                   help="time moe_forward (default), moe_backward (gradients of the layer) or moe_block_forward "
                        "(decoder block: attention and the layer; workloads block_T*)")
    p.add_argument("--power", action="store_true",
                   help="forward pass: also report socket power and graphics clock (amd-smi) over the timed "
                        "steps; needs a timed region of a few seconds (many --steps)")
    p.add_argument("--weight-layout", choices=["packed", "rowmajor"], default="packed",
                   help="backward and train passes: expert weights (and the weight gradients) fragment-packed "
                        "(default) or row-major")
    return p.parse_args()


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "copy", "bytes_per_copy": n, "copies": 3}), flush=True)


def _code_only(src: str) -> str:
    """C/C++ source with comments removed and runs of whitespace collapsed (string and character
    literals kept as written), so that editing a comment leaves the digest of the code unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(files) -> str:
    """sha256 (first 16 hex digits) of the code of the named kernel sources (comments and layout
    ignored), in the order given: a counter summary is only valid for the code it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_33_amd", "csrc")
    for f in files:
        h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if taken on the current source
    of the files that define the kernel (listed in the summary as `source_files:`)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    f = re.search(r"source_files:\s*([^\n]+)", txt)
    m = re.search(r"source_digest:\s*(\w+)", txt)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not f or not m or not b or m.group(1) != source_digest(f.group(1).split()):
        return None
    return float(b.group(1))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the data-parallel layer needs no exchange between GPUs, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi

    torch.cuda.set_device(0)
    if args.probe == "copy":
        copy_probe()
        return

    w = mi.WORKLOADS[args.workload]
    # started before this process touches the GPU: the sampler is a child shell
    sampler = PowerSampler() if args.power and args.pass_ == "forward" else None
    if args.pass_ in ("backward", "train"):
        backward_bench(args, w, train=args.pass_ == "train")
        return
    if args.pass_ == "block":
        block_bench(args, w)
        return
    out, ctx = forward_bench(w, args.steps, args.warmup, sampler)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, ctx["x_host"], ctx["host_layer0"], args.cpu_seconds)
    del ctx
    if args.workload == "decode_T32" and not args.no_extra:
        # the other single-layer targets, timed in the same run: the prefill layer (the matrix-core
        # bound target) and the tiny fp32 layer (latency only)
        torch.cuda.empty_cache()
        p, pctx = forward_bench(mi.WORKLOADS["prefill_T4096"], min(args.steps, 20), min(args.warmup, 3))
        del pctx
        out["prefill_T4096"] = {k: p[k] for k in ("value", "unit", "ms_per_step", "step_tflops", "step_frac_mfma",
                                                   "roofline")}
        out["prefill_T4096"]["steps"] = min(args.steps, 20)
        torch.cuda.empty_cache()
        t, tctx = forward_bench(mi.WORKLOADS["tiny_f32"], args.steps, args.warmup)
        del tctx
        out["tiny_f32"] = {"value": t["value"], "unit": t["unit"], "ms_per_step": t["ms_per_step"],
                           "steps": args.steps, "dtype": "f32"}
    print(json.dumps(out), flush=True)


class PowerSampler:
    """Socket power and graphics clock over the timed steps, read with `amd-smi metric -p -c` about
    four times a second by a child shell (in its own process group) that runs from construction
    until summary(); rocm-smi gives the power cap once at its start."""

    CMD = ("rocm-smi --showmaxpower 2>/dev/null | grep -i 'max graphics package power'; "
           "while :; do echo \"T $(date +%s.%N)\"; amd-smi metric -p -c 2>/dev/null; sleep 0.2; done")

    def __init__(self):
        self.f = tempfile.NamedTemporaryFile("w+", prefix="moe_power_", suffix=".txt", delete=False)
        self.p = subprocess.Popen(["bash", "-c", self.CMD], stdout=self.f, stderr=subprocess.DEVNULL,
                                  start_new_session=True)

    def summary(self, t0, t1):
        os.killpg(self.p.pid, signal.SIGTERM)
        self.p.wait()
        self.f.close()
        text = open(self.f.name).read()
        os.unlink(self.f.name)
        return parse_power(text, t0, t1)


def parse_power(text, t0, t1):
    """Summary of the PowerSampler log `text` (blocks of amd-smi output, each after a line
    `T <unix time>`) over the samples taken inside the wall-clock interval [t0, t1]."""
    cap = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", text)
    samples, cur, sec = [], None, ""
    for line in text.splitlines():
        t = line.strip()
        if t.startswith("T "):
            cur = {"t": float(t[2:]), "w": None, "mhz": []}
            samples.append(cur)
        elif cur is None:
            continue
        elif t.endswith(":") and " " not in t:
            sec = t[:-1]
        elif t.startswith("SOCKET_POWER:"):
            m = re.search(r"([0-9.]+)\s*W", t)
            cur["w"] = float(m.group(1)) if m else None
        elif t.startswith("CLK:") and sec.startswith("GFX_"):
            m = re.search(r"([0-9.]+)\s*MHz", t)
            if m:
                cur["mhz"].append(float(m.group(1)))
    # samples taken inside the timed steps; the readings are averages over about the last second,
    # so the first second of the timed steps is skipped
    inside = [x for x in samples if t0 + 1.0 <= x["t"] <= t1 - 0.5 and x["w"] is not None and x["mhz"]]

    def med(v):
        v = sorted(v)
        return v[len(v) // 2] if v else None
    ws = [x["w"] for x in inside]
    clk = [sum(x["mhz"]) / len(x["mhz"]) for x in inside]
    return {"socket_w_median": med(ws), "socket_w_min": min(ws) if ws else None,
            "socket_w_max": max(ws) if ws else None, "gfx_mhz_median": med(clk),
            "gfx_mhz_min": min(clk) if clk else None, "gfx_mhz_max": max(clk) if clk else None,
            "power_cap_w": float(cap.group(1)) if cap else None, "samples": len(inside),
            "timed_s": round(t1 - t0, 2), "source": "amd-smi metric -p -c (socket power, mean of the GFX clocks)"}


def forward_bench(w, steps, warmup, sampler=None):
    """One step = one moe_forward over the workload's batch (all layers of a stack), inputs resident
    in HBM, fragment-packed weights. Returns (the bench record without cpu_baseline, host context).
    With a PowerSampler, the record also carries socket power and graphics clock over the timed steps."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_33_amd as moe
    from sparse_mixture_experts_33_amd.moe import MOE_STAGE_EXPERT_UP, stage_event_array

    dt = moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    s_x = 2 if w.dtype == "bf16" else 4

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    dims = moe.Dims(w.T, w.d, w.F, w.E, w.K, dt, moe.MOE_LAYOUT_PACKED)

    def packed(a, which):
        # one-time weight rearrangement at load time (like converting a checkpoint), not timed
        out = torch.empty_like(a)
        moe.moe_pack_weights(dims, which, a, out)
        torch.cuda.synchronize()
        return out

    t_gen = time.time()
    layers = []
    host_layer0 = None
    for layer in range(w.layers):
        W = mi.layer_weights(w, layer)
        L = {k: (dev(v) if v is not None else None) for k, v in W.items()}
        L["w1"] = packed(L["w1"], moe.MOE_W_UP)
        L["w3"] = packed(L["w3"], moe.MOE_W_UP)
        L["w2"] = packed(L["w2"], moe.MOE_W_DOWN)
        layers.append(L)
        if layer == 0:
            host_layer0 = W
        else:
            del W
        if w.layers > 1 and (layer + 1) % 4 == 0:
            log(f"[bench] {w.name}: {layer + 1} of {w.layers} layers generated ({time.time() - t_gen:.0f}s)")
    x_host = mi.tokens(w)
    x = dev(x_host)
    h0 = dev(mi.residual0(w)) if w.layers > 1 else None
    log(f"[bench] {w.name}: inputs generated and resident in HBM in {time.time() - t_gen:.1f}s")

    ws = torch.empty(moe.moe_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # routing of layer 0 (untimed) to count the experts that receive tokens
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    wt = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")
    L0 = layers[0]
    moe.moe_route(dims, x, L0["w_gate"], idx, wt, gate_bias=L0["bias"])
    counts = torch.bincount(idx.flatten().long(), minlength=w.E).cpu().numpy()
    active = int((counts > 0).sum())

    if w.layers == 1:
        y = torch.empty((w.T, w.d), dtype=tdt, device="cuda")
    else:
        h = torch.empty((w.T, w.d), dtype=torch.float32, device="cuda")
        xn = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")

    def step(events=None):
        if w.layers == 1:
            moe.moe_forward(dims, x, L0["w_gate"], L0["w1"], L0["w3"], L0["w2"], y, ws, gate_bias=L0["bias"],
                            stage_events=events)
        else:
            h.copy_(h0)
            for li, L in enumerate(layers):
                moe.moe_rmsnorm(w.T, w.d, w.eps, h, xn)
                moe.moe_forward(dims, xn, L["w_gate"], L["w1"], L["w3"], L["w2"], h, ws, gate_bias=L["bias"],
                                accumulate=True, stage_events=events if li == 0 else None)

    # Start and end of the dominant kernel (grouped GEMM 1 + SwiGLU), taken from its own dispatch on
    # the stream it runs on, on every `stride`-th timed step: a timed dispatch costs the step about
    # 8 us of extra latency, so timing every step would slow the decode step by ~2%.
    stride = max(1, steps // 10)
    sampled = list(range(0, steps, stride))
    ev = {}
    for i in sampled:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)  # torch creates the underlying event on its first record
        b.record(stream)
        ev[i] = (a, b)
    torch.cuda.synchronize()
    ev_arrays = {i: stage_event_array({2 * MOE_STAGE_EXPERT_UP: a.cuda_event, 2 * MOE_STAGE_EXPERT_UP + 1: b.cuda_event})
                 for i, (a, b) in ev.items()}

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0_wall = time.time()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev_arrays.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t1_wall = time.time()

    ms_step = elapsed * 1e3 / steps
    tokens_s = w.T * steps / elapsed
    up_ms = float(np.mean([a.elapsed_time(b) for a, b in ev.values()]))

    # algorithmic work per step (only routed experts count)
    S = w.T * w.K
    flops_layer = 2 * w.T * w.d * w.E + 6 * S * w.d * w.F
    bytes_layer = active * 3 * w.d * w.F * s_x + w.d * w.E * s_x + w.T * w.d * s_x + w.T * w.d * (4 if w.layers > 1 else s_x)
    step_flops = flops_layer * w.layers
    step_bytes = bytes_layer * w.layers
    # dominant kernel: grouped GEMM 1 (w1 and w3 of each routed expert, fused SwiGLU)
    up_flops = 4 * S * w.d * w.F
    up_bytes = active * 2 * w.F * w.d * s_x + S * w.d * s_x + S * w.F * s_x
    intensity = up_flops / up_bytes
    peak_tf = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    hbm_bound = intensity < peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved = up_bytes / (up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = up_flops / (up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4)}
    tr = stored_traffic("expert_up", w.name)
    roof["traffic"] = tr
    roof["kernel"] = "expert_up (grouped GEMM w1,w3 + SwiGLU)"
    roof["kernel_ms"] = round(up_ms, 4)
    roof["kernel_ms_sampled_steps"] = len(sampled)
    roof["algorithmic"] = {"bytes": up_bytes, "flops": up_flops}

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "F": w.F, "E": w.E, "K": w.K, "layers": w.layers,
                   "router_bias": "1.5*ln(1/(e+1))" if w.skew_bias else None, "active_experts": active,
                   "weight_layout": "fragment-packed (moe_pack_weights, at load time)",
                   "parallelism": "single GPU"},
        "step_tflops": round(step_flops / (ms_step * 1e-3) / 1e12, 2),
        "step_hbm_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_mfma": round(step_flops / (ms_step * 1e-3) / 1e12 / peak_tf, 4),
        "step_frac_hbm": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if sampler is not None:
        out["power"] = sampler.summary(t0_wall, t1_wall)
    return out, {"x_host": x_host, "host_layer0": host_layer0, "layers": layers}


BWD_METRIC = "MoE-layer backward tokens/s + TFLOP/s vs peak (E=8,K=2,d=4096,F=14336)"


TRAIN_METRIC = "MoE-layer training-step tokens/s (forward keeping activations + backward) + TFLOP/s vs peak"


def backward_bench(args, w, train=False):
    """One step = one moe_backward call (routing and expert pre-activations recomputed from x; dx,
    dW_g, dw1, dw3, dw2 in fp32) over the workload's tokens, inputs resident in HBM.
    train: one step = moe_forward keeping the expert pre-activations (moe_opts.activations) and
    moe_backward reading them. The expert weights are one copy both calls take, fragment-packed at
    load time (the weight gradients then come out in the same packed order, as an elementwise
    optimizer step on the packed weights wants them) or row-major (--weight-layout rowmajor)."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_33_amd as moe

    assert w.dtype == "bf16" and w.layers == 1, "the backward pass is timed on one bf16 layer"

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    packed = args.weight_layout == "packed"
    dims = moe.Dims(w.T, w.d, w.F, w.E, w.K, moe.MOE_BF16,
                    moe.MOE_LAYOUT_PACKED if packed else moe.MOE_LAYOUT_ROWMAJOR)
    W = mi.layer_weights(w)
    L = {k: (dev(v) if v is not None else None) for k, v in W.items()}
    if packed:
        for name, which in (("w1", moe.MOE_W_UP), ("w3", moe.MOE_W_UP), ("w2", moe.MOE_W_DOWN)):
            pk = torch.empty_like(L[name])  # load-time weight rearrangement, not timed
            moe.moe_pack_weights(dims, which, L[name], pk)
            L[name] = pk
        torch.cuda.synchronize()
    x_host, dy_host = mi.tokens(w), mi.upstream_grad(w)
    x, dy = dev(x_host), dev(dy_host)
    f32 = dict(dtype=torch.float32, device="cuda")
    dx = torch.empty((w.T, w.d), **f32)
    dwg = torch.empty((w.d, w.E), **f32)
    dw1 = torch.empty((w.E, w.F, w.d), **f32)
    dw3 = torch.empty((w.E, w.F, w.d), **f32)
    dw2 = torch.empty((w.E, w.d, w.F), **f32)
    ws = torch.empty(moe.moe_backward_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    act = torch.empty((2 * w.T * w.K * w.F,), **f32) if train else None
    y = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda") if train else None
    fws = torch.empty(moe.moe_workspace_bytes(dims), dtype=torch.uint8, device="cuda") if train else None
    mid = [(torch.cuda.Event(enable_timing=True)) for _ in range(args.steps + args.warmup)] if train else None
    it = [0]

    def step():
        if train:
            moe.moe_forward(dims, x, L["w_gate"], L["w1"], L["w3"], L["w2"], y, fws, gate_bias=L["bias"],
                            activations=act)
            mid[it[0]].record(stream)
            it[0] += 1
        moe.moe_backward(dims, x, L["w_gate"], L["w1"], L["w3"], L["w2"], dy, dx, dwg, dw1, dw3, dw2, ws,
                         gate_bias=L["bias"], activations=act)

    for _ in range(args.warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # algorithmic work of a backward pass: the gradient products w2^T dy, [w1|w3]^T [da|db] and the
    # three weight gradients (6 T*K*d*F multiply-adds, twice the forward), plus the router's two
    # T*d*E products. The recomputed forward products are implementation work, not counted. A
    # training step adds the forward's 6 T*K*d*F + 2 T*d*E.
    S = w.T * w.K
    flops = 12 * S * w.d * w.F + 4 * w.T * w.d * w.E
    if train:
        flops += 6 * S * w.d * w.F + 2 * w.T * w.d * w.E
        fwd_ms = float(np.mean([a.elapsed_time(m) for (a, _), m in zip(ev, mid[args.warmup:])]))
    tf = flops / (call_ms * 1e-3) / 1e12
    out = {
        "metric": TRAIN_METRIC if train else BWD_METRIC,
        "value": round(w.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens and upstream gradient, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "pass": "train" if train else "backward", "T": w.T, "d": w.d, "F": w.F,
                   "E": w.E, "K": w.K,
                   "weight_layout": "fragment-packed weights and weight gradients" if packed else "row-major",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": ("moe_forward + moe_backward, whole step" if train else "moe_backward, whole call")
                     + " (HIP events around each call)", "kernel_ms": round(call_ms, 4),
                     "algorithmic": {"flops": flops}},
        "cpu_baseline": None,
    }
    if train:
        out["forward_ms"] = round(fwd_ms, 4)
        out["backward_ms"] = round(call_ms - fwd_ms, 4)
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle_threads()
        sample = np.linspace(0, w.T - 1, 16).astype(np.int64)
        done, reps, t1 = 0, 0, time.perf_counter()
        while True:
            if train:
                oracle.forward(x_host, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, bias=W["bias"], tokens=sample,
                               threads=threads)
            oracle.backward_tokens(x_host, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, dy_host.astype(np.float64),
                                   sample, bias=W["bias"], threads=threads)
            done += len(sample)
            reps += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, **host_cores(),
                               "kind": "oracle",
                               "sample": ("forward outputs, " if train else "") +
                                         f"dx and logit gradients of {len(sample)} tokens x {reps} repetitions "
                                         f"({el:.1f}s; the weight-gradient sums are not included)"}
    print(json.dumps(out), flush=True)


BLOCK_METRIC = "Decoder-block tokens/s (causal GQA attention 32/8 heads + MoE layer, d=4096) + TFLOP/s vs peak"


def block_bench(args, w):
    """One step = one moe_block_forward call over a single sequence of w.T positions (norm, q/k/v
    projection, rotary embedding, causal grouped-query attention, output projection, residual, norm,
    the mixture-of-experts layer, residual), inputs resident in HBM. The residual stream is updated in
    place from step to step (its values do not change the work)."""
    import numpy as np
    import torch

    import moe_inputs as mi
    import sparse_mixture_experts_33_amd as moe
    from sparse_mixture_experts_33_amd.moe import MOE_BLOCK_NUM_STAGES, MOE_STAGE_ATTENTION, MOE_STAGE_EXPERT_UP

    assert w.dtype == "bf16" and w.layers == 1, "the block is timed on one bf16 layer"

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    t_gen = time.time()
    dims = moe.Dims(w.T, w.d, w.F, w.E, w.K, moe.MOE_BF16, moe.MOE_LAYOUT_PACKED)
    at = moe.AttnDims(w.T, w.d, w.n_heads, w.n_kv_heads, w.head_dim, w.rope_base, w.eps)
    W = mi.layer_weights(w)
    BW = mi.block_weights(w)
    L = {k: (dev(v) if v is not None else None) for k, v in W.items()}
    for name, which in (("w1", moe.MOE_W_UP), ("w3", moe.MOE_W_UP), ("w2", moe.MOE_W_DOWN)):
        packed = torch.empty_like(L[name])  # load-time weight rearrangement, not timed
        moe.moe_pack_weights(dims, which, L[name], packed)
        L[name] = packed
    wqkv, wo = dev(BW["w_qkv"]), dev(BW["w_o"])
    h0_host = mi.residual0(w)
    h = dev(h0_host)
    ws = torch.empty(moe.moe_block_workspace_bytes(dims, at), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs generated and resident in HBM in {time.time() - t_gen:.1f}s")

    # per timed step: the whole call, the attention kernel and the grouped GEMM 1 (from their dispatches)
    ev = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for x in e:
            x.record(stream)  # torch creates the underlying event on its first record
        ev.append(e)
    torch.cuda.synchronize()
    arrays = [moe.stage_event_array({2 * MOE_STAGE_ATTENTION: e[2].cuda_event, 2 * MOE_STAGE_ATTENTION + 1: e[3].cuda_event,
                                     2 * MOE_STAGE_EXPERT_UP: e[4].cuda_event, 2 * MOE_STAGE_EXPERT_UP + 1: e[5].cuda_event},
                                    MOE_BLOCK_NUM_STAGES) for e in ev]

    def step(arr=None):
        moe.moe_block_forward(dims, at, h, wqkv, wo, L["w_gate"], L["w1"], L["w3"], L["w2"], ws,
                              gate_bias=L["bias"], stage_events=arr)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e, arr in zip(ev, arrays):
        e[0].record(stream)
        step(arr)
        e[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    att_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    up_ms = float(np.mean([e[4].elapsed_time(e[5]) for e in ev]))

    # algorithmic work: projections, causal attention (each position attends to itself and the
    # positions before it: 2 T (T+1) D multiply-adds per query head for q.k and p.v), the layer
    T, d, D, Hq, Hkv = w.T, w.d, w.head_dim, w.n_heads, w.n_kv_heads
    att_flops = 2 * Hq * D * T * (T + 1)
    proj_flops = 2 * T * d * (Hq + 2 * Hkv) * D + 2 * T * Hq * D * d
    moe_flops = 2 * T * d * w.E + 6 * T * w.K * d * w.F
    block_flops = att_flops + proj_flops + moe_flops
    up_flops = 4 * T * w.K * d * w.F
    att_tf = att_flops / (att_ms * 1e-3) / 1e12
    out = {
        "metric": BLOCK_METRIC,
        "value": round(T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) residual stream, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "pass": "block", "T": T, "d": d, "F": w.F, "E": w.E, "K": w.K,
                   "n_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "rope_base": w.rope_base,
                   "weight_layout": "fragment-packed experts, row-major attention weights",
                   "parallelism": "single GPU"},
        "step_tflops": round(block_flops / (call_ms * 1e-3) / 1e12, 2),
        "step_frac_mfma": round(block_flops / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "block_ms": round(call_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(att_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attention (causal grouped-query flash attention)", "kernel_ms": round(att_ms, 4),
                     "algorithmic": {"flops": att_flops}},
        "expert_up": {"achieved": round(up_flops / (up_ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                      "kernel_ms": round(up_ms, 4), "flops": up_flops},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle_threads()
        # early positions: the oracle projects keys and values of every position up to the last one
        sample = np.array([0, 85, 170, 255], dtype=np.int64)
        h64 = h0_host.astype(np.float64)
        done, reps, t1 = 0, 0, time.perf_counter()
        while True:
            oracle.block(h64, BW["w_qkv"], BW["w_o"], W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, Hq, Hkv,
                         w.rope_base, w.eps, tokens=sample, bias=W["bias"], threads=threads)
            done += len(sample)
            reps += 1
            if time.perf_counter() - t1 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, **host_cores(),
                               "kind": "oracle",
                               "sample": f"block outputs of positions {list(map(int, sample))} (keys and values of "
                                         f"positions 0-255 projected each time) x {reps} repetitions ({el:.1f}s)"}
    print(json.dumps(out), flush=True)


def host_cores() -> dict:
    """The host's logical CPUs (as the OS reports them) and those this process may run on; the oracle
    uses at most 16 threads (the host share of one GPU)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"host_logical_cpus": os.cpu_count(), "host_cpus_usable": usable}


def oracle_threads() -> int:
    return max(1, min(16, host_cores()["host_cpus_usable"]))


def cpu_baseline(w, x_host, W, seconds):
    """The CPU oracle (fp64, plain loops, host threads) on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    threads = oracle_threads()
    sample = np.arange(min(w.T, 32), dtype=np.int64) if w.T <= 32 else np.linspace(0, w.T - 1, 16).astype(np.int64)
    done, t0 = 0, time.perf_counter()
    reps = 0
    while True:
        oracle.forward(x_host, W["w_gate"], W["w1"], W["w3"], W["w2"], w.K, bias=W["bias"], tokens=sample,
                       threads=threads)
        done += len(sample)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    note = f"{len(sample)} tokens of layer 0 x {reps} repetitions ({el:.1f}s)"
    if w.layers > 1:
        note += "; one layer of the stack, so tokens/s is per layer"
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, **host_cores(), "kind": "oracle",
            "sample": note}


if __name__ == "__main__":
    main()
