"""Benchmark of the attention-layer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-configs] [--no-cpu-baseline] [--sweep]

One step is one pass of the whole path over one batch of synthetic input, in
the two shapes the headline metric is quoted on:
  * prefill phase -- long-context grouped-query prefill, B=2, L=8192, H_q=16,
    H_kv=4, d=128, causal, bf16 (Q, K, V given; 0.1% of feature channels x20);
  * decode phase  -- Llama-2-7B-shaped GQA decode, B=32, H_q=32, H_kv=8, d=128,
    hidden 4096: fused QKV GEMM of the 32 new tokens, the query heads taken as a
    strided view of the packed qkv rows (no copy), then split-KV attention over
    a contiguous cache of 4096 slots with lengths drawn from U{1024..4096}.
Inputs are resident in HBM before timing.  W warm-up steps run first; then K
steps are timed between two device synchronisations with nothing else on the
stream (`ms_per_step`).  A second timed pass of K steps records HIP events on
the stream the kernels run on around each part of every step: the per-kernel
durations and the roofline figure come from it.

Then every configuration is measured on its own (`configs`; skipped with
--no-configs): the tiny fp32 layer, the TinyLlama-shaped layers (projection,
prefill, whole layer eager and as one HIP graph), the MQA decode loop (eager
and as one HIP graph), the
Llama-2-7B decode sweep (cold caches) with its projections and, for GQA-8,
the whole decode step (projection with RoPE and KV append, decode) eager and
as one HIP graph, the four
long-context prefills in bf16 and FP8, and two packed variable-length batches
(persistent heaviest-first workers against the per-row-block grid).  Each
carries its roofline fraction.

Prints ONE JSON line: `value` is the whole step's algorithmic TFLOP/s (prefill
+ GEMM + decode FLOPs over the step time); `roofline` is the dominant kernel
(prefill attention, MFMA-bound); `cpu_baseline` times the CPU oracle on
bounded samples of every configuration.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
COPY_BYTES = 256 << 20      # calibration copy: reads and writes this many bytes
FLUSH_BYTES = 512 << 20     # cold-cache timing: a clean read of this many bytes before each call
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_prefill_long_kv4_causal_traffic.json")
# what the prefill kernels' machine code depends on: their source, the shared
# device helpers and the build flags
KERNEL_SRCS = [os.path.join(ROOT, "mqa_qkv_proj_amd", "csrc", "attn_prefill.hip"),
               os.path.join(ROOT, "mqa_qkv_proj_amd", "csrc", "common.h"),
               os.path.join(ROOT, "mqa_qkv_proj_amd", "build.py")]


def kernel_digest(paths=KERNEL_SRCS):
    """SHA-256 over the files a kernel is built from, in order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-configs", action="store_true", help="skip the per-configuration measurements")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=24.0, help="CPU oracle budget over all configurations")
    p.add_argument("--sweep", action="store_true",
                   help="also time paged decode and a packed variable-length batch (stderr)")
    p.add_argument("--calib-copy", action="store_true",
                   help="run one 256 MiB device-to-device copy first (known-size reference for HBM "
                        "byte counters)")
    return p.parse_args()


def prefill_flops(B, H_q, d, L_q, L_kv, causal):
    off = L_kv - L_q
    pairs = sum(min(L_kv, i + off + 1) for i in range(L_q)) if causal else L_q * L_kv
    return 4.0 * B * H_q * d * pairs


def gemm_roof_us(M, K, N):
    """Time of the projection at its roofline: max(MFMA time, HBM time of x, W, qkv)."""
    fl = 2.0 * M * K * N
    by = 2.0 * (K * N + M * K + M * N)
    return max(fl / (PEAK_BF16_TFLOPS * 1e6), by / (PEAK_HBM_GBS * 1e3)), fl, by


class Timer:
    """HIP-event timing on one stream; cold calls read a clean 512 MB buffer first
    (outside the events), which evicts the 256 MB Infinity Cache without leaving
    dirty lines."""

    def __init__(self, torch, dev, stream):
        self.torch, self.stream = torch, stream
        self.flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def spin_up(self, fn, seconds=0.05):
        """Run fn back to back for `seconds` first: the GPU's clock ramps up over
        several ms of sustained load (a long-context prefill measured 610 us in
        bursts of 10 calls from idle and 508 us in bursts of 200), so every
        figure here is taken at the steady clock of a sustained workload."""
        t = self.torch
        t0 = time.perf_counter()
        while True:
            for _ in range(3):
                fn()
            t.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return

    def warm(self, fn, n=20):
        t = self.torch
        with t.cuda.stream(self.stream):
            self.spin_up(fn)
            s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            s.record(self.stream)
            for _ in range(n):
                fn()
            e.record(self.stream)
            e.synchronize()
        return s.elapsed_time(e) / n * 1e3  # us

    def graphed(self, fn, n=20):
        """fn called n times back to back inside one captured HIP graph, replayed:
        the kernels' time without the host's launch gaps between them."""
        t = self.torch
        with t.cuda.stream(self.stream):
            self.spin_up(fn)
            t.cuda.synchronize()
            g = t.cuda.CUDAGraph()
            with t.cuda.graph(g, stream=self.stream):
                for _ in range(n):
                    fn()
            best = None
            for _ in range(3):
                g.replay()  # warm replay, then the timed one
                s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
                s.record(self.stream)
                g.replay()
                e.record(self.stream)
                e.synchronize()
                us = s.elapsed_time(e) / n * 1e3
                best = us if best is None else min(best, us)
            del g
        return best

    def cold(self, fn, n=15):
        t = self.torch
        ts = []
        with t.cuda.stream(self.stream):
            self.spin_up(fn)
            for _ in range(n):
                t.sum(self.flush, dim=0, out=self.flush_out)
                s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
                s.record(self.stream)
                fn()
                e.record(self.stream)
                e.synchronize()
                ts.append(s.elapsed_time(e) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]  # median, us


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no multi-GPU "
              "collectives to measure", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mqa_qkv_proj_amd as m
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)

    def up(a):
        bits = W.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    wp = W.WORKLOADS["long_kv4_causal"]
    pin = W.prefill_inputs(wp)
    Qp, Kp, Vp = up(pin["q"]), up(pin["k"]), up(pin["v"])
    del pin
    wd = W.WORKLOADS["llama7b_decode_kv8"]
    din = W.decode_inputs(wd)
    kc, vc = up(din["k_cache"]), up(din["v_cache"])
    lens_np = din["seq_lens"]
    lens = torch.from_numpy(lens_np).to(dev)
    del din
    pj = W.proj_inputs(wd)
    x, wq = up(pj["x"]), up(pj["w"])
    del pj
    Op = torch.empty(wp.B, wp.L, wp.H_q, wp.d, dtype=torch.bfloat16, device=dev)
    qkv = torch.empty(wd.B, wd.N, dtype=torch.bfloat16, device=dev)
    Od = torch.empty(wd.B, wd.H_q, wd.d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(m.decode_workspace_bytes(wd.B, wd.H_q, wd.H_kv, wd.d, wd.L_max), dtype=torch.uint8,
                     device=dev)
    ws_proj = torch.empty(max(16, m.qkv_proj_workspace_bytes(wd.B, wd.hidden, wd.H_q, wd.H_kv, wd.d)),
                          dtype=torch.uint8, device=dev)
    ws_pf = torch.empty(m.prefill_workspace_bytes(wp.B, wp.L, wp.H_kv, wp.d), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    if args.calib_copy:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    scale_p = 1.0 / math.sqrt(wp.d)
    scale_d = 1.0 / math.sqrt(wd.d)

    # ---------------------------------------------------------------- work per step
    fl_prefill = prefill_flops(wp.B, wp.H_q, wp.d, wp.L, wp.L, wp.causal)
    fl_gemm = 2.0 * wd.B * wd.hidden * wd.N
    by_gemm = 2.0 * (wd.hidden * wd.N + wd.B * wd.hidden + wd.B * wd.N)
    kv_tokens = int(lens_np.astype(np.int64).sum())
    by_decode = 2.0 * (kv_tokens * wd.H_kv * wd.d * 2 + 2 * wd.B * wd.H_q * wd.d)
    fl_decode = 4.0 * wd.H_q * wd.d * kv_tokens
    q_view = qkv[:, :wd.H_q * wd.d].unflatten(-1, (wd.H_q, wd.d))  # split: a strided view

    ev_names = ("p0", "p1", "g1", "d1")
    ev = {k: [] for k in ev_names}

    def step(record):
        e = {k: torch.cuda.Event(enable_timing=True) for k in ev_names} if record else None
        if record:
            e["p0"].record(stream)
        m.gqa_attn_prefill(Qp, Kp, Vp, causal=True, scale=scale_p, out=Op, workspace=ws_pf)
        if record:
            e["p1"].record(stream)  # also the start of the projection
        m.qkv_proj(x, wq, wd.H_q, wd.H_kv, wd.d, out=qkv, workspace=ws_proj)
        if record:
            e["g1"].record(stream)
        m.gqa_attn_decode(q_view, kc, vc, lens, scale=scale_d, workspace=ws, out=Od)
        if record:
            e["d1"].record(stream)
            for k in ev_names:
                ev[k].append(e[k])

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(False)
        # timed region 1: the steps alone (no event records between kernels)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            step(False)
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start
        # timed region 2: the same steps with HIP events around each part, for
        # the per-kernel durations (each record adds a few us between kernels)
        t2 = time.perf_counter()
        for _ in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        t_total_ev = time.perf_counter() - t2

    def avg_ms(a, b):
        return sum(x.elapsed_time(y) for x, y in zip(ev[a], ev[b])) / len(ev[a])

    # Side measurement outside the timed steps: the same prefill with FP8 scores after
    # the random-sign Hadamard map (gqa_attn_prefill_fp8), for comparison only.
    timer = Timer(torch, dev, stream)
    signs = torch.from_numpy(W.random_signs(wp.seed, 6, wp.d)).to(dev)
    ws_f8 = torch.empty(m.prefill_fp8_workspace_bytes(wp.B, wp.L, wp.L, wp.H_q, wp.H_kv, wp.d), dtype=torch.uint8,
                        device=dev)
    us_f8 = timer.warm(lambda: m.gqa_attn_prefill_fp8(Qp, Kp, Vp, signs=signs, causal=True, scale=scale_p, out=Op,
                                                      workspace=ws_f8), n=10)
    del ws_f8

    ms_prefill = avg_ms("p0", "p1")
    ms_gemm = avg_ms("p1", "g1")
    ms_decode = avg_ms("g1", "d1")
    ms_step = t_total * 1e3 / args.steps
    fl_step = fl_prefill + fl_gemm + fl_decode

    pre_tf = fl_prefill / (ms_prefill * 1e-3) / 1e12
    dec_gbs = by_decode / (ms_decode * 1e-3) / 1e9
    gemm_tf = fl_gemm / (ms_gemm * 1e-3) / 1e12
    gemm_gbs = by_gemm / (ms_gemm * 1e-3) / 1e9
    gemm_roof, _, _ = gemm_roof_us(wd.B, wd.hidden, wd.N)

    out = {
        "metric": "prefill attn TFLOPS + decode KV GB/s (frac. of roofline), 1 MI355X",
        "value": round(fl_step / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs, random-init weights)",
        "config": {
            "workload": "long-context GQA prefill (B=2, L=8192, H_q=16, H_kv=4, d=128, causal) + "
                        "Llama-2-7B GQA decode step (B=32, H_q=32, H_kv=8, d=128, hidden=4096, "
                        "KV lengths U{1024..4096} of 4096)",
            "prefill": {"B": wp.B, "L": wp.L, "H_q": wp.H_q, "H_kv": wp.H_kv, "d": wp.d, "causal": True},
            "decode": {"B": wd.B, "H_q": wd.H_q, "H_kv": wd.H_kv, "d": wd.d, "L_max": wd.L_max,
                       "hidden": wd.hidden, "kv_tokens": kv_tokens},
        },
        "ms_per_step_with_events": round(t_total_ev * 1e3 / args.steps, 4),
        "prefill": {"tflops": round(pre_tf, 2), "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                    "us": round(ms_prefill * 1e3, 1), "gflop": round(fl_prefill / 1e9, 2)},
        "decode": {"gbps": round(dec_gbs, 1), "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "us": round(ms_decode * 1e3, 2), "mbytes": round(by_decode / 1e6, 2)},
        "qkv_proj": {"tflops": round(gemm_tf, 2), "gbps": round(gemm_gbs, 1),
                     "frac": round(gemm_roof / (ms_gemm * 1e3), 4), "us": round(ms_gemm * 1e3, 2)},
        "prefill_fp8": {"tflops": round(fl_prefill / us_f8 / 1e6, 2), "us": round(us_f8, 1),
                        "speedup_vs_bf16": round(ms_prefill * 1e3 / us_f8, 3),
                        "note": "same workload, e4m3 Q/K scores after the random-sign Hadamard map; not in value"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "gqa_attn_prefill (d=128, causal): V-image pre-pass + attention kernel"},
        "cpu_baseline": None,
    }
    del Qp, Kp, Vp, Op, ws_pf
    torch.cuda.empty_cache()
    if not args.no_configs:
        out["configs"] = measure_configs(m, W, torch, np, dev, stream, timer, up,
                                         dict(kc=kc, vc=vc, lens=lens_np, x=x, w=wq))
    if args.sweep:
        extra_sweep(m, W, torch, np, dev, timer)
    del kc, vc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds, args.no_configs)
    print(json.dumps(out), flush=True)


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or None when
    the kernels' source or build flags changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        digest = kernel_digest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- every configuration

def measure_configs(m, W, torch, np, dev, stream, timer, up, kv8):
    """Each configuration's kernels on their own, with roofline fractions."""
    res = {}
    t_cfg = time.time()

    # -- tiny fp32 layer: projection + attention (parity config, launch-bound)
    wl = W.WORKLOADS["tiny_f32"]
    pj = W.proj_inputs(wl)
    x = torch.from_numpy(pj["x"]).to(dev).view(wl.B, wl.L, wl.hidden)
    w = torch.from_numpy(pj["w"]).to(dev)
    qkv = torch.empty(wl.B, wl.L, wl.N, dtype=torch.float32, device=dev)
    o = torch.empty(wl.B, wl.L, wl.H_q, wl.d, dtype=torch.float32, device=dev)

    def tiny_layer():
        m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d, out=qkv)
        q, k, v = m.split_qkv(qkv, wl.H_q, wl.H_kv, wl.d)
        m.gqa_attn_prefill(q, k, v, causal=True, out=o)
    us = timer.warm(tiny_layer)
    fl = 2.0 * wl.L * wl.hidden * wl.N + prefill_flops(wl.B, wl.H_q, wl.d, wl.L, wl.L, True)
    res[wl.name] = {"layer_us": round(us, 2), "tflops": round(fl / us / 1e6, 3),
                    "frac": round(fl / us / 1e6 / PEAK_FP32_TFLOPS, 4), "peak": "fp32 157.3 TFLOP/s",
                    "note": "parity configuration; launch-bound"}
    log(json.dumps({"config": wl.name, **res[wl.name]}))

    # -- TinyLlama-shaped layers: projection, prefill on the split views, whole layer
    for L in (128, 512, 2048):
        wl = W.WORKLOADS[f"tinyllama_L{L}"]
        pj = W.proj_inputs(wl)
        x, w = up(pj["x"]).view(wl.B, wl.L, wl.hidden), up(pj["w"])
        M = wl.B * wl.L
        qkv = torch.empty(wl.B, wl.L, wl.N, dtype=torch.bfloat16, device=dev)
        o = torch.empty(wl.B, wl.L, wl.H_q, wl.d, dtype=torch.bfloat16, device=dev)
        wsg = m.qkv_proj_workspace_bytes(M, wl.hidden, wl.H_q, wl.H_kv, wl.d)
        wsg = torch.empty(max(wsg, 16), dtype=torch.uint8, device=dev)
        wsp = torch.empty(m.prefill_workspace_bytes(wl.B, wl.L, wl.H_kv, wl.d), dtype=torch.uint8, device=dev)
        q, k, v = m.split_qkv(qkv, wl.H_q, wl.H_kv, wl.d)
        pos = torch.from_numpy(W.prefill_positions(wl.B, wl.L)).to(dev)
        th = torch.from_numpy(W.rope_inv_freq(wl.d)).to(dev)
        proj = lambda: m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=wsg)
        proj_rope = lambda: m.qkv_proj_rope(x, w, pos, th, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=wsg)
        attn = lambda: m.gqa_attn_prefill(q, k, v, causal=True, out=o, workspace=wsp)

        def layer():
            proj()
            attn()

        def layer_rope():
            proj_rope()
            attn()
        us_g, us_a, us_l = timer.warm(proj), timer.warm(attn), timer.warm(layer)
        us_gr, us_lr = timer.warm(proj_rope), timer.warm(layer_rope)
        layer()
        torch.cuda.synchronize()
        o_eager = o.clone()
        us_lg = timer.graphed(layer)  # o now holds the last replay's output
        torch.cuda.synchronize()
        graph_same = bool(torch.equal(o, o_eager))
        us_lrg = timer.graphed(layer_rope)
        roof_g, fl_g, by_g = gemm_roof_us(M, wl.hidden, wl.N)
        fl_a = prefill_flops(wl.B, wl.H_q, wl.d, wl.L, wl.L, True)
        res[wl.name] = {
            "qkv_proj": {"us": round(us_g, 2), "tflops": round(fl_g / us_g / 1e6, 2),
                         "bound": "hbm" if by_g / (PEAK_HBM_GBS * 1e3) > fl_g / (PEAK_BF16_TFLOPS * 1e6) else "mfma",
                         "frac": round(roof_g / us_g, 4)},
            "prefill": {"us": round(us_a, 2), "tflops": round(fl_a / us_a / 1e6, 2),
                        "frac": round(fl_a / us_a / 1e6 / PEAK_BF16_TFLOPS, 4)},
            "layer_us": round(us_l, 2), "layer_tflops": round((fl_g + fl_a) / us_l / 1e6, 2),
            "qkv_proj_rope_us": round(us_gr, 2), "layer_rope_us": round(us_lr, 2),
            "layer_graph_us": round(us_lg, 2), "layer_rope_graph_us": round(us_lrg, 2),
            "graph_output_equal": graph_same}
        log(json.dumps({"config": wl.name, **res[wl.name]}))
        del x, w, qkv, o, wsg, wsp, q, k, v, pos, th

    # -- MQA decode: the 1024-step loop (projection + KV append, decode, lengths + 1)
    res["mqa_decode"] = decode_loop(m, W, torch, np, dev, stream, up)
    log(json.dumps({"config": "mqa_decode", **res["mqa_decode"]}))

    # -- Llama-2-7B decode sweep, cold caches (the caches of the main step for
    #    H_kv = 8; seeded device draws of the same distribution for 32 and 4)
    for hkv in (32, 8, 4):
        wl = W.WORKLOADS[f"llama7b_decode_kv{hkv}"]
        if hkv == 8:
            kc, vc, lens_np = kv8["kc"], kv8["vc"], kv8["lens"]
        else:
            g = torch.Generator(device=dev).manual_seed(wl.seed)
            shape = (wl.B, wl.L_max, wl.H_kv, wl.d)
            kc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            vc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            lens_np = W.decode_lengths(wl)
        lens = torch.from_numpy(lens_np).to(dev)
        q = up(W.decode_step_q(wl, 0))
        o = torch.empty_like(q)
        wsd = torch.empty(m.decode_workspace_bytes(wl.B, wl.H_q, wl.H_kv, wl.d, wl.L_max), dtype=torch.uint8,
                          device=dev)
        by = 2.0 * (int(lens_np.astype(np.int64).sum()) * wl.H_kv * wl.d * 2 + 2 * wl.B * wl.H_q * wl.d)
        us_c = timer.cold(lambda: m.gqa_attn_decode(q, kc, vc, lens, workspace=wsd, out=o))
        us_w = timer.warm(lambda: m.gqa_attn_decode(q, kc, vc, lens, workspace=wsd, out=o))
        if hkv == 8:
            x, w = kv8["x"], kv8["w"]
        else:
            pj = W.proj_inputs(wl)
            x, w = up(pj["x"]), up(pj["w"])
        qkv = torch.empty(wl.B, wl.N, dtype=torch.bfloat16, device=dev)
        wsg = torch.empty(max(16, m.qkv_proj_workspace_bytes(wl.B, wl.hidden, wl.H_q, wl.H_kv, wl.d)),
                          dtype=torch.uint8, device=dev)
        proj = lambda: m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=wsg)
        gus_c, gus_w = timer.cold(proj), timer.warm(proj)
        roof_g, _, by_g = gemm_roof_us(wl.B, wl.hidden, wl.N)
        step_rec = {}
        if hkv == 8:
            # the whole decode step as the model runs it: the projection with the
            # rotary embedding and the new token's K/V appended to the caches, the
            # decode on the q view, lengths + 1; 20 steps eagerly and as one
            # captured HIP graph (lengths restored before each run)
            th = torch.from_numpy(W.rope_inv_freq(wl.d)).to(dev)
            lens_s = lens.clone()
            qv = qkv[:, :wl.H_q * wl.d].unflatten(-1, (wl.H_q, wl.d))
            nsteps = 20

            def steps_run():
                for _ in range(nsteps):
                    m.qkv_proj_append_rope(x, w, kc, vc, lens_s, th, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=wsg)
                    m.gqa_attn_decode(qv, kc, vc, lens_s, workspace=wsd, out=o)
                    lens_s.add_(1)

            def steps_timed(fn):
                lens_s.copy_(lens)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                return e0.elapsed_time(e1) * 1e3 / nsteps

            with torch.cuda.stream(stream):
                steps_timed(steps_run)  # warm-up
                st_eager = min(steps_timed(steps_run) for _ in range(3))
                graph = torch.cuda.CUDAGraph()
                lens_s.copy_(lens)
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=stream):
                    steps_run()
                st_graph = min(steps_timed(graph.replay) for _ in range(3))
                del graph
            step_rec = {"decode_step_rope_append": {
                "steps": nsteps, "eager_us_per_step": round(st_eager, 2), "graph_us_per_step": round(st_graph, 2),
                "note": "qkv_proj_append_rope + gqa_attn_decode + lengths + 1, caches warm from the runs above"}}
        res[wl.name] = {
            **step_rec,
            "decode": {"us_cold": round(us_c, 2), "gbps_cold": round(by / us_c / 1e3, 1),
                       "frac_cold": round(by / us_c / 1e3 / PEAK_HBM_GBS, 4), "us_warm": round(us_w, 2),
                       "mbytes": round(by / 1e6, 2)},
            "qkv_proj": {"us_cold": round(gus_c, 2), "gbps_cold": round(by_g / gus_c / 1e3, 1),
                         "frac_cold": round(roof_g / gus_c, 4), "us_warm": round(gus_w, 2),
                         "mbytes": round(by_g / 1e6, 2)}}
        log(json.dumps({"config": wl.name, **res[wl.name]}))
        del q, o, wsd, qkv, wsg, x, w
        if hkv != 8:
            del kc, vc
        torch.cuda.empty_cache()

    # -- long-context prefills, bf16 and FP8 (the FP8 call includes its pre-passes;
    #    half its FLOPs (Q K^T) on fp8 matrix cores, half (P V) on fp16 ones)
    mixed_peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
    for name in ("long_kv16_causal", "long_kv16_full", "long_kv4_causal", "long_kv4_full"):
        wl = W.WORKLOADS[name]
        pin = W.prefill_inputs(wl)
        q, k, v = up(pin["q"]), up(pin["k"]), up(pin["v"])
        del pin
        o = torch.empty_like(q)
        wsp = torch.empty(m.prefill_workspace_bytes(wl.B, wl.L, wl.H_kv, wl.d), dtype=torch.uint8, device=dev)
        us = timer.warm(lambda: m.gqa_attn_prefill(q, k, v, causal=wl.causal, out=o, workspace=wsp), n=10)
        signs = torch.from_numpy(W.random_signs(wl.seed, 6, wl.d)).to(dev)
        ws8 = torch.empty(m.prefill_fp8_workspace_bytes(wl.B, wl.L, wl.L, wl.H_q, wl.H_kv, wl.d),
                          dtype=torch.uint8, device=dev)
        us8 = timer.warm(lambda: m.gqa_attn_prefill_fp8(q, k, v, signs=signs, causal=wl.causal, out=o,
                                                        workspace=ws8), n=10)
        fl = prefill_flops(wl.B, wl.H_q, wl.d, wl.L, wl.L, wl.causal)
        res[name] = {"prefill": {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1),
                                 "frac": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)},
                     "prefill_fp8": {"us": round(us8, 1), "tflops": round(fl / us8 / 1e6, 1),
                                     "frac_of_mixed_peak": round(fl / us8 / 1e6 / mixed_peak, 4),
                                     "speedup_vs_bf16": round(us / us8, 3)}}
        log(json.dumps({"config": name, **res[name]}))
        del q, k, v, o, wsp, ws8
        torch.cuda.empty_cache()
    # -- packed variable-length batches (causal): the persistent heaviest-first
    #    workers (workspace with the row-block schedule) against the grid of one
    #    workgroup per row block (workspace of V images only).  TinyLlama heads
    #    over 8 sequences of U{128..2048} tokens; long-context heads over 16
    #    sequences of U{256..8192}
    for name, n, lo, hi, H_q, H_kv, d, seed in (("varlen_tinyllama_8", 8, 128, 2048, 32, 4, 64, 1007),
                                                 ("varlen_long_16", 16, 256, 8192, 16, 4, 128, 1008)):
        lens = np.random.default_rng(seed).integers(lo, hi, size=n, endpoint=True).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        tot, L = int(cu[-1]), int(lens.max())
        g = torch.Generator(device=dev).manual_seed(seed)
        q = torch.randn(tot, H_q, d, generator=g, device=dev).to(torch.bfloat16)
        k = torch.randn(tot, H_kv, d, generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn(tot, H_kv, d, generator=g, device=dev).to(torch.bfloat16)
        cu_d = torch.from_numpy(cu).to(dev)
        o = torch.empty_like(q)
        ws_s = torch.empty(m.prefill_varlen_workspace_bytes(n, L, tot, H_q, H_kv, d), dtype=torch.uint8, device=dev)
        ws_g = torch.empty(m.prefill_workspace_bytes(n, L, H_kv, d), dtype=torch.uint8, device=dev)
        fl = sum(prefill_flops(1, H_q, d, int(x), int(x), True) for x in lens)
        us_s = timer.warm(lambda: m.gqa_attn_prefill_varlen(q, k, v, cu_d, cu_d, L, L, out=o, workspace=ws_s))
        us_g = timer.warm(lambda: m.gqa_attn_prefill_varlen(q, k, v, cu_d, cu_d, L, L, out=o, workspace=ws_g))
        res[name] = {"lengths": lens.tolist(), "H_q": H_q, "H_kv": H_kv, "d": d,
                     "scheduled": {"us": round(us_s, 2), "tflops": round(fl / us_s / 1e6, 1),
                                   "frac": round(fl / us_s / 1e6 / PEAK_BF16_TFLOPS, 4)},
                     "grid": {"us": round(us_g, 2), "tflops": round(fl / us_g / 1e6, 1)},
                     "speedup": round(us_g / us_s, 3)}
        log(json.dumps({"config": name, **res[name]}))
        del q, k, v, o, ws_s, ws_g
        torch.cuda.empty_cache()
    res["seconds"] = round(time.time() - t_cfg, 1)
    return res


def decode_loop(m, W, torch, np, dev, stream, up):
    """The MQA decode workload as it runs: 1024 steps of (projection with the new
    token's K/V appended to the cache, decode, lengths + 1), the cache growing
    from 17 to 1040 keys.  Timed eagerly and as one captured HIP graph of all
    steps (3 kernels per step)."""
    wl = W.WORKLOADS["mqa_decode"]
    steps = wl.len_hi - wl.len_lo + 1
    din = W.decode_inputs(wl)
    kc, vc = up(din["k_cache"]), up(din["v_cache"])
    lens0 = torch.from_numpy(W.decode_lengths(wl, 0)).to(dev)
    lens = lens0.clone()
    w = up(W.proj_inputs(wl)["w"])
    xs = torch.stack([up(W.proj_inputs(wl, step=s)["x"]) for s in range(steps)])
    qkv = torch.empty(wl.B, wl.N, dtype=torch.bfloat16, device=dev)
    o = torch.empty(wl.B, wl.H_q, wl.d, dtype=torch.bfloat16, device=dev)
    ws_p = torch.empty(max(16, m.qkv_proj_workspace_bytes(wl.B, wl.hidden, wl.H_q, wl.H_kv, wl.d)),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(m.decode_workspace_bytes(wl.B, wl.H_q, wl.H_kv, wl.d, wl.L_max), dtype=torch.uint8,
                       device=dev)
    scale = 1.0 / math.sqrt(wl.d)
    q_view = qkv[:, :wl.H_q * wl.d].unflatten(-1, (wl.H_q, wl.d))

    th = torch.from_numpy(W.rope_inv_freq(wl.d)).to(dev)

    def run_all(rope=False):
        for s in range(steps):
            if rope:
                m.qkv_proj_append_rope(xs[s], w, kc, vc, lens, th, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=ws_p)
            else:
                m.qkv_proj_append(xs[s], w, kc, vc, lens, wl.H_q, wl.H_kv, wl.d, out=qkv, workspace=ws_p)
            m.gqa_attn_decode(q_view, kc, vc, lens, scale=scale, workspace=ws_d, out=o)
            lens.add_(1)

    def timed(fn):
        lens.copy_(lens0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps  # us per step

    with torch.cuda.stream(stream):
        lens.copy_(lens0)
        run_all()  # warm-up
        eager = min(timed(run_all) for _ in range(3))
        out_eager = o.clone()
        graph = torch.cuda.CUDAGraph()
        lens.copy_(lens0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            run_all()
        graphed = min(timed(graph.replay) for _ in range(3))
        same = bool(torch.equal(o, out_eager))
        # the same loop with the rotary embedding in the projection epilogue
        graph_r = torch.cuda.CUDAGraph()
        lens.copy_(lens0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph_r, stream=stream):
            run_all(rope=True)
        graphed_r = min(timed(graph_r.replay) for _ in range(3))
        del graph_r
        # one decode call at the final length (1040 keys), warm: the cache is resident
        lens.fill_(wl.len_hi)
        dec_us = 0.0
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(50):
            m.gqa_attn_decode(q_view, kc, vc, lens, scale=scale, workspace=ws_d, out=o)
        s1.record(stream)
        s1.synchronize()
        dec_us = s0.elapsed_time(s1) * 1e3 / 50
    kv_bytes = sum(2.0 * wl.B * (wl.len_lo + s) * wl.H_kv * wl.d * 2 for s in range(steps)) / steps
    w_bytes = 2.0 * wl.hidden * wl.N
    kv_last = 2.0 * wl.B * wl.len_hi * wl.H_kv * wl.d * 2
    return {"steps": steps, "eager_us_per_step": round(eager, 2), "graph_us_per_step": round(graphed, 2),
            "graph_speedup": round(eager / graphed, 2), "graph_rope_us_per_step": round(graphed_r, 2), "bytes_per_step_mb": round((kv_bytes + w_bytes) / 1e6, 2),
            "graph_gbps": round((kv_bytes + w_bytes) / graphed / 1e3, 1),
            "graph_frac_hbm": round((kv_bytes + w_bytes) / graphed / 1e3 / PEAK_HBM_GBS, 4),
            "decode_at_1040_us": round(dec_us, 2), "decode_at_1040_gbps": round(kv_last / dec_us / 1e3, 1),
            "last_step_output_equal": same,
            "note": "cache-resident (4.3 MB) and launch-bound; the graph runs all 1024 steps as one launch"}


def extra_sweep(m, W, torch, np, dev, timer):
    """Paged decode (16-key pages in a shuffled pool) beside the contiguous call,
    and a packed variable-length batch against one call per sequence (stderr)."""
    for hkv in (8, 4):
        wl = W.WORKLOADS[f"llama7b_decode_kv{hkv}"]
        g = torch.Generator(device=dev).manual_seed(wl.seed)
        shape = (wl.B, wl.L_max, wl.H_kv, wl.d)
        kc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        lens_np = W.decode_lengths(wl)
        lens = torch.from_numpy(lens_np).to(dev)
        q = torch.randn(wl.B, wl.H_q, wl.d, generator=g, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        ws = torch.empty(m.decode_workspace_bytes(wl.B, wl.H_q, wl.H_kv, wl.d, wl.L_max), dtype=torch.uint8,
                         device=dev)
        P = 16
        pps = wl.L_max // P
        perm = torch.from_numpy(np.random.default_rng(wl.seed).permutation(wl.B * pps).astype(np.int32))
        table = perm.reshape(wl.B, pps).to(dev)
        kp = torch.empty(wl.B * pps, P, wl.H_kv, wl.d, dtype=torch.bfloat16, device=dev)
        vp = torch.empty_like(kp)
        kp[table.flatten().long()] = kc.reshape(wl.B * pps, P, wl.H_kv, wl.d)
        vp[table.flatten().long()] = vc.reshape(wl.B * pps, P, wl.H_kv, wl.d)
        by = 2.0 * (int(lens_np.sum()) * wl.H_kv * wl.d * 2 + 2 * wl.B * wl.H_q * wl.d)
        us_c = timer.cold(lambda: m.gqa_attn_decode(q, kc, vc, lens, workspace=ws, out=o))
        us_pc = timer.cold(lambda: m.gqa_attn_decode_paged(q, kp, vp, table, lens, workspace=ws, out=o))
        log(json.dumps({"sweep": wl.name, "decode_us_cold": round(us_c, 2), "paged16_us_cold": round(us_pc, 2),
                        "paged16_gbps_cold": round(by / us_pc / 1e3, 1)}))
        del kc, vc, kp, vp
        torch.cuda.empty_cache()
    H_q, H_kv, d = 32, 4, 64
    lens = np.random.default_rng(1007).integers(128, 2048, size=8, endpoint=True).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tot = int(cu[-1])
    g = torch.Generator(device="cpu").manual_seed(1007)
    q = torch.randn(tot, H_q, d, generator=g).to(torch.bfloat16).to(dev)
    k = torch.randn(tot, H_kv, d, generator=g).to(torch.bfloat16).to(dev)
    v = torch.randn(tot, H_kv, d, generator=g).to(torch.bfloat16).to(dev)
    cu_d = torch.from_numpy(cu).to(dev)
    o = torch.empty_like(q)
    L = int(lens.max())
    ws = torch.empty(m.prefill_varlen_workspace_bytes(len(lens), L, tot, H_q, H_kv, d), dtype=torch.uint8,
                     device=dev)
    fl = sum(4.0 * H_q * d * n * (n + 1) / 2 for n in lens.tolist())
    us_v = timer.warm(lambda: m.gqa_attn_prefill_varlen(q, k, v, cu_d, cu_d, L, L, causal=True, out=o, workspace=ws))
    views = [(q[None, cu[b]:cu[b + 1]], k[None, cu[b]:cu[b + 1]], v[None, cu[b]:cu[b + 1]], o[None, cu[b]:cu[b + 1]])
             for b in range(len(lens))]

    def per_seq():
        for qb, kb, vb, ob in views:
            m.gqa_attn_prefill(qb, kb, vb, causal=True, out=ob, workspace=ws)
    us_s = timer.warm(per_seq)
    log(json.dumps({"sweep": "varlen_tinyllama_8", "lengths": lens.tolist(), "varlen_us": round(us_v, 2),
                    "varlen_tflops": round(fl / us_v / 1e6, 1), "per_sequence_us": round(us_s, 2),
                    "per_sequence_tflops": round(fl / us_s / 1e6, 1)}))


# ----------------------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(W, seconds, main_only):
    """Time the fp64 CPU oracle (as it stands) on bounded samples of every
    configuration, on this host's cores.  The headline figure is the
    long-context causal prefill sample in TFLOP/s; `configs` gives each
    configuration's oracle rate in its own unit."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    per = {}
    budget = seconds if main_only else seconds / 3.0

    # long-context causal prefill rows, heaviest 512-row blocks first, head by head, batch by batch
    wp = W.WORKLOADS["long_kv4_causal"]
    inp = W.prefill_inputs(wp)
    q, k, v = inp["q"], inp["k"], inp["v"]
    scale = 1.0 / math.sqrt(wp.d)
    flops, rows_done, t0 = 0.0, 0, time.perf_counter()
    blk = 512
    order = [(b, h, r0) for b in range(wp.B) for r0 in range(wp.L - blk, -1, -blk) for h in range(wp.H_q)]
    for b, h, r0 in order:
        rows = np.arange(r0, r0 + blk)
        oracle.attention_rows(q, k, v, b, h, rows, True, scale)
        flops += 4.0 * wp.d * float((rows + 1).sum())
        rows_done += blk
        if time.perf_counter() - t0 >= budget:
            break
    dt_main = time.perf_counter() - t0
    main_rate = flops / dt_main / 1e12
    per["long_kv4_causal"] = {"tflops": round(main_rate, 6), "seconds": round(dt_main, 2),
                              "sample": f"{rows_done} query rows, heaviest 512-row blocks first"}
    del q, k, v, inp

    if not main_only:
        share = (seconds - budget) / 6.0

        def timed_until(fn, limit):
            n, t = 0, time.perf_counter()
            while True:
                fn(n)
                n += 1
                if time.perf_counter() - t >= limit:
                    return n, time.perf_counter() - t

        # tiny fp32 and TinyLlama layers: whole x -> O passes
        for name in ("tiny_f32", "tinyllama_L128", "tinyllama_L512", "tinyllama_L2048"):
            wl = W.WORKLOADS[name]
            pj = W.proj_inputs(wl)
            fl = 2.0 * wl.B * wl.L * wl.hidden * wl.N + prefill_flops(wl.B, wl.H_q, wl.d, wl.L, wl.L, True)

            def layer(_):
                qkv = oracle.qkv_proj(pj["x"], pj["w"]).reshape(wl.B, wl.L, wl.N)
                qq, kk, vv = oracle.split_qkv(qkv, wl.H_q, wl.H_kv, wl.d)
                oracle.attention(qq, kk, vv, True, 1.0 / math.sqrt(wl.d))
            n, dt = timed_until(layer, share / 4.0)
            per[name] = {"tflops": round(fl * n / dt / 1e12, 6), "seconds": round(dt, 2),
                         "sample": f"{n} whole layer pass(es), x -> O"}

        # MQA decode: the first steps of the 1024-step loop (decode only)
        wl = W.WORKLOADS["mqa_decode"]
        din = W.decode_inputs(wl)

        def mqa_step(s):
            oracle.decode(W.decode_step_q(wl, s), din["k_cache"], din["v_cache"], W.decode_lengths(wl, s),
                          1.0 / math.sqrt(wl.d))
        n, dt = timed_until(mqa_step, share)
        by = sum(2.0 * wl.B * (wl.len_lo + s) * wl.H_kv * wl.d * 2 for s in range(n))
        per["mqa_decode"] = {"gbps": round(by / dt / 1e9, 4), "us_per_step": round(dt / n * 1e6, 1),
                             "seconds": round(dt, 2), "sample": f"decode steps 0..{n - 1} of 1024"}

        # Llama-2-7B decode: one step over the first sequences of each variant
        for hkv in (32, 8, 4):
            wl = W.WORKLOADS[f"llama7b_decode_kv{hkv}"]
            nb = 2
            din = W.decode_inputs(wl, batch=range(nb))

            def dstep(_):
                oracle.decode(din["q"], din["k_cache"], din["v_cache"], din["seq_lens"], 1.0 / math.sqrt(wl.d))
            n, dt = timed_until(dstep, share / 3.0)
            by = n * 2.0 * int(din["seq_lens"].astype(np.int64).sum()) * wl.H_kv * wl.d * 2
            per[wl.name] = {"gbps": round(by / dt / 1e9, 4), "seconds": round(dt, 2),
                            "sample": f"{n} decode step(s) of sequences 0..{nb - 1}"}
            del din

        # packed variable-length batches: whole sequences, shortest first, one at a time
        for name, nseq, lo, hi, H_q, H_kv, d, seed in (("varlen_tinyllama_8", 8, 128, 2048, 32, 4, 64, 1007),
                                                        ("varlen_long_16", 16, 256, 8192, 16, 4, 128, 1008)):
            lens = sorted(np.random.default_rng(seed).integers(lo, hi, size=nseq, endpoint=True).tolist())
            rng = np.random.default_rng(seed)
            fl, done, t = 0.0, 0, time.perf_counter()
            for n in lens:
                qs = rng.standard_normal((n, H_q, d), dtype=np.float32)
                ks = rng.standard_normal((n, H_kv, d), dtype=np.float32)
                vs = rng.standard_normal((n, H_kv, d), dtype=np.float32)
                cu = np.array([0, n], dtype=np.int32)
                oracle.attention_varlen(qs, ks, vs, cu, cu, True, 1.0 / math.sqrt(d))
                fl += prefill_flops(1, H_q, d, n, n, True)
                done += 1
                if time.perf_counter() - t >= share / 2.0:
                    break
            dt = time.perf_counter() - t
            per[name] = {"tflops": round(fl / dt / 1e12, 6), "seconds": round(dt, 2),
                         "sample": f"{done} of the {nseq} sequences, shortest first"}
    total = sum(p["seconds"] for p in per.values())
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return {"value": round(main_rate, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "sample": per["long_kv4_causal"]["sample"] + f" of the long-context causal prefill, fp64 numpy, "
                      f"{dt_main:.1f}s; every configuration in `configs` ({total:.1f}s in all)",
            "configs": per}


if __name__ == "__main__":
    main()
