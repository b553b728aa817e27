"""Benchmark of the attention-layer hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--sweep] [--decode-loop]

One step is one pass of the whole path over one batch of synthetic input, in
the two shapes the headline metric is quoted on:
  * prefill phase -- long-context grouped-query prefill, B=2, L=8192, H_q=16,
    H_kv=4, d=128, causal, bf16 (Q, K, V given; 0.1% of feature channels x20);
  * decode phase  -- Llama-2-7B-shaped GQA decode, B=32, H_q=32, H_kv=8, d=128,
    hidden 4096: fused QKV GEMM of the 32 new tokens, the query heads taken as a
    strided view of the packed qkv rows (no copy), then split-KV attention over
    a contiguous cache of 4096 slots with lengths drawn from U{1024..4096}.
Inputs are resident in HBM before timing.  Warm-up steps run first; then K
steps are timed between two device synchronisations.  Per-kernel durations
come from HIP events recorded on the stream the kernels run on, during the
last max(10, K/5) of the timed steps (each event record adds about 3 us
between kernels, so the other steps run without them).

Prints ONE JSON line: `value` is the whole step's algorithmic TFLOP/s (prefill
+ GEMM + decode FLOPs over the step time); `prefill`, `decode` and `qkv_proj`
give each kernel's own rate and roofline fraction; `roofline` is the dominant
kernel (prefill, MFMA-bound); `cpu_baseline` times the CPU oracle on a bounded
sample of the same prefill workload.
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
COPY_BYTES = 256 << 20      # calibration copy: reads and writes this many bytes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_prefill_long_kv4_causal_traffic.json")
# what the prefill kernels' machine code depends on: their source, the shared
# device helpers and the build flags
KERNEL_SRCS = [os.path.join(ROOT, "mqa_qkv_proj_amd", "csrc", "attn_prefill.hip"),
               os.path.join(ROOT, "mqa_qkv_proj_amd", "csrc", "common.h"),
               os.path.join(ROOT, "mqa_qkv_proj_amd", "build.py")]


def kernel_digest():
    """SHA-256 over the files the prefill kernels are built from, in order."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--sweep", action="store_true", help="also time every configuration (stderr)")
    p.add_argument("--decode-loop", action="store_true",
                   help="also time the 1024-step MQA decode loop, eager and as one HIP graph (stderr)")
    p.add_argument("--calib-copy", action="store_true",
                   help="run one 256 MiB device-to-device copy first (known-size reference for HBM "
                        "byte counters)")
    return p.parse_args()


def prefill_flops(B, H_q, d, L_q, L_kv, causal):
    off = L_kv - L_q
    pairs = sum(min(L_kv, i + off + 1) for i in range(L_q)) if causal else L_q * L_kv
    return 4.0 * B * H_q * d * pairs


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
    by_prefill = 2.0 * (wp.B * wp.L * (wp.H_q + 2 * wp.H_kv) * wp.d + wp.B * wp.L * wp.H_q * wp.d)

    # Per-part durations come from HIP events recorded on the bench stream during
    # the last n_ev timed steps only: each event record costs about 3 us of GPU
    # time between kernels, which is instrumentation, not work of the step.
    ev = {k: [] for k in ("p0", "p1", "g1", "d1")}
    n_ev = min(args.steps, max(10, args.steps // 5))

    def step(record):
        e = {k: torch.cuda.Event(enable_timing=True) for k in ev} if record else None
        if record:
            e["p0"].record(stream)
        m.gqa_attn_prefill(Qp, Kp, Vp, causal=True, scale=scale_p, out=Op, workspace=ws_pf)
        if record:
            e["p1"].record(stream)  # also the start of the projection
        m.qkv_proj(x, wq, wd.H_q, wd.H_kv, wd.d, out=qkv, workspace=ws_proj)
        q_view = qkv[:, :wd.H_q * wd.d].unflatten(-1, (wd.H_q, wd.d))  # split: a strided view
        if record:
            e["g1"].record(stream)
        m.gqa_attn_decode(q_view, kc, vc, lens, scale=scale_d, workspace=ws, out=Od)
        if record:
            e["d1"].record(stream)
            for k in ev:
                ev[k].append(e[k])

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(False)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            step(i >= args.steps - n_ev)
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t_start

    def avg_ms(a, b):
        return sum(x.elapsed_time(y) for x, y in zip(ev[a], ev[b])) / len(ev[a])

    # Side measurement outside the timed steps: the same prefill with FP8 scores after
    # the random-sign Hadamard map (gqa_attn_prefill_fp8), for comparison only.
    signs = torch.from_numpy(W.random_signs(wp.seed, 6, wp.d)).to(dev)
    ws_f8 = torch.empty(m.prefill_fp8_workspace_bytes(wp.B, wp.L, wp.L, wp.H_q, wp.H_kv, wp.d), dtype=torch.uint8,
                        device=dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            m.gqa_attn_prefill_fp8(Qp, Kp, Vp, signs=signs, causal=True, scale=scale_p, out=Op, workspace=ws_f8)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(10):
            m.gqa_attn_prefill_fp8(Qp, Kp, Vp, signs=signs, causal=True, scale=scale_p, out=Op, workspace=ws_f8)
        f1.record(stream)
        f1.synchronize()
    ms_f8 = f0.elapsed_time(f1) / 10
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
        "prefill": {"tflops": round(pre_tf, 2), "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                    "us": round(ms_prefill * 1e3, 1), "gflop": round(fl_prefill / 1e9, 2)},
        "decode": {"gbps": round(dec_gbs, 1), "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                   "us": round(ms_decode * 1e3, 2), "mbytes": round(by_decode / 1e6, 2)},
        "qkv_proj": {"tflops": round(gemm_tf, 2), "gbps": round(gemm_gbs, 1),
                     "frac_hbm": round(gemm_gbs / PEAK_HBM_GBS, 4), "us": round(ms_gemm * 1e3, 2)},
        "prefill_fp8": {"tflops": round(fl_prefill / (ms_f8 * 1e-3) / 1e12, 2), "us": round(ms_f8 * 1e3, 1),
                        "speedup_vs_bf16": round(ms_prefill / ms_f8, 3),
                        "note": "same workload, e4m3 Q/K scores after the random-sign Hadamard map; not in value"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "gqa_attn_prefill (d=128, causal): V-image pre-pass + attention kernel"},
        "cpu_baseline": None,
    }
    if args.sweep:
        sweep(m, W, torch, dev, stream)
    if args.decode_loop:
        decode_loop(m, W, torch, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, wp, args.cpu_seconds)
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


def cpu_baseline(W, wp, seconds):
    """Time the fp64 CPU oracle on a bounded sample of the prefill workload."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    inp = W.prefill_inputs(wp, batch=range(0, wp.B))
    q, k, v = inp["q"], inp["k"], inp["v"]
    scale = 1.0 / math.sqrt(wp.d)
    flops, rows_done, t0 = 0.0, 0, time.perf_counter()
    blk = 512
    # causal row blocks, from the last (heaviest) block backwards, head by head, batch by batch
    order = [(b, h, r0) for b in range(wp.B) for r0 in range(wp.L - blk, -1, -blk) for h in range(wp.H_q)]
    for b, h, r0 in order:
        rows = np.arange(r0, r0 + blk)
        oracle.attention_rows(q, k, v, b, h, rows, True, scale)
        flops += 4.0 * wp.d * float((rows + 1).sum())
        rows_done += blk
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows_done} query rows (blocks of {blk}, heaviest first, batch by batch) of the "
                      f"causal prefill, fp64 numpy, {dt:.1f}s"}


def sweep(m, W, torch, dev, stream):
    """Time every configuration's kernels (to stderr); used for the design tables."""
    import numpy as np

    def up(a):
        bits = W.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def timeit(fn, n=20):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            for _ in range(n):
                fn()
            e.record(stream)
            e.synchronize()
        return s.elapsed_time(e) / n * 1e3  # us

    # cold-cache timing for the streaming kernels: before each call, read a
    # 512 MB buffer (clean lines, so nothing is written back) outside the events,
    # which evicts the 256 MB Infinity Cache
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def timeit_cold(fn, n=20):
        ts = []
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            for _ in range(n):
                torch.sum(flush, dim=0, out=flush_out)
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record(stream)
                fn()
                e.record(stream)
                e.synchronize()
                ts.append(s.elapsed_time(e) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]  # median, us

    for name, wl in W.WORKLOADS.items():
        if wl.dtype != "bf16":
            continue
        if wl.kind == "prefill":
            pin = W.prefill_inputs(wl)
            q, k, v = up(pin["q"]), up(pin["k"]), up(pin["v"])
            o = torch.empty_like(q)
            wsp = torch.empty(m.prefill_workspace_bytes(wl.B, wl.L, wl.H_kv, wl.d), dtype=torch.uint8, device=dev)
            us = timeit(lambda: m.gqa_attn_prefill(q, k, v, causal=wl.causal, out=o, workspace=wsp))
            fl = prefill_flops(wl.B, wl.H_q, wl.d, wl.L, wl.L, wl.causal)
            log(json.dumps({"sweep": name, "kernel": "prefill", "us": round(us, 2),
                            "tflops": round(fl / us / 1e6, 2), "frac": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}))
            if wl.d == 128:
                # FP8 scores after the random-sign Hadamard map (pre-passes included);
                # half the FLOPs (Q K^T) on the fp8 matrix cores, half (P V) on fp16 ones
                signs = torch.from_numpy(W.random_signs(wl.seed, 6, wl.d)).to(dev)
                ws8 = torch.empty(m.prefill_fp8_workspace_bytes(wl.B, wl.L, wl.L, wl.H_q, wl.H_kv, wl.d),
                                  dtype=torch.uint8, device=dev)
                us8 = timeit(lambda: m.gqa_attn_prefill_fp8(q, k, v, signs=signs, causal=wl.causal, out=o,
                                                            workspace=ws8))
                mixed_peak = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
                log(json.dumps({"sweep": name, "kernel": "prefill_fp8", "us": round(us8, 2),
                                "tflops": round(fl / us8 / 1e6, 2), "speedup_vs_bf16": round(us / us8, 3),
                                "frac_of_mixed_peak": round(fl / us8 / 1e6 / mixed_peak, 4)}))
                del ws8
            if wl.hidden:
                pj = W.proj_inputs(wl)
                x, w = up(pj["x"]), up(pj["w"])
                us = timeit(lambda: m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d))
                fl = 2.0 * x.shape[0] * wl.hidden * wl.N
                log(json.dumps({"sweep": name, "kernel": "qkv_proj", "us": round(us, 2),
                                "tflops": round(fl / us / 1e6, 2)}))
            del q, k, v, o, wsp
        else:
            din = W.decode_inputs(wl)
            kc, vc = up(din["k_cache"]), up(din["v_cache"])
            lens_np = din["seq_lens"]
            if name == "mqa_decode":
                lens_np = np.full(wl.B, wl.len_hi, np.int32)
            lens = torch.from_numpy(lens_np).to(dev)
            q = up(din["q"])
            o = torch.empty_like(q)
            ws = torch.empty(m.decode_workspace_bytes(wl.B, wl.H_q, wl.H_kv, wl.d, wl.L_max), dtype=torch.uint8,
                             device=dev)
            us = timeit(lambda: m.gqa_attn_decode(q, kc, vc, lens, workspace=ws, out=o))
            us_c = timeit_cold(lambda: m.gqa_attn_decode(q, kc, vc, lens, workspace=ws, out=o))
            by = 2.0 * (int(lens_np.sum()) * wl.H_kv * wl.d * 2 + 2 * wl.B * wl.H_q * wl.d)
            log(json.dumps({"sweep": name, "kernel": "decode", "us": round(us, 2),
                            "gbps": round(by / us / 1e3, 1), "frac": round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                            "us_cold": round(us_c, 2), "gbps_cold": round(by / us_c / 1e3, 1),
                            "frac_cold": round(by / us_c / 1e3 / PEAK_HBM_GBS, 4)}))
            # the same rows in a shuffled pool of 16-key pages
            P = 16
            pps = wl.L_max // P
            perm = torch.from_numpy(np.random.default_rng(wl.seed).permutation(wl.B * pps).astype(np.int32))
            table = perm.reshape(wl.B, pps).to(dev)
            kp = torch.empty(wl.B * pps, P, wl.H_kv, wl.d, dtype=torch.bfloat16, device=dev)
            vp = torch.empty_like(kp)
            kp[table.flatten().long()] = kc.reshape(wl.B * pps, P, wl.H_kv, wl.d)
            vp[table.flatten().long()] = vc.reshape(wl.B * pps, P, wl.H_kv, wl.d)
            us_p = timeit(lambda: m.gqa_attn_decode_paged(q, kp, vp, table, lens, workspace=ws, out=o))
            us_pc = timeit_cold(lambda: m.gqa_attn_decode_paged(q, kp, vp, table, lens, workspace=ws, out=o))
            log(json.dumps({"sweep": name, "kernel": "decode_paged16", "us": round(us_p, 2),
                            "gbps": round(by / us_p / 1e3, 1), "frac": round(by / us_p / 1e3 / PEAK_HBM_GBS, 4),
                            "us_cold": round(us_pc, 2), "gbps_cold": round(by / us_pc / 1e3, 1)}))
            del kp, vp
            pj = W.proj_inputs(wl)
            x, w = up(pj["x"]), up(pj["w"])
            us = timeit(lambda: m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d))
            us_c = timeit_cold(lambda: m.qkv_proj(x, w, wl.H_q, wl.H_kv, wl.d))
            by = 2.0 * (wl.hidden * wl.N + x.shape[0] * (wl.hidden + wl.N))
            log(json.dumps({"sweep": name, "kernel": "qkv_proj", "us": round(us, 2),
                            "gbps": round(by / us / 1e3, 1), "us_cold": round(us_c, 2),
                            "gbps_cold": round(by / us_c / 1e3, 1)}))
            del kc, vc
        torch.cuda.empty_cache()
    varlen_batch(m, W, torch, dev, timeit)


def varlen_batch(m, W, torch, dev, timeit):
    """A packed batch of 8 TinyLlama-shaped prompts (H_q=32, H_kv=4, d=64, causal)
    with seeded lengths U{128..2048}: one variable-length call against one
    fixed-length call per prompt (same kernels, same bits)."""
    import numpy as np

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
    ws = torch.empty(m.prefill_workspace_bytes(len(lens), L, H_kv, d), dtype=torch.uint8, device=dev)
    fl = sum(4.0 * H_q * d * n * (n + 1) / 2 for n in lens.tolist())
    us_v = timeit(lambda: m.gqa_attn_prefill_varlen(q, k, v, cu_d, cu_d, L, L, causal=True, out=o, workspace=ws))
    views = [(q[None, cu[b]:cu[b + 1]], k[None, cu[b]:cu[b + 1]], v[None, cu[b]:cu[b + 1]], o[None, cu[b]:cu[b + 1]])
             for b in range(len(lens))]

    def per_seq():
        for qb, kb, vb, ob in views:
            m.gqa_attn_prefill(qb, kb, vb, causal=True, out=ob, workspace=ws)
    us_s = timeit(per_seq)
    log(json.dumps({"sweep": "varlen_tinyllama_8", "lengths": lens.tolist(), "varlen_us": round(us_v, 2),
                    "varlen_tflops": round(fl / us_v / 1e6, 1), "per_sequence_us": round(us_s, 2),
                    "per_sequence_tflops": round(fl / us_s / 1e6, 1)}))


def decode_loop(m, W, torch, dev, stream):
    """The MQA decode workload as it runs: 1024 steps of (projection with the new
    token's K/V appended to the cache, decode, lengths + 1), the cache growing
    from 17 to 1040 keys.  Timed eagerly and as one captured HIP graph of all
    steps (3 kernels per step); prints per-step times to stderr."""
    import numpy as np

    wl = W.WORKLOADS["mqa_decode"]
    steps = wl.len_hi - wl.len_lo + 1

    def up(a):
        bits = W.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

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

    def run_all():
        for s in range(steps):
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
    kv_bytes = sum(2.0 * wl.B * (wl.len_lo + s) * wl.H_kv * wl.d * 2 for s in range(steps)) / steps
    w_bytes = 2.0 * wl.hidden * wl.N
    log(json.dumps({"decode_loop": wl.name, "steps": steps, "eager_us_per_step": round(eager, 2),
                    "graph_us_per_step": round(graphed, 2), "graph_speedup": round(eager / graphed, 2),
                    "bytes_per_step_mb": round((kv_bytes + w_bytes) / 1e6, 2),
                    "graph_gbps": round((kv_bytes + w_bytes) / graphed / 1e3, 1),
                    "last_step_output_equal": same}))


if __name__ == "__main__":
    main()
