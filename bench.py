#!/usr/bin/env python3
"""Throughput of the quantized linear layer on one MI355X: the 3B-scale linear stack.

Workload (the pages' "3B-scale config": hidden 2048, intermediate 11008, 36
layers; their linear-backend microbench runs q_proj / up_proj / down_proj at
M = 1, 16, 256, 1024 tokens -- "Nano-vLLM-MoE" README, section "FP8 W8A8 static
quantization"):
  36 layers x {q_proj 2048->2048, up_proj 2048->11008, down_proj 11008->2048},
  chained (each output is the next input), in two variants
    * INT8 W8A16 (per-channel weight scales), and
    * FP8 W8A8 static (per-tensor weight scale, per-layer input scales
      calibrated offline on a 64-row batch through the bf16-dequant chain),
  swept over M in {1, 16, 256, 1024}.
One step = the 8 chains (2 variants x 4 M) = 864 GEMMs.  In the FP8 W8A8 chain
each layer's epilogue writes, beside its bf16 output, that output's codes at the
next layer's static input scale (qlq_qlinear_w8a8_static_requant), so the only
separate activation quantization is the one of the chain's input; the last layer
writes no codes.  Each chain is captured once
as a HIP graph and replayed, so the timed region holds GPU work only; weights
(1.65 GiB per variant) are far larger than the 256 MB last-level cache, so
every step streams them from HBM.

`next_rows` (not part of the step or of `value`), timed the same way after the
main region:
  * the same stack in INT8 W8A8 with dynamic per-token activation scales
    (quantize_act_dynamic + qlinear_w8a8_dynamic per layer);
  * the same stack through the routed Linear (qlq_linear: INT8 dynamic W8A8,
    a bf16 bias per projection, BF16 fallback for M <= 32);
  * the mixed K-int8 / V-FP8 KV-cache codec on the 7B shape of the pages' KV
    section (28 layers x 4 KV heads x head_dim 128): quantize T new tokens and
    decode T cached tokens per layer, T from 1 to 32768 (the 32K context of
    the pages' PPL table).

Output: one JSON line on stdout.  `value` is the whole step's TFLOP/s (2 M N K
per GEMM); `cases` gives us, TFLOP/s, algorithmic GB/s and roofline fractions per
(variant, M); `roofline` is for the dominant kernel; `cpu_baseline` times the
oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "qlinear µs, TFLOP/s and HBM GB/s at M=1/16/256/1024; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "int8": 5000.0}
VARIANTS = (("int8_w8a16", "w8a16", "int8", "per_channel"),
            ("fp8_w8a8_static", "w8a8_static_requant", "fp8_e4m3fn", "per_tensor"))
NEXT_VARIANTS = (("int8_w8a8_dynamic", "w8a8_dynamic", "int8", "per_channel"),
                 ("int8_linear_routed", "linear_routed", "int8", "per_channel"))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_bytes(scheme, M, K, N, per_tensor):
    """Algorithmic HBM bytes of one layer call (weight codes + scales + activations in + out),
    including the activation quantization the call implies:
      w8a16               N K + scales + 2 M K + 2 M N
      w8a8_static_fused   M <= 16: bf16 x read once by the GEMM: N K + scales + 2 M K + 2 M N
                          M > 16: quantization pass (2 M K read, M K written) + GEMM on codes (M K)
      w8a8_static_requant GEMM on codes (M K) that also writes the next layer's codes (M N):
                          N K + scales + M K + 3 M N; a chain adds one quantization pass (3 M K)
                          for its input and its last call writes no codes (see chain_bytes)
      w8a8_dynamic        quantization pass (2 M K read, M K + 4 M written) + GEMM (M K + 4 M)"""
    scale = 4 if per_tensor else 4 * N
    if scheme == "w8a16":
        return N * K + scale + 2 * M * K + 2 * M * N
    if scheme == "w8a8_static_fused" and M <= 16:
        return N * K + scale + 2 * M * K + 2 * M * N
    if scheme == "w8a8_static_fused":
        return N * K + scale + 4 * M * K + 2 * M * N
    if scheme == "w8a8_static_requant":
        return N * K + scale + M * K + 3 * M * N
    if scheme == "w8a8_dynamic":
        return N * K + scale + 4 * M * K + 8 * M + 2 * M * N
    if scheme == "linear_routed":      # dynamic W8A8 + bias; BF16 fallback (W8A16 bytes) at M <= 32
        if M <= 32:
            return N * K + scale + 2 * M * K + 2 * M * N + 2 * N
        return N * K + scale + 4 * M * K + 8 * M + 2 * M * N + 2 * N
    return N * K + scale + M * K + 2 * M * N


def chain_bytes(scheme, M, projs, layers, per_tensor):
    """Algorithmic bytes of one chain of layers x projs calls."""
    total = sum(gemm_bytes(scheme, M, K, N, per_tensor) for _, K, N in projs) * layers
    if scheme == "w8a8_static_requant":
        total += 3 * M * projs[0][1] - M * projs[-1][2]   # the input's quantization; no codes after the last
    return total


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_gemm_mfma_int8_w8a16_stack.txt")


def kernel_sources_hash():
    """sha256 over the HIP sources (name + bytes, sorted): identifies the kernels a profile measured."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "weight_quantized_linear_qlinear_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(family):
    """L2<->fabric bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a device copy of known size) from the
    committed counter profile, or None when the profile is for another kernel family or the kernels changed
    since it was taken.  The 256 MB last-level cache can serve these requests, so they bound HBM bytes from
    above."""
    if family != ("int8_w8a16", "large") or not os.path.exists(TRAFFIC_PROFILE):
        return None
    kv = {}
    for line in open(TRAFFIC_PROFILE):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != kernel_sources_hash():
        return None
    return int(float(kv["fabric_bytes_per_launch"]))


def build_stack(qlq, synth, torch, dev, seed, layers):
    """Quantized weights of both variants and the calibrated FP8 input scales."""
    import numpy as np
    qi, qf = [], []
    t0 = time.time()
    for l in range(layers):
        ri, rf = [], []
        for p in range(3):
            w = synth.stack_weight(seed, l, p, dev)
            ri.append(qlq.quantize_weight(w, "int8", "per_channel"))
            rf.append(qlq.quantize_weight(w, "fp8_e4m3fn", "per_tensor"))
            del w
        qi.append(ri)
        qf.append(rf)
    torch.cuda.synchronize()
    log(f"[bench] quantized {layers}x3 weights in {time.time() - t0:.1f}s")
    # offline calibration: a 64-row batch through the bf16-dequant chain of the FP8 weights
    calib, _ = synth.stack_inputs(seed, 1)
    h = torch.from_numpy(np.ascontiguousarray(calib).view(np.int16)).view(torch.bfloat16).to(dev)
    scales = torch.empty(layers * 3, dtype=torch.float32, device=dev)
    for l in range(layers):
        for p in range(3):
            qlq.calibrate_input_scale(h, "fp8_e4m3fn", out=scales[3 * l + p: 3 * l + p + 1])
            h = qlq.qlinear_w8a16(h, qf[l][p])
    sx = scales.cpu().tolist()
    return qi, qf, [[sx[3 * l + p] for p in range(3)] for l in range(layers)]


COLD_BYTES = 1 << 30       # rotated buffer sets per single-GEMM workload: past the 256 MB MALL and the L2s


def single_gemm_rows(qlq, synth, torch, dev, min_launches=200, warmup=3):
    """The four single-GEMM workloads (the pages' microbench shapes), each as one call
    of the library per launch.

    Cold (primary): R independent {packed W, scales, x, y} sets totalling >= 1 GiB, one
    launch per set in a captured graph, so every launch reads its weights from HBM.
    Hot (secondary): the same graph over one set (weights resident in the MALL/L2;
    comparable to the pages' cache-resident microbench, not an HBM figure).  Each graph
    is replayed until >= min_launches launches were timed; figures are per launch,
    with p10/p50/p90 over the replays.  W8A8 rows time the GEMM on codes
    (qlinear_w8a8_static) and, as `layer`, the one-call static W8A8 layer from bf16 x
    (quantization pass + GEMM, qlinear_w8a8_static_fused)."""
    import numpy as np
    res = {}
    stream = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    for idx, (name, c) in enumerate(synth.CASES.items()):
        inp = synth.case_inputs(c)
        qw = qlq.quantize_weight(torch.from_numpy(inp.w).to(dev), c.qtype, c.granularity)
        x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).view(torch.bfloat16).to(dev)
        w8a8 = c.scheme != "w8a16"
        M, K, N = c.M, c.K, c.N
        sx = 1.0
        if w8a8:
            cal = torch.from_numpy(np.ascontiguousarray(inp.calib).view(np.int16)).view(torch.bfloat16).to(dev)
            sx = qlq.calibrate_input_scale(cal, c.qtype).item()
        per_tensor = c.granularity == "per_tensor"
        set_bytes = qw.packed.numel() + 4 * qw.scale.numel() + 2 * M * K + 2 * M * N
        R = max(1, -(-COLD_BYTES // set_bytes))
        sets = []
        for _ in range(R):
            w_r = qlq.QuantizedWeight(qw.packed.clone(), qw.scale.clone(), qw.N, qw.K, qw.qtype, qw.granularity)
            x_r = x.clone()
            xq_r = qlq.quantize_act_static(x_r, sx, c.qtype) if w8a8 else None
            sets.append((w_r, x_r, xq_r, torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        ws_need = qlq.workspace_bytes("w8a8_static_fused" if w8a8 else "w8a16", M, K, N, c.qtype)
        ws = torch.zeros(max(ws_need, 256), dtype=torch.uint8, device=dev)

        def call(kind, st):
            w_r, x_r, xq_r, y_r = st
            if kind == "gemm" and not w8a8:
                qlq.qlinear_w8a16(x_r, w_r, out=y_r, workspace=ws)
            elif kind == "gemm":
                qlq.qlinear_w8a8_static(xq_r, sx, w_r, out=y_r, workspace=ws)
            else:
                qlq.qlinear_w8a8_static_fused(x_r, sx, w_r, out=y_r, workspace=ws)

        row = {"config": idx, "scheme": c.scheme, "qtype": c.qtype, "M": M, "K": K, "N": N, "cold_sets": R,
               "cold_bytes": R * set_bytes}
        flops = 2 * M * N * K
        for kind in (("gemm", "layer") if w8a8 else ("gemm",)):
            byts = N * K + (4 if per_tensor else 4 * N) + 2 * M * N + (2 * M * K if not w8a8 else M * K)
            if kind == "layer":
                byts += 3 * M * K
            dt = "bf16" if not w8a8 else ("fp8" if c.qtype == "fp8_e4m3fn" else "int8")
            for temp, picks in (("cold", sets), ("hot", [sets[0]] * R)):
                for st in picks[:2]:
                    call(kind, st)                      # eager warm-up (and LDS limits) outside capture
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for st in picks:
                        call(kind, st)
                reps = max(3, -(-min_launches // R))
                for _ in range(warmup):
                    g.replay()
                evs = []
                for _ in range(reps):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(cur)
                    g.replay()
                    e1.record(cur)
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                per = np.array([a.elapsed_time(b) * 1e3 / R for a, b in evs])
                us = float(per.mean())
                t_hbm = byts / (HBM_PEAK_GBS * 1e9) * 1e6
                t_mfma = flops / (MFMA_PEAK_TFLOPS[dt] * 1e12) * 1e6
                key = f"{kind}_{temp}"
                row[key] = {"us": round(us, 3), "p10_us": round(float(np.percentile(per, 10)), 3),
                            "p50_us": round(float(np.percentile(per, 50)), 3),
                            "p90_us": round(float(np.percentile(per, 90)), 3),
                            "launches": int(R * reps), "tflops": round(flops / us / 1e6, 3),
                            "gbs": round(byts / us / 1e3, 1), "algorithmic_bytes": int(byts),
                            "hbm_frac": round(t_hbm / us, 3), "mfma_frac": round(t_mfma / us, 3),
                            "bound": "hbm" if t_hbm >= t_mfma else "mfma"}
                if temp == "hot":
                    row[key]["note"] = "one buffer set: MALL/L2-resident, not an HBM figure"
                del g
        res[f"config{idx}/{name}"] = row
        del sets, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log(f"[bench] single GEMM {name}: cold {row['gemm_cold']['us']} us over {R} sets")
    return res


KV_LAYERS, KV_HEADS, KV_DIM = 28, 4, 128
KV_TOKENS = (1, 16, 256, 1024, 8192, 32768)     # new tokens per step up to a 32K context read


def kv_rows(qlq, torch, dev, Ts, steps, warmup):
    """Time the KV-cache codec: one graph per (op, T) over the 28 layers."""
    import numpy as np
    Tmax = max(Ts)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    shape = (KV_LAYERS, Tmax, KV_HEADS, KV_DIM)
    k = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    q = [qlq.kv_quantize(k[l], v[l]) for l in range(KV_LAYERS)]
    ko = torch.empty((Tmax, KV_HEADS, KV_DIM), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    per_entry = 2 * KV_DIM + 2 * (KV_DIM // 32) + 2
    res = {}
    stream = torch.cuda.Stream()
    for op in ("kv_quantize", "kv_dequantize"):
        for T in Ts:
            def run():
                for l in range(KV_LAYERS):
                    if op == "kv_quantize":
                        e = q[l]
                        qlq.kv_quantize(k[l, :T], v[l, :T], out=qlq.QuantizedKV(e.k_codes[:T], e.k_scales[:T],
                                                                                e.v_codes[:T], e.v_scales[:T]))
                    else:
                        e = q[l]
                        qlq.kv_dequantize(qlq.QuantizedKV(e.k_codes[:T], e.k_scales[:T], e.v_codes[:T],
                                                          e.v_scales[:T]), ko[:T], vo[:T])
            run()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                run()
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps / KV_LAYERS
            entries = T * KV_HEADS
            byts = entries * (4 * KV_DIM + per_entry)             # bf16 K and V one way, codes + scales the other
            res[f"{op}/T={T}"] = {"us_per_layer": round(us, 3), "gbs": round(byts / us / 1e3, 1),
                                  "hbm_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 3), "bound": "hbm"}
    return res


BUCKET_M = (1, 5, 13, 30, 50, 100, 300)   # not buckets (except 1): padded to 1, 8, 16, 32, 64, 128, 512


def bucket_rows(qlq, synth, torch, dev, qi, L, steps, warmup):
    """The INT8 W8A16 stack through decode-batch graph buckets (GraphBuckets): one captured
    graph per bucket size (1, 2, 4, ..., 512); a batch of M rows is copied into its
    bucket's input (pad rows zeroed) and the bucket's graph is replayed."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    mids = {}

    def fn(x, y):
        b = x.shape[0]
        h = x
        for l in range(L):
            for p, (_, K, N) in enumerate(synth.STACK_PROJS):
                last = l == L - 1 and p == len(synth.STACK_PROJS) - 1
                out = y if last else mids.setdefault((b, l % 2, p), torch.empty((b, N), dtype=torch.bfloat16,
                                                                                  device=dev))
                qlq.qlinear_w8a16(h, qi[l][p], out=out, workspace=ws)
                h = out

    gb = qlq.GraphBuckets(fn, synth.HIDDEN, synth.HIDDEN, device=dev)
    res = {}
    cur = torch.cuda.current_stream()
    for M in BUCKET_M:
        x = torch.randn((M, synth.HIDDEN), device=dev).to(torch.bfloat16)
        for _ in range(warmup):
            gb(x)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(steps):
            gb(x)
        e1.record(cur)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        b = gb.bucket_for(M)
        flops = sum(2 * M * N * K for _, K, N in synth.STACK_PROJS) * L
        res[f"bucketed_int8_w8a16/M={M}"] = {"bucket": b, "us_per_stack": round(us, 2),
                                              "us_per_gemm": round(us / (3 * L), 3),
                                              "tflops_real_rows": round(flops / us / 1e6, 2)}
    return res


CPU_SAMPLE_LAYERS = 2


def cpu_baseline(seed, layers_w, sx):
    """Time the oracle on the first CPU_SAMPLE_LAYERS layers of the stack (both variants, every M):
    about 10 s of host work."""
    import numpy as np
    import oracle
    import synth
    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info() if i["user_api"] == "blas")
    except Exception:
        threads = os.cpu_count()
    # offline steps (not timed): the oracle's own quantized weights
    w_host = [[w.cpu().numpy() for w in lw] for lw in layers_w]
    qi = [[oracle.quantize_weight(w, "int8", "per_channel") for w in lw] for lw in w_host]
    qf = [[oracle.quantize_weight(w, "fp8_e4m3fn", "per_tensor") for w in lw] for lw in w_host]
    flops = 0
    t0 = time.perf_counter()
    for M in synth.STACK_M:
        _, x = synth.stack_inputs(seed, M)
        h = x
        for l in range(len(layers_w)):
            for p, (_, K, N) in enumerate(synth.STACK_PROJS):
                h = oracle.qlinear_w8a16(h, qi[l][p][0], qi[l][p][1], "int8")
                flops += 2 * M * N * K
        h = x
        for l in range(len(layers_w)):
            for p, (_, K, N) in enumerate(synth.STACK_PROJS):
                s = np.float32(sx[l][p])
                xq = oracle.quantize_act_static(h, s, "fp8_e4m3fn")
                h = oracle.qlinear_w8a8_static(xq, s, qf[l][p][0], qf[l][p][1], "fp8_e4m3fn")
                flops += 2 * M * N * K
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt, "cpu": platform.processor() or platform.machine(),
            "sample": f"layers 0-{len(layers_w) - 1} of the stack (q_proj, up_proj, down_proj chained), "
                      "INT8 W8A16 and FP8 W8A8 "
                      "(activation quantization included, offline weight quantization and calibration "
                      "excluded), M in {1,16,256,1024}; float64 NumPy oracle"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layers", type=int, default=36, help="decoder layers in the stack (36 = the pages' config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only: skip next_rows and the single-GEMM workloads (short profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run one 256 MiB device copy (known HBM bytes) so that "
                         "profiler byte counters can be scaled")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the quantized linear layer runs on a single MI355X, and "
              "no multi-GPU sharding is run. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    import weight_quantized_linear_qlinear_amd as qlq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = args.layers
    qi, qf, sx = build_stack(qlq, synth, torch, dev, args.seed, L)
    variants = {"int8_w8a16": qi, "fp8_w8a8_static": qf, "int8_w8a8_dynamic": qi, "int8_linear_routed": qi}
    # routed Linear: a bf16 bias per layer and projection, BF16 fallback at M <= 32
    gb = torch.Generator(device=dev)
    gb.manual_seed(args.seed + 77)
    biases = [[(torch.randn(N, generator=gb, device=dev) * 0.1).to(torch.bfloat16) for _, _, N in synth.STACK_PROJS]
              for _ in range(L)]

    # buffers: inputs per M, ping-pong activations, codes, one shared workspace
    Ms = synth.STACK_M
    Mmax = max(Ms)
    x0 = {}
    for M in Ms:
        _, x = synth.stack_inputs(args.seed, M)
        x0[M] = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    hbuf = [torch.empty(Mmax * synth.INTERMEDIATE, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    xqbuf = torch.empty(Mmax * synth.INTERMEDIATE, dtype=torch.uint8, device=dev)
    cbuf = [torch.empty(Mmax * synth.INTERMEDIATE, dtype=torch.uint8, device=dev) for _ in range(2)]
    sxbuf = torch.empty(Mmax, dtype=torch.float32, device=dev)
    ws_need = 0
    for _, scheme, qtype, _ in VARIANTS + NEXT_VARIANTS:
        for M in Ms:
            for _, K, N in synth.STACK_PROJS:
                if scheme == "linear_routed":
                    ws_need = max(ws_need, qlq.linear_workspace_bytes("w8a8_dynamic", M, K, N, qtype))
                elif scheme == "w8a8_static_requant":
                    ws_need = max(ws_need, qlq.workspace_bytes("w8a8_static", M, K, N, qtype))
                else:
                    ws_need = max(ws_need, qlq.workspace_bytes(scheme, M, K, N, qtype))
    ws = torch.zeros(max(ws_need, 256), dtype=torch.uint8, device=dev)

    scheme_of = {v[0]: v[1] for v in VARIANTS + NEXT_VARIANTS}

    def chain(vname, M):
        scheme = scheme_of[vname]
        h = x0[M]
        i = 0
        P = len(synth.STACK_PROJS)
        if scheme == "w8a8_static_requant":            # the chain's input: one quantization pass
            K0 = synth.STACK_PROJS[0][1]
            xq = qlq.quantize_act_static(h, sx[0][0], "fp8_e4m3fn", out=cbuf[1][: M * K0].view(M, K0))
        for l in range(L):
            for p, (_, K, N) in enumerate(synth.STACK_PROJS):
                out = hbuf[i % 2][: M * N].view(M, N)
                qw = variants[vname][l][p]
                if scheme == "w8a16":
                    qlq.qlinear_w8a16(h, qw, out=out, workspace=ws)
                elif scheme == "w8a8_static_requant":
                    # this layer's epilogue writes the codes of its output at the next layer's scale
                    last = l == L - 1 and p == P - 1
                    if last:
                        qlq.qlinear_w8a8_static(xq, sx[l][p], qw, out=out, workspace=ws)
                    else:
                        nxt = sx[l][p + 1] if p + 1 < P else sx[l + 1][0]
                        _, xq = qlq.qlinear_w8a8_static_requant(xq, sx[l][p], qw, nxt, out=out,
                                                                out_codes=cbuf[i % 2][: M * N].view(M, N),
                                                                workspace=ws)
                elif scheme == "w8a8_static_fused":
                    qlq.qlinear_w8a8_static_fused(h, sx[l][p], qw, out=out, workspace=ws)
                elif scheme == "linear_routed":
                    qlq.linear("w8a8_dynamic", h, qw, bias=biases[l][p], bf16_fallback_max_m=32, out=out,
                               workspace=ws)
                else:
                    xq, xs = qlq.quantize_act_dynamic(h, "int8", out=xqbuf[: M * K].view(M, K), x_scale=sxbuf[:M])
                    qlq.qlinear_w8a8_dynamic(xq, xs, qw, out=out, workspace=ws)
                h = out
                i += 1
        return h

    # capture one graph per (variant, M)
    cases = [(v[0], M) for v in VARIANTS for M in Ms]
    next_cases = [] if args.only_step else [(v[0], M) for v in NEXT_VARIANTS for M in Ms]
    graphs = {}
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    for c in cases + next_cases:
        chain(*c)                                   # eager warm-up outside capture
    torch.cuda.synchronize()
    for c in cases + next_cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            chain(*c)
        graphs[c] = g
    torch.cuda.synchronize()
    log(f"[bench] captured {len(graphs)} graphs of {3 * L} GEMMs each")

    cur = torch.cuda.current_stream()
    ev = {c: [] for c in cases + next_cases}

    def step(timed, cases=cases):
        for c in cases:
            if timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(cur)
                graphs[c].replay()
                e1.record(cur)
                ev[c].append((e0, e1))
            else:
                graphs[c].replay()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # the widened rows, timed after the main region (not part of the step)
    if not args.only_step:
        for _ in range(args.warmup):
            step(False, next_cases)
        for _ in range(args.steps):
            step(True, next_cases)
    torch.cuda.synchronize()

    # per-case figures
    def figures(vlist, groups=None):
        res, flops_all = {}, 0
        for vname, scheme, qtype, gran in vlist:
            for M in Ms:
                us = sum(a.elapsed_time(b) for a, b in ev[(vname, M)]) * 1e3 / args.steps
                flops = sum(2 * M * N * K for _, K, N in synth.STACK_PROJS) * L
                byts = chain_bytes(scheme, M, synth.STACK_PROJS, L, gran == "per_tensor")
                dt = "bf16" if (scheme == "w8a16" or (scheme == "linear_routed" and M <= 32)) else \
                    ("fp8" if qtype == "fp8_e4m3fn" else "int8")
                t_hbm = byts / (HBM_PEAK_GBS * 1e9) * 1e6
                t_mfma = flops / (MFMA_PEAK_TFLOPS[dt] * 1e12) * 1e6
                flops_all += flops
                res[f"{vname}/M={M}"] = {
                    "us_per_stack": round(us, 2), "us_per_gemm": round(us / (3 * L), 3),
                    "tflops": round(flops / us / 1e6, 2), "gbs": round(byts / us / 1e3, 1),
                    "hbm_frac": round(t_hbm / us, 3), "mfma_frac": round(t_mfma / us, 3),
                    "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                    "frac": round(max(t_hbm, t_mfma) / us, 3)}
                if groups is not None:
                    fam = (vname, "small" if M <= 16 else "large")
                    g = groups.setdefault(fam, {"us": 0.0, "flops": 0, "bytes": 0, "launches": 0, "dt": dt})
                    g["us"] += us
                    g["flops"] += flops
                    g["bytes"] += byts
                    g["launches"] += 3 * L
        return res, flops_all

    groups = {}
    out_cases, tot_flops = figures(VARIANTS, groups)
    next_cases_out = {}
    if not args.only_step:
        next_cases_out, _ = figures(NEXT_VARIANTS)
        next_cases_out.update(kv_rows(qlq, torch, dev, KV_TOKENS, args.steps, args.warmup))
        next_cases_out.update(bucket_rows(qlq, synth, torch, dev, qi, L, args.steps, args.warmup))
        out_cases.update(single_gemm_rows(qlq, synth, torch, dev))
    # dominant kernel: the (variant, kernel family) group with the most time
    fam, g = max(groups.items(), key=lambda kv: kv[1]["us"])
    avg_us = g["us"] / g["launches"]
    t_hbm = g["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6
    t_mfma = g["flops"] / (MFMA_PEAK_TFLOPS[g["dt"]] * 1e12) * 1e6
    if t_mfma >= t_hbm:
        achieved = g["flops"] / g["launches"] / (avg_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS[g["dt"]],
                "unit": "TFLOP/s"}
    else:
        achieved = g["bytes"] / g["launches"] / (avg_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 3)
    roof["traffic"] = profiled_traffic(fam)
    roof["traffic_note"] = ("bytes between the L2s and the fabric per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "scaled by a 256 MiB device copy); the MALL can serve them, so an upper bound on HBM "
                            "bytes; profiles/traffic_gemm_mfma_int8_w8a16_stack.txt")
    roof["algorithmic_bytes_per_launch"] = int(g["bytes"] / g["launches"])
    kernel_name = {("int8_w8a16", "large"): "gemm_mfma_kernel<int8, W8A16, *> (M=256 and M=1024 launches)",
                   ("int8_w8a16", "small"): "gemm_small_kernel<int8, W8A16> (M=1 and M=16 launches)",
                   ("fp8_w8a8_static", "large"): "gemm_mfma_kernel<fp8, W8A8, *> + quant_act_kernel<fp8>",
                   ("fp8_w8a8_static", "small"): "gemm_small_kernel<fp8, W8A8, fused quantization>"}[fam]
    roof["kernel"] = kernel_name
    roof["avg_launch_us"] = round(avg_us, 3)
    roof["launches_per_step"] = g["launches"]

    value = tot_flops / (ms_per_step * 1e-3) / 1e12
    line = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp8", "data": "synthetic",
            "config": {"workload": f"3B-scale linear stack: {L} layers x {{q_proj 2048->2048, up_proj "
                                   f"2048->11008, down_proj 11008->2048}} chained; INT8 W8A16 and FP8 W8A8 "
                                   f"static (each epilogue also writes the next layer's activation codes); "
                                   f"M in {{1,16,256,1024}}; one HIP graph per chain",
                       "layers": L, "M": list(Ms), "variants": [v[0] for v in VARIANTS],
                       "gemms_per_step": 3 * L * len(cases)},
            "cases": out_cases, "roofline": roof,
            "next_rows": {"note": "INT8 W8A8 with dynamic per-token activation scales on the same stack, the "
                                  "routed Linear, the mixed K-int8/V-FP8 KV-cache codec (28 layers x 4 KV heads "
                                  "x 128), and the INT8 W8A16 stack through decode-batch graph buckets (M padded "
                                  "to 1, 2, 4, ..., 512); timed after the step, not part of value or ms_per_step",
                          "cases": next_cases_out}}
    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 256 MiB read + 256 MiB written")
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on its sample ...")
        lw = [[synth.stack_weight(args.seed, l, p, dev) for p in range(3)] for l in range(CPU_SAMPLE_LAYERS)]
        line["cpu_baseline"] = cpu_baseline(args.seed, lw, sx[:CPU_SAMPLE_LAYERS])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
