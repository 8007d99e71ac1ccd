"""Benchmark: the full Q8_0 decode weight sweep at M=1 on one MI355X.

One step = one pass of the decode hot path over one token: 145 GEMV launches
in dependency order on one stream (36 layers x {qkv 6144x2560, o 2560x4096,
gate_up 19456x2560, down 2560x9728}, then the LM head 151936x2560), Q8_0
weights (4.27 GB, all resident in HBM), bf16 activations, fp32 outputs.
Inputs are seeded and synthetic with the workload's shapes and distributions.

Printed: one JSON line with the achieved GB/s of the whole step (algorithmic
bytes / wall time per step, HIP events on the launch stream), the equivalent
decode tokens/s, a roofline object for the GEMV kernel (algorithmic bytes per
launch / mean launch duration) and the fp64 CPU oracle timed on a bounded
sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) for M=1 quant GEMV; equiv. decode tok/s"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q8_0_sweep_m1_traffic.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "q8_0_sweep_m1_kernel_trace.md")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", choices=["chain", "graph", "eager"], default="graph",
                    help="chain: one persistent kernel runs the 145 products in dependency order (grid barrier "
                         "between products); graph: the 145 launches replayed from one captured HIP graph; "
                         "eager: the 145 launches issued one by one")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-others", action="store_true",
                    help="c2: skip the other workloads (c0, c1, c3, c4) measured after the sweep")
    ap.add_argument("--no-events", action="store_true", help="skip the roofline / per-shape timing pass")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--workload", choices=["c2", "c2f", "c2n", "c0", "c1", "c3", "c4", "gemm", "stream", "kq"],
                    default="c2",
                    help="c2: the full Q8_0 decode sweep (the headline line); c2f: the same sweep with the decode "
                         "step's neighbours fused in (RMSNorm, SwiGLU, residual; qgemv_fused) next to the plain "
                         "sweep; c0/c1/c3/c4: the other workloads, each timed over >= 1 GiB of distinct weight "
                         "copies so the device-side cache cannot serve repeated reads; gemm: qgemm on the c3 "
                         "matrices at 16..128 tokens; stream: the read-only streaming ceiling over a 4 GiB buffer; "
                         "c2n: the c2 sweep through the NVFP4 decode cache (Q8_0 re-quantized at load); "
                         "kq: the c2 decode layer's matrices in Q4_K and Q6_K")
    ap.add_argument("--tokens", default="16,32,64,128",
                    help="gemm workload: the token counts to run (comma-separated, 1..128)")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def graph_time(torch, fn, reps):
    """Capture fn's launches in one HIP graph; return microseconds per replay."""
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def copies_for(nbytes):
    """Distinct weight copies so that one pass touches at least 1 GiB."""
    return max(2, -(-(1 << 30) // nbytes))


MFMA_FLOP = 2 * 16 * 16 * 32           # one v_mfma_f32_16x16x32_bf16
MFMA_BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16


def mfma_issued(fmt, n, k):
    """MFMA instructions one matrix-core launch issues: per 16-row unit and
    step, one per (row group, block)."""
    import block_quantized_weight_amd as q
    lo = q.layout(fmt, n, k)
    L, S, tiles = lo["lanes_per_row"], lo["steps"], lo["tiles"]
    tpw = L // 4 if L >= 8 else 1
    units = -(-tiles // tpw)
    per_step = L if L >= 4 else 4
    return units * S * per_step


def run_other(args, collect=None):
    """Per-launch throughput of the other workloads (one JSON line per case;
    with `collect` a list, the lines are appended to it instead of printed)."""
    import torch
    import block_quantized_weight_amd as q

    if not os.path.exists(q.LIB_PATH):
        from block_quantized_weight_amd import build as b
        b.build()
    q.lib()
    dev = torch.device("cuda:0")

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def packed_copies(fmt, canon, n, k, reps):
        pb = q.packed_bytes(fmt, n, k)
        buf = torch.empty(reps * pb, dtype=torch.uint8, device=dev)
        c = torch.from_numpy(canon.reshape(-1)).to(dev)
        for r in range(reps):
            q.pack(fmt, c, n, k, out=buf[r * pb:(r + 1) * pb])
        return [buf[r * pb:(r + 1) * pb] for r in range(reps)]

    def emit(name, gbs, us, extra):
        line = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                "config": {"workload": name}, "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        line.update(extra)
        if collect is not None:
            collect.append(line)
        else:
            print(json.dumps(line), flush=True)

    def dense_case(cfg, mats, xt, ms, label, fmt=None):
        """mats: [(name, n, k, matrix index)]; times each matrix and the whole set
        (fmt: the weight format, by default the config's)."""
        fmt = wl.CONFIGS[cfg]["fmt"] if fmt is None else fmt
        wsz = sum(q.packed_bytes(fmt, n, k) for _, n, k, _ in mats)
        reps = copies_for(wsz)
        ws = {}
        for name, n, k, j in mats:
            canon = wl.blocks_for(fmt, n, k, config=cfg, matrix=j)
            ws[name] = packed_copies(fmt, canon, n, k, reps)
        for m in ms:
            xs, ys, per = {}, {}, {}
            for name, n, k, j in mats:
                rng = wl.rng_for(cfg, j, "x")
                if xt == "f32":
                    xs[name] = torch.from_numpy(wl.x_f32((m, k), rng)).to(dev)
                else:
                    xs[name] = bf16_dev(wl.x_bf16_bits((m, k), rng))
                ys[name] = torch.empty((m, n), dtype=torch.float32, device=dev)
            xb = 4 if xt == "f32" else 2
            set_bytes = 0
            useful_flop = issued_flop = 0
            for name, n, k, j in mats:
                b = wl.canon_bytes(fmt, n, k) + m * k * xb + m * n * 4
                set_bytes += b
                path = q.dense_path(fmt, n, k, q.X_F32 if xt == "f32" else q.X_BF16, m)
                if path == q.PATH_MFMA:
                    useful_flop += 2 * m * n * k
                    issued_flop += mfma_issued(fmt, n, k) * MFMA_FLOP

                def one(name=name, n=n, k=k):
                    for r in range(reps):
                        q.qgemv(fmt, ws[name][r], n, k, xs[name], y=ys[name])
                us = graph_time(torch, one, max(2, args.steps // 3)) / reps
                per[name] = {"n": n, "k": k, "bytes": b, "us": round(us, 3), "gbs": round(b / us / 1e3, 1),
                             "path": {q.PATH_MFMA: "mfma", q.PATH_VALU_ONE: "valu_one"}.get(path, "valu")}

            def whole():
                for r in range(reps):
                    for name, n, k, j in mats:
                        q.qgemv(fmt, ws[name][r], n, k, xs[name], y=ys[name])
            us = graph_time(torch, whole, max(2, args.steps // 3)) / reps
            gbs = set_bytes / us / 1e3
            extra = {"per_matrix": per, "bytes_per_set": set_bytes, "tokens_per_s": round(m * 1e6 / us, 1),
                     "weight_copies": reps}
            if issued_flop:
                # matrix-core work of the set: algorithmic 2*m*n*k against the bf16 dense peak,
                # and what the MFMAs issue (16 token rows per instruction)
                extra["mfma"] = {"useful_tflops": round(useful_flop / us / 1e6, 2),
                                 "issued_tflops": round(issued_flop / us / 1e6, 2),
                                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                                 "frac": round(useful_flop / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 5)}
            emit(f"{label} m={m}", gbs, us, extra)

    def gemm_case(cfg, mats, ms, label):
        """qgemm on bf16 tokens: each matrix and the whole set per token count, against the
        same tokens as co-batch calls of 8 (qgemv)."""
        fmt = wl.CONFIGS[cfg]["fmt"]
        wsz = sum(q.packed_bytes(fmt, n, k) for _, n, k, _ in mats)
        reps = copies_for(wsz)
        ws = {}
        for name, n, k, j in mats:
            ws[name] = packed_copies(fmt, wl.blocks_for(fmt, n, k, config=cfg, matrix=j), n, k, reps)
        for m in ms:
            xs = {name: bf16_dev(wl.x_bf16_bits((m, k), wl.rng_for(cfg, j, "x"))) for name, n, k, j in mats}
            ys = {name: torch.empty((m, n), dtype=torch.float32, device=dev) for name, n, k, j in mats}
            set_bytes = sum(n * (k // 32) * wl.BLOCK_BYTES[fmt] + m * k * 2 + m * n * 4 for _, n, k, _ in mats)
            flop = sum(2 * m * n * k for _, n, k, _ in mats)
            per = {}
            for name, n, k, j in mats:
                def one(name=name, n=n, k=k):
                    for r in range(reps):
                        q.qgemm(fmt, ws[name][r], n, k, xs[name], y=ys[name])
                us = graph_time(torch, one, max(2, args.steps // 3)) / reps
                b = n * (k // 32) * wl.BLOCK_BYTES[fmt] + m * k * 2 + m * n * 4
                per[name] = {"n": n, "k": k, "us": round(us, 3), "gbs": round(b / us / 1e3, 1),
                             "tflops": round(2 * m * n * k / us / 1e6, 2),
                             "path": "mfma" if q.gemm_path(fmt, n, k, q.X_BF16, m) == q.PATH_MFMA else "valu"}

            def whole():
                for r in range(reps):
                    for name, n, k, j in mats:
                        q.qgemm(fmt, ws[name][r], n, k, xs[name], y=ys[name])

            def cobatch():
                for r in range(reps):
                    for name, n, k, j in mats:
                        for t0 in range(0, m, 8):
                            q.qgemv(fmt, ws[name][r], n, k, xs[name][t0:t0 + 8], y=ys[name][t0:t0 + 8])
            us = graph_time(torch, whole, max(2, args.steps // 3)) / reps
            us8 = graph_time(torch, cobatch, max(2, args.steps // 3)) / reps
            emit(f"{label} m={m}", set_bytes / us / 1e3, us,
                 {"per_matrix": per, "bytes_per_set": set_bytes, "tokens_per_s": round(m * 1e6 / us, 1),
                  "weight_copies": reps,
                  "mfma": {"useful_tflops": round(flop / us / 1e6, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                           "frac": round(flop / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 5)},
                  "as_cobatches_of_8": {"us": round(us8, 3), "tokens_per_s": round(m * 1e6 / us8, 1)}})

    if args.workload == "stream":
        # the achievable read rate: every byte of a 4 GiB buffer (16x the device cache) read once per pass
        nbytes = 4 << 30
        buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        sink = torch.empty(q.STREAM_SINK, dtype=torch.int32, device=dev)
        for _ in range(max(1, args.warmup)):
            q.read_stream(buf, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, args.steps)
        e0.record()
        for _ in range(reps):
            q.read_stream(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        emit("read-only stream, 4 GiB buffer, 16-byte nontemporal loads (qg_read_stream)", nbytes / us / 1e3, us,
             {"bytes_per_pass": nbytes, "passes": reps})
    elif args.workload == "gemm":
        gemm_case(3, [("qkv", 6144, 4096, 0), ("gate_up", 24576, 4096, 1), ("down", 4096, 12288, 2)],
                  [int(t) for t in args.tokens.split(",")],
                  "q4_0 qgemm, 8b-like: qkv 6144x4096 + gate_up 24576x4096 + down 4096x12288")
    elif args.workload == "kq":
        # the decode layer of the full sweep's shapes in the K-quant formats
        layer = [(nm, n, k, j) for j, (nm, n, k) in enumerate(wl.configs.C2_LAYER_MATS)]
        for fmt, fname in ((q.Q4_K, "q4_k"), (q.Q6_K, "q6_k")):
            dense_case(2, layer, "bf16", [1], f"{fname} decode layer: qkv 6144x2560 + o 2560x4096 + gate_up "
                       "19456x2560 + down 2560x9728, x bf16", fmt=fmt)
    elif args.workload == "c0":
        dense_case(0, [("w", 2048, 2048, 0)], "f32", [1], "q8_0 2048x2048, x fp32")
    elif args.workload == "c1":
        dense_case(1, [("gate_up", 19456, 2560, 0), ("down", 2560, 9728, 1)], "bf16", [1],
                   "q4_0 qwen3-4b-like layer: gate_up 19456x2560 + down 2560x9728, x bf16")
    elif args.workload == "c3":
        dense_case(3, [("qkv", 6144, 4096, 0), ("gate_up", 24576, 4096, 1), ("down", 4096, 12288, 2)], "bf16",
                   [2, 4, 8], "q4_0 co-batch, 8b-like: qkv 6144x4096 + gate_up 24576x4096 + down 4096x12288")
    elif args.workload == "c4":
        c = wl.CONFIGS[4]
        fmt, E, top_k = q.MXFP4, c["n_experts"], c["top_k"]
        (gn, gk), (dn, dk) = (3584, 2048), (2048, 1792)
        gpb, dpb = q.packed_bytes(fmt, gn, gk), q.packed_bytes(fmt, dn, dk)
        reps = copies_for(E * (gpb + dpb))
        ge = torch.empty(reps * E * gpb, dtype=torch.uint8, device=dev)
        de = torch.empty(reps * E * dpb, dtype=torch.uint8, device=dev)
        for e in range(E):
            gc = torch.from_numpy(wl.blocks_for(fmt, gn, gk, config=4, matrix=2 * e).reshape(-1)).to(dev)
            dc = torch.from_numpy(wl.blocks_for(fmt, dn, dk, config=4, matrix=2 * e + 1).reshape(-1)).to(dev)
            for r in range(reps):
                q.pack(fmt, gc, gn, gk, out=ge[(r * E + e) * gpb:(r * E + e + 1) * gpb])
                q.pack(fmt, dc, dn, dk, out=de[(r * E + e) * dpb:(r * E + e + 1) * dpb])
        for m in (1, 4):
            logits, ids, g = wl.router_topk(m, E, top_k, wl.rng_for(4, m, "router"))
            distinct = len(set(ids.reshape(-1).tolist()))
            tid, tw = torch.from_numpy(ids).to(dev), torch.from_numpy(g).to(dev)
            lg = torch.from_numpy(logits).to(dev)
            rid = torch.empty_like(tid)
            rw = torch.empty_like(tw)
            x = bf16_dev(wl.x_bf16_bits((m, gk), wl.rng_for(4, m, "x")))
            h = bf16_dev(wl.x_bf16_bits((m, top_k, dk), wl.rng_for(4, m, "h")))
            yg = torch.empty((m, top_k, gn), dtype=torch.float32, device=dev)
            yd = torch.empty((m, dn), dtype=torch.float32, device=dev)
            gbytes = distinct * gn * (gk // 32) * 17 + m * gk * 2 + m * top_k * gn * 4 + m * top_k * 8
            dbytes = distinct * dn * (dk // 32) * 17 + m * top_k * dk * 2 + m * dn * 4 + m * top_k * 8
            per = {}

            def gate(r):
                q.moe_qgemv_topk(fmt, ge[r * E * gpb:(r + 1) * E * gpb], E, gn, gk, tid, tw, x, q.MOE_GATE_UP, y=yg)

            def down(r):
                q.moe_qgemv_topk(fmt, de[r * E * dpb:(r + 1) * E * dpb], E, dn, dk, tid, tw, h, q.MOE_DOWN_COMBINE,
                                 y=yd)
            for nm, f, b in (("gate_up", gate, gbytes), ("down_combine", down, dbytes)):
                us = graph_time(torch, lambda f=f: [f(r) for r in range(reps)], max(2, args.steps // 3)) / reps
                per[nm] = {"bytes": b, "us": round(us, 3), "gbs": round(b / us / 1e3, 1)}
            us = graph_time(torch, lambda: [(gate(r), down(r)) for r in range(reps)], max(2, args.steps // 3)) / reps

            # the device router (top-k + softmax of the logits), alone and in front of the two products
            def route():
                q.moe_router_topk(lg, top_k, ids=rid, weights=rw)
            rus = graph_time(torch, lambda: [route() for _ in range(reps)], max(2, args.steps // 3)) / reps
            wus = graph_time(torch, lambda: [(route(), gate(r), down(r)) for r in range(reps)],
                             max(2, args.steps // 3)) / reps
            per["router"] = {"us": round(rus, 3)}

            # the expert FFN fused (moe_qgemv_topk_fused): fp32 hidden state ->
            # gate_up with RMSNorm + SwiGLU -> bf16 -> down-combine + residual (in place)
            hid = torch.from_numpy(wl.x_f32((m, gk), wl.rng_for(4, m, "x"))).to(dev)
            gam = torch.from_numpy(wl.norm_weight_f32(gk, wl.rng_for(4, m, "gamma"))).to(dev)
            act = torch.empty((m, top_k, gn // 2), dtype=torch.bfloat16, device=dev)

            def fgate(r):
                q.moe_qgemv_topk_fused(fmt, ge[r * E * gpb:(r + 1) * E * gpb], E, gn, gk, tid, tw, hid, q.MOE_GATE_UP,
                                       norm_weight=gam, eps=1e-6, act=q.ACT_SWIGLU, y=act)

            def fdown(r):
                q.moe_qgemv_topk_fused(fmt, de[r * E * dpb:(r + 1) * E * dpb], E, dn, dk, tid, tw, act,
                                       q.MOE_DOWN_COMBINE, residual=hid, y=hid)
            fg_bytes = distinct * gn * (gk // 32) * 17 + m * gk * 4 + gk * 4 + m * top_k * (gn // 2) * 2 + m * top_k * 8
            fd_bytes = distinct * dn * (dk // 32) * 17 + m * top_k * dk * 2 + 2 * m * dn * 4 + m * top_k * 8
            fused = {}
            for nm, f, b in (("gate_up_norm_swiglu", fgate, fg_bytes), ("down_combine_residual", fdown, fd_bytes)):
                fu = graph_time(torch, lambda f=f: [f(r) for r in range(reps)], max(2, args.steps // 3)) / reps
                fused[nm] = {"bytes": b, "us": round(fu, 3), "gbs": round(b / fu / 1e3, 1)}
            fused["router_and_both"] = {"us": round(graph_time(torch, lambda: [(route(), fgate(r), fdown(r))
                                                                              for r in range(reps)],
                                                               max(2, args.steps // 3)) / reps, 3)}
            emit(f"mxfp4 moe 32 experts top-4: gate_up 3584x2048 + down 2048x1792 m={m}", (gbytes + dbytes) / us / 1e3,
                 us, {"per_mode": per, "distinct_experts": distinct, "bytes_per_set": gbytes + dbytes,
                      "weight_copies": reps, "us_with_device_router": round(wus, 3), "fused_ffn": fused})
    if args.calib_copy_mib:
        # a device copy of known size, for scaling the HBM byte counters of the same run
        nb = args.calib_copy_mib << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest():
    """sha256 over the HIP sources and the build script (its compiler flags):
    ties recorded counter values to a kernel version."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_weight_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "block_quantized_weight_amd", "build.py"), "rb") as fh:
        h.update(b"build.py" + fh.read())
    return h.hexdigest()[:16]


def recorded_profile(path, key):
    """A figure recorded in a committed rocprofv3 summary for the current
    kernel sources (its source_digest line must match), or None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_val = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != source_digest():
        return None
    return float(m_val.group(1))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_fused_sweep(args, torch, q, dev, shapes, wviews, xs, ys, fmt, config):
    """The decode sweep with its neighbours fused in, against the plain sweep.

    Dataflow per layer (attention itself is not part of the path; its output
    is a fixed synthetic bf16 vector per layer):
        qkv     = W_qkv RMSNorm(h)                        (fp32 out)
        h       = W_o attn + h                            (residual, in place)
        a       = SwiGLU(W_gate_up RMSNorm(h))            (bf16 out, F = 9728)
        h       = W_down a + h                            (residual, in place)
    then logits = W_lm RMSNorm(h).  h is the fp32 hidden state (2560).
    Algorithmic bytes per launch: weights + activations read + norm weights +
    residual read + outputs written."""
    hidden = 2560
    h = torch.from_numpy(wl.x_f32((1, hidden), wl.rng_for(config, 200, "x"))).to(dev)
    a = torch.empty((1, 9728), dtype=torch.bfloat16, device=dev)
    calls, alg = [], []
    for i, (j, name, n, k) in enumerate(shapes):
        kind = name.split(".")[-1]
        wb = n * (k // 32) * 34
        if kind in ("qkv", "gate_up", "lm_head"):
            g = torch.from_numpy(wl.norm_weight_f32(k, wl.rng_for(config, j, "gamma"))).to(dev)
            if kind == "gate_up":
                calls.append(dict(i=i, x=h, norm_weight=g, act=q.ACT_SWIGLU, residual=None, y=a))
                alg.append(wb + 4 * k + 4 * k + 2 * (n // 2))
            else:
                calls.append(dict(i=i, x=h, norm_weight=g, act=q.ACT_NONE, residual=None, y=ys[i]))
                alg.append(wb + 4 * k + 4 * k + 4 * n)
        else:
            x = xs[i] if kind == "o" else a
            calls.append(dict(i=i, x=x, norm_weight=None, act=q.ACT_NONE, residual=h, y=h))
            alg.append(wb + 2 * k + 4 * n + 4 * n)
    plain_alg = [n * (k // 32) * 34 + 2 * k + 4 * n for (_, _, n, k) in shapes]

    def fused(idx=None):
        for c in calls if idx is None else [calls[t] for t in idx]:
            _, _, n, k = shapes[c["i"]]
            q.qgemv_fused(fmt, wviews[c["i"]], n, k, c["x"], norm_weight=c["norm_weight"], eps=1e-6,
                          act=c["act"], residual=c["residual"], y=c["y"])

    def plain(idx=None):
        for i in range(len(shapes)) if idx is None else idx:
            _, _, n, k = shapes[i]
            q.qgemv(fmt, wviews[i], n, k, xs[i], y=ys[i])

    # the same dataflow unfused, for comparison only: the plain products with
    # the norm, gate and residual steps done by separate torch kernels
    # (bf16 copies of the normalised activations feed the plain products)
    gam = {c["i"]: c["norm_weight"] for c in calls if c["norm_weight"] is not None}
    xb = {i: torch.empty((1, k), dtype=torch.bfloat16, device=dev) for i, (_, _, n, k) in enumerate(shapes)}
    gu_out = torch.empty((1, 19456), dtype=torch.float32, device=dev)

    def unfused():
        for i, (_, name, n, k) in enumerate(shapes):
            kind = name.split(".")[-1]
            if kind in ("qkv", "gate_up", "lm_head"):
                xb[i].copy_(torch.nn.functional.rms_norm(h, (k,), gam[i], 1e-6))
                if kind == "gate_up":
                    q.qgemv(fmt, wviews[i], n, k, xb[i], y=gu_out)
                    a.copy_(torch.nn.functional.silu(gu_out[:, : n // 2]) * gu_out[:, n // 2:])
                else:
                    q.qgemv(fmt, wviews[i], n, k, xb[i], y=ys[i])
            else:
                q.qgemv(fmt, wviews[i], n, k, xs[i] if kind == "o" else a, y=ys[i])
                h.add_(ys[i])

    reps = max(1, args.steps)
    us_f = graph_time(torch, fused, reps)
    us_p = graph_time(torch, plain, reps)
    us_u = graph_time(torch, unfused, reps)
    log(args, f"unfused (plain products + torch norm / SwiGLU / add kernels) {us_u:.1f} us")
    fb, pb = sum(alg), sum(plain_alg)
    log(args, f"fused sweep {us_f:.1f} us ({fb / us_f / 1e3:.1f} GB/s); plain {us_p:.1f} us ({pb / us_p / 1e3:.1f} GB/s)")
    groups = {}
    for i, (_, name, n, k) in enumerate(shapes):
        groups.setdefault(name.split(".")[-1], []).append(i)
    per_shape = {}
    for key, idx in groups.items():
        uf = graph_time(torch, lambda idx=idx: fused(idx), 5) / len(idx)
        up = graph_time(torch, lambda idx=idx: plain(idx), 5) / len(idx)
        _, _, n, k = shapes[idx[0]]
        per_shape[key] = {"n": n, "k": k, "fused": {"bytes": alg[idx[0]], "us": round(uf, 3),
                                                    "gbs": round(alg[idx[0]] / uf / 1e3, 1)},
                          "plain": {"bytes": plain_alg[idx[0]], "us": round(up, 3),
                                    "gbs": round(plain_alg[idx[0]] / up / 1e3, 1)}}
    log(args, f"per shape {per_shape}")
    out = {
        "metric": METRIC, "value": round(fb / us_f / 1e3, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": reps, "warmup": args.warmup, "ms_per_step": round(us_f * 1e-3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "q8_0 full decode sweep with RMSNorm / SwiGLU / residual fused (qgemv_fused), "
                               "M=1: 36 x {qkv+norm, o+residual, gate_up+norm+SwiGLU->bf16, down+residual} "
                               "+ lm_head+norm", "launches_per_step": len(shapes), "bytes_per_step": fb},
        "pct_of_peak": round(100.0 * fb / us_f / 1e3 / HBM_PEAK_GBS, 2),
        "equiv_decode_tok_s": round(1e6 / us_f, 1),
        "plain_sweep": {"us": round(us_p, 1), "gbs": round(pb / us_p / 1e3, 1), "bytes": pb},
        "fused_over_plain_time": round(us_f / us_p, 4),
        "unfused_sweep": {"us": round(us_u, 1), "what": "plain products + torch rms_norm / silu*mul / add "
                                                        "kernels between them, one graph"},
        "fused_over_unfused_time": round(us_f / us_u, 4),
        "per_shape": per_shape,
    }
    print(json.dumps(out), flush=True)


def run_nvfp4_sweep(args, torch, q, dev, shapes, config):
    """The decode sweep through the NVFP4 decode cache: every Q8_0 matrix of
    the sweep re-quantized to NVFP4 at load time (qg_requant_q8_0_nvfp4), then
    the 145 products on the NVFP4 copy (qgemv_nvfp4), one graph.  Reports the
    NVFP4 bytes streamed, and, on a sample, the product's parity with the
    oracle of the NVFP4 tensor and its deviation from the Q8_0 product."""
    import oracle
    fmt = q.NVFP4
    offs, total = [], 0
    for (_, _, n, k) in shapes:
        offs.append(total)
        total += q.packed_bytes(fmt, n, k)
    nvbuf = torch.empty(total, dtype=torch.uint8, device=dev)
    xs, ys = [], []
    t0 = time.time()
    t_req = 0.0
    def gen(item):
        j, _, n, k = item
        return wl.blocks_for(q.Q8_0, n, k, config=config, matrix=j)

    with ThreadPoolExecutor(max_workers=8) as ex:
        for base in range(0, len(shapes), 16):
            chunk = shapes[base:base + 16]
            for i, blocks in enumerate(ex.map(gen, chunk)):
                j, _, n, k = chunk[i]
                idx = base + i
                canon = torch.from_numpy(blocks.reshape(-1)).to(dev)
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                q.requant_q8_0_nvfp4(canon, n, k, out=nvbuf[offs[idx]:offs[idx] + q.packed_bytes(fmt, n, k)])
                torch.cuda.synchronize()
                t_req += time.perf_counter() - t1
                del canon
                xb = wl.x_bf16_bits((1, k), wl.rng_for(config, j, "x"))
                xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16))
                ys.append(torch.empty((1, n), dtype=torch.float32, device=dev))
    log(args, f"decode cache built in {time.time() - t0:.1f} s ({t_req * 1e3:.1f} ms of re-quantization kernels)")
    wv = [nvbuf[offs[i]:offs[i] + q.packed_bytes(fmt, n, k)] for i, (_, _, n, k) in enumerate(shapes)]
    alg = [n * (k // 32) * 18 + 2 * k + 4 * n for (_, _, n, k) in shapes]

    def sweep(idx=None):
        for i in range(len(shapes)) if idx is None else idx:
            _, _, n, k = shapes[i]
            q.qgemv(fmt, wv[i], n, k, xs[i], y=ys[i])

    us = graph_time(torch, sweep, max(1, args.steps))
    gbs = sum(alg) / us / 1e3
    groups = {}
    for i, (_, name, n, k) in enumerate(shapes):
        groups.setdefault(name.split(".")[-1], []).append(i)
    per_shape = {}
    for key, idx in groups.items():
        u = graph_time(torch, lambda idx=idx: sweep(idx), 5) / len(idx)
        _, _, n, k = shapes[idx[0]]
        per_shape[key] = {"n": n, "k": k, "bytes": alg[idx[0]], "us": round(u, 3), "gbs": round(alg[idx[0]] / u / 1e3, 1)}
    # sample: layer 0's four matrices in full and every 9th LM-head row
    sweep()
    torch.cuda.synchronize()
    parity, deviation = 0.0, 0.0
    for i, rows in [(0, None), (1, None), (2, None), (3, None), (144, np.arange(0, 151936, 9))]:
        j, name, n, k = shapes[i]
        nv = q.unpack(fmt, wv[i], n, k).cpu().numpy()
        xb = wl.x_bf16_bits((1, k), wl.rng_for(config, j, "x"))
        yg = ys[i].cpu().numpy()
        yg = yg if rows is None else yg[:, rows]
        ref, l1 = oracle.gemv(oracle.NVFP4, nv, n, k, xb, oracle.X_BF16, rows=rows)
        parity = max(parity, oracle.max_rel_err(yg, ref, l1))
        canon8 = wl.blocks_for(q.Q8_0, n, k, config=config, matrix=j)
        ref8, l18 = oracle.gemv(oracle.Q8_0, canon8, n, k, xb, oracle.X_BF16, rows=rows)
        deviation = max(deviation, oracle.max_rel_err(yg, ref8, l18))
    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "q8_0 full decode sweep through the NVFP4 decode cache (re-quantized at load), M=1: "
                               "36 x {qkv 6144x2560, o 2560x4096, gate_up 19456x2560, down 2560x9728} + lm_head "
                               "151936x2560; bf16 x, fp32 y", "launches_per_step": len(shapes),
                   "bytes_per_step": sum(alg)},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "equiv_decode_tok_s": round(1e6 / us, 1),
        "per_shape": per_shape,
        "requant_ms": round(t_req * 1e3, 2),
        "parity_max_rel_err_vs_nvfp4_oracle": parity,
        "deviation_max_rel_err_vs_q8_0_oracle": deviation,
        "sample": "layer 0 (qkv, o, gate_up, down) in full + every 9th LM-head row",
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded design is described but not run)", file=sys.stderr)
        sys.exit(2)
    if args.workload not in ("c2", "c2f", "c2n"):
        run_other(args)
        return

    import torch
    import block_quantized_weight_amd as q

    if not os.path.exists(q.LIB_PATH):
        from block_quantized_weight_amd import build as b
        b.build()
    q.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    shapes = wl.c2_sweep_shapes()
    fmt, config = q.Q8_0, 2
    if args.workload == "c2n":
        run_nvfp4_sweep(args, torch, q, dev, shapes, config)
        return
    offs, total = [], 0
    for (_, _, n, k) in shapes:
        offs.append(total)
        total += q.packed_bytes(fmt, n, k)
    log(args, f"sweep: {len(shapes)} matrices, {total / 1e9:.3f} GB packed")

    # ---- resident inputs: packed weights, activations, outputs
    t0 = time.time()
    wbuf = torch.empty(total, dtype=torch.uint8, device=dev)
    xs, ys = [], []

    def gen(item):
        j, name, n, k = item
        return wl.blocks_for(fmt, n, k, config=config, matrix=j)

    with ThreadPoolExecutor(max_workers=8) as ex:
        for base in range(0, len(shapes), 16):
            chunk = shapes[base:base + 16]
            for i, canon in enumerate(ex.map(gen, chunk)):
                j, name, n, k = chunk[i]
                idx = base + i
                c = torch.from_numpy(canon.reshape(-1)).to(dev)
                q.pack(fmt, c, n, k, out=wbuf[offs[idx]:offs[idx] + q.packed_bytes(fmt, n, k)])
                xb = wl.x_bf16_bits((1, k), wl.rng_for(config, j, "x"))
                xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16))
                ys.append(torch.empty((1, n), dtype=torch.float32, device=dev))
                del c
    torch.cuda.synchronize()
    log(args, f"inputs generated, packed and resident in {time.time() - t0:.1f} s")

    wviews = [wbuf[offs[i]:offs[i] + q.packed_bytes(fmt, n, k)] for i, (_, _, n, k) in enumerate(shapes)]
    if args.workload == "c2f":
        run_fused_sweep(args, torch, q, dev, shapes, wviews, xs, ys, fmt, config)
        return
    # algorithmic bytes: canonical weights + x (bf16) + y (fp32)
    alg = [n * (k // 32) * 34 + 2 * k + 4 * n for (_, _, n, k) in shapes]
    step_bytes = sum(alg)

    def step_launches():
        for i, (_, _, n, k) in enumerate(shapes):
            q.qgemv(fmt, wviews[i], n, k, xs[i], y=ys[i])

    chain = None
    if args.mode == "chain":
        chain = q.Chain(fmt, [(wviews[i], n, k, xs[i], ys[i]) for i, (_, _, n, k) in enumerate(shapes)])

    def step():
        if chain is not None:
            chain.run()
        else:
            step_launches()

    stream = torch.cuda.current_stream()
    for _ in range(2):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.mode == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step()
        stream.wait_stream(side)
        torch.cuda.synchronize()

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    log(args, f"{args.mode}: {ms_step * 1e3:.1f} us/step, {gbs:.1f} GB/s, {1e3 / ms_step:.1f} tok/s")
    if chain is not None and q.chain_error() != 0:
        raise RuntimeError("a chain barrier timed out: the timed run is invalid")

    # the same 145 launches issued one by one from the host (no graph), for comparison
    eager_us = None
    if args.mode != "eager" and not args.no_events:
        for _ in range(2):
            step_launches()
        torch.cuda.synchronize()
        reps = max(3, args.steps // 3)
        e0.record(stream)
        for _ in range(reps):
            step_launches()
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_time(e1) * 1e3 / reps
        log(args, f"eager launches: {eager_us:.1f} us/step")

    # ---- roofline of the GEMV kernel.  Every launch of the step is the vector
    # GEMV (Q8_0, bf16 x, M=1: o in its one-batch form k_dense_one, the other
    # shapes in k_dense); its mean launch duration is the graph step time over
    # the 145 launches (the rocprofv3 kernel-trace average agrees to within the
    # ~0.2 us gaps between graph nodes).  Per-shape durations come from one
    # graph of the 36 distinct matrices of each shape (144 for the LM head, which
    # is timed alone).
    roof = None
    per_shape = {}
    if not args.no_events:
        mean_dur = ms_step * 1e-3 / len(shapes)
        mean_bytes = step_bytes / len(shapes)
        achieved = mean_bytes / mean_dur / 1e9
        traffic = recorded_profile(TRAFFIC_FILE, "hbm_bytes_per_launch")
        trace_us = recorded_profile(TRACE_FILE, "mean_gemv_us")
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "qg::k_dense / k_dense_one<Q8_0, bf16 x, M=1>" if args.mode != "chain"
                          else "qg::k_chain<Q8_0, bf16 x, M=1>",
                "bytes_per_launch": round(mean_bytes), "mean_launch_us": round(mean_dur * 1e6, 3),
                "basis": {
                    "achieved": "algorithmic bytes per product / (timed region on the launch stream, HIP events, "
                                "/ products per step); includes the gaps between graph nodes" if args.mode != "chain"
                                else "algorithmic bytes per product / (timed region / products per step) of the "
                                     "one persistent launch",
                    "traffic": "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, scaled by a device copy of known "
                               "size, recorded in " + os.path.relpath(TRAFFIC_FILE, ROOT) +
                               " for these kernel sources (null if the sources changed since)",
                    "trace_mean_gemv_us": trace_us,
                    "trace_source": os.path.relpath(TRACE_FILE, ROOT)}}
        sink = torch.empty(q.STREAM_SINK, dtype=torch.int32, device=dev)
        groups = {}
        for i, (_, name, n, k) in enumerate(shapes):
            groups.setdefault(name.split(".")[-1], []).append(i)
        for key, idx in groups.items():
            def launches(idx=idx):
                for i in idx:
                    _, _, n, k = shapes[i]
                    q.qgemv(fmt, wviews[i], n, k, xs[i], y=ys[i])
            us = graph_time(torch, launches, 5) / len(idx)

            def reads(idx=idx):
                for i in idx:
                    q.read_stream(wviews[i], sink)
            rus = graph_time(torch, reads, 5) / len(idx)
            _, _, n, k = shapes[idx[0]]
            per_shape[key] = {"n": n, "k": k, "bytes": alg[idx[0]], "us": round(us, 3),
                              "gbs": round(alg[idx[0]] / us / 1e3, 1), "launches": len(idx),
                              "read_only_us": round(rus, 3)}
        roof["basis"]["per_shape_sum_us"] = round(sum(v["us"] * v["launches"] for v in per_shape.values()), 1)
        log(args, f"roofline {roof}; per shape {per_shape}")

        # The same 145 launches as plain reads of the same bytes (qg_read_stream over each
        # matrix's packed weights, one graph): what this launch structure allows a kernel that
        # only streams; and the launch floor alone (the same call over 256 bytes).
        tiny = wbuf[:256]

        def read_launches():
            for i in range(len(shapes)):
                q.read_stream(wviews[i], sink)

        def empty_launches():
            for _ in range(len(shapes)):
                q.read_stream(tiny, sink)
        reps = max(3, args.steps // 3)
        read_us = graph_time(torch, read_launches, reps)
        floor_us = graph_time(torch, empty_launches, reps) / len(shapes)
        packed_total = sum(q.packed_bytes(fmt, n, k) for (_, _, n, k) in shapes)
        read_sweep = {"us": round(read_us, 1), "gbs": round(packed_total / read_us / 1e3, 1),
                      "gemv_step_over_read_step": round(ms_step * 1e3 / read_us, 4),
                      "launch_floor_us": round(floor_us, 3),
                      "kernel": "qg_read_stream (16-byte nontemporal loads, every byte once)"}
        roof["same_launches_read_only"] = read_sweep
        log(args, f"read-only sweep of the same launches: {read_sweep}")

    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(args, f"calibration copy of {nb} bytes done")

    # ---- the other workloads, measured in the same run (same code as --workload c0/c1/c3/c4)
    others = None
    if not args.no_events and not args.no_others:
        lines = []
        for wk in ("c0", "c1", "c3", "c4"):
            sub = argparse.Namespace(**vars(args))
            sub.workload, sub.calib_copy_mib = wk, 0
            run_other(sub, collect=lines)
        others = {}
        for ln in lines:
            e = {"us": round(ln["ms_per_step"] * 1e3, 3), "gbs": ln["value"], "pct_of_peak": ln["pct_of_peak"]}
            for key in ("per_matrix", "per_mode"):
                if key in ln:
                    e[key] = {nm: {f: v[f] for f in ("us", "gbs", "path") if f in v} for nm, v in ln[key].items()}
            others[ln["config"]["workload"]] = e
        log(args, f"other workloads: {others}")

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        import oracle
        lm_rows = np.arange(0, 151936, 9)
        sample = [(shapes[i], None) for i in range(40)] + [(shapes[144], lm_rows)]
        t_cpu, bytes_cpu, worst = 0.0, 0, 0.0
        for (j, name, n, k), rows in sample:
            canon = wl.blocks_for(fmt, n, k, config=config, matrix=j)
            xb = wl.x_bf16_bits((1, k), wl.rng_for(config, j, "x"))
            t1 = time.perf_counter()
            yref, l1 = oracle.gemv(fmt, canon, n, k, xb, oracle.X_BF16, rows=rows)
            t_cpu += time.perf_counter() - t1
            nr = n if rows is None else len(rows)
            bytes_cpu += nr * (k // 32) * 34 + 2 * k + 4 * nr
            idx = [s[0] for s in shapes].index(j)
            yg = ys[idx].cpu().numpy()
            yg = yg if rows is None else yg[:, rows]
            worst = max(worst, oracle.max_rel_err(yg, yref, l1))
        cores = oracle.threads()
        # one core: the oracle on the Q8_0 2048x2048 (fp32 x) and Q4_0 2560x9728 (bf16 x) workloads
        one = {}
        oracle.set_threads(1)
        try:
            for name, cfg, f, n, k, xt in (("q8_0 2048x2048 fp32 x", 0, q.Q8_0, 2048, 2048, oracle.X_F32),
                                           ("q4_0 2560x9728 bf16 x", 1, q.Q4_0, 2560, 9728, oracle.X_BF16)):
                canon = wl.blocks_for(f, n, k, config=cfg, matrix=0 if cfg == 0 else 1)
                rng = wl.rng_for(cfg, 0 if cfg == 0 else 1, "x")
                xv = wl.x_f32((1, k), rng) if xt == oracle.X_F32 else wl.x_bf16_bits((1, k), rng)
                t1 = time.perf_counter()
                oracle.gemv(f, canon, n, k, xv, xt)
                dt = time.perf_counter() - t1
                b = n * (k // 32) * wl.BLOCK_BYTES[f] + k * (4 if xt == oracle.X_F32 else 2) + 4 * n
                one[name] = {"s": round(dt, 4), "gbs": round(b / dt / 1e9, 4)}
        finally:
            oracle.set_threads(cores)
        cpu = {"value": round(bytes_cpu / t_cpu / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": "layers 0-9 (qkv, o, gate_up, down) in full + every 9th LM-head row; "
                         f"{bytes_cpu / 1e6:.1f} MB of the sweep's algorithmic bytes, {t_cpu:.1f} s wall",
               "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
               "one_core": one,
               "gpu_vs_oracle_max_rel_err": worst}
        log(args, f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "q8_0 full decode weight sweep, M=1: 36 x {qkv 6144x2560, o 2560x4096, "
                               "gate_up 19456x2560, down 2560x9728} + lm_head 151936x2560; bf16 x, fp32 y",
                   "launches_per_step": len(shapes), "bytes_per_step": step_bytes, "mode": args.mode},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "equiv_decode_tok_s": round(1e3 / ms_step, 1),
        "roofline": roof,
        "eager_us_per_step": None if eager_us is None else round(eager_us, 1),
        "per_shape": per_shape or None,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
