"""Benchmark: the full Q8_0 decode weight sweep at M=1 on one MI355X.

One step = one pass of the decode hot path over one token: 145 GEMV launches
in dependency order on one stream (36 layers x {qkv 6144x2560, o 2560x4096,
gate_up 19456x2560, down 2560x9728}, then the LM head 151936x2560), Q8_0
weights (4.27 GB, all resident in HBM), bf16 activations, fp32 outputs.
Inputs are seeded and synthetic with the workload's shapes and distributions.

Printed: one JSON line with the achieved GB/s of the whole step (algorithmic
bytes / wall time per step), the equivalent decode tokens/s, a roofline object
for the GEMV kernel (algorithmic bytes per launch / mean launch duration from
HIP events around each launch) and the fp64 CPU oracle timed on a bounded
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
    ap.add_argument("--no-events", action="store_true", help="skip the per-launch event pass")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest():
    """sha256 over the HIP sources: ties recorded counter values to a kernel version."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_quantized_weight_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Measured HBM bytes per launch for the current kernel sources, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != source_digest():
        return None
    return float(m_val.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sharded design is described but not run)", file=sys.stderr)
        sys.exit(2)

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

    # ---- per-launch durations (HIP events around every launch, eager, same stream)
    roof = None
    per_shape = {}
    if not args.no_events:
        reps = 3
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in shapes]
        durs = np.zeros((reps, len(shapes)))
        for r in range(reps):
            for i, (_, _, n, k) in enumerate(shapes):
                ev[i][0].record(stream)
                q.qgemv(fmt, wviews[i], n, k, xs[i], y=ys[i])
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            for i in range(len(shapes)):
                durs[r, i] = ev[i][0].elapsed_time(ev[i][1]) * 1e-3
        mean_dur = float(durs.mean())
        mean_bytes = step_bytes / len(shapes)
        achieved = mean_bytes / mean_dur / 1e9
        traffic = recorded_traffic()
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "qg::k_dense<Q8_0, bf16 x, M=1>",
                "bytes_per_launch": round(mean_bytes), "mean_launch_us": round(mean_dur * 1e6, 3)}
        for i, (_, name, n, k) in enumerate(shapes):
            key = name.split(".")[-1]
            d = per_shape.setdefault(key, {"n": n, "k": k, "bytes": alg[i], "us": []})
            d["us"].extend(list(durs[:, i] * 1e6))
        for key, d in per_shape.items():
            us = float(np.mean(d.pop("us")))
            d["us"] = round(us, 3)
            d["gbs"] = round(d["bytes"] / (us * 1e-6) / 1e9, 1)
        log(args, f"events: mean launch {mean_dur * 1e6:.2f} us, {achieved:.1f} GB/s per launch; {per_shape}")

    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(args, f"calibration copy of {nb} bytes done")

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        import oracle
        lm_rows = np.arange(0, 151936, 37)[:4096]
        sample = [(shapes[i], None) for i in range(4)] + [(shapes[144], lm_rows)]
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
        cpu = {"value": round(bytes_cpu / t_cpu / 1e9, 4), "unit": "GB/s", "cores": oracle.threads(),
               "kind": "oracle",
               "sample": "layer-0 qkv, o, gate_up, down in full + 4096 LM-head rows (every 37th); "
                         f"{bytes_cpu / 1e6:.1f} MB of the sweep's algorithmic bytes, {t_cpu:.1f} s wall",
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
        "per_shape": per_shape or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
