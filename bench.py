"""Decode-throughput benchmark of the quantized matvec path on one MI355X.

One step = one decode token through the Llama-3-8B-shaped stack: 32 layers,
hidden 4096, each layer = rmsnorm+QKV matvec (4096->6144), O matvec
(4096->4096, + residual), rmsnorm + gate.up SwiGLU (4096->14336 x2), down
matvec (14336->4096, + residual); 4-bit codes, group 64, fp16 scale + bias,
fp32 activations; the attention output is stood in by the q-slice of the QKV
output. Weights are seeded synthetic data of those shapes (3.93 GB, resident
in HBM before timing). The 128 launches of a token are captured once in a HIP
graph and replayed.

Prints ONE JSON line: value = algorithmic bytes per token / time per token
(GB/s), plus equivalent tokens/s, the roofline of the dominant kernel (the
gate.up SwiGLU launch, timed per launch with HIP events on its stream), the
measured device-to-device copy bandwidth, and the CPU oracle's throughput on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of roofline) for 4-bit group-64 GEMV; equiv decode tok/s"
HBM_PEAK_GBS = 8000.0
EPS = 1e-5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qswiglu_llama3_8b.json")
KERNEL_SOURCES = ["qg_mv.hip", "qg_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dequant_gemv_qgemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: this build runs on one GPU only; --gpus above 1 is not supported "
              "(the sharding plan is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_gemv_qgemv_amd as qg
    import synth

    if not os.path.exists(qg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    model = dict(synth.LLAMA3_8B)
    model["layers"] = args.layers
    H, FF, QD = model["hidden"], model["ffn"], model["q_dim"]

    # ---- weights (host, then HBM) -------------------------------------------
    t0 = time.time()
    host_layers, layers = [], []
    for li in range(model["layers"]):
        w = synth.layer_weights(args.seed, model, li)
        host_layers.append(w)
        d = {k: qg.QMat.from_host(v, dev) for k, v in w.items() if isinstance(v, dict)}
        d["g_attn"] = torch.from_numpy(w["g_attn"].view(np.int16)).to(dev)
        d["g_ffn"] = torch.from_numpy(w["g_ffn"].view(np.int16)).to(dev)
        layers.append(d)
    torch.cuda.synchronize()
    weight_bytes = sum(m.nbytes() for d in layers for k, m in d.items() if isinstance(m, qg.QMat))
    log(f"weights: {model['layers']} layers, {weight_bytes / 1e9:.3f} GB in HBM "
        f"({time.time() - t0:.1f} s)")

    # activation traffic per token (fp32 reads/writes of x, qkv, h, u + norm weights)
    act_bytes = model["layers"] * 4 * (
        (H + model["qkv"]) + (QD + H + H) + (H + FF) + (FF + H + H)) + model["layers"] * 2 * H * 2
    step_bytes = weight_bytes + act_bytes

    # ---- buffers ---------------------------------------------------------------
    x0 = torch.from_numpy(synth.activations(args.seed, "x0", H, np.float32)).to(dev)
    x = torch.empty(H, dtype=torch.float32, device=dev)
    qkv = torch.empty(model["qkv"], dtype=torch.float32, device=dev)
    h = torch.empty(H, dtype=torch.float32, device=dev)
    u = torch.empty(FF, dtype=torch.float32, device=dev)
    ws = qg.workspace(qg.QG_OP_SWIGLU, FF, H, 1, 4, 0, 1, dev)

    def token():
        x.copy_(x0)
        for d in layers:
            qg.qgemv_rmsnorm(d["qkv"], x, d["g_attn"], EPS, y=qkv, ws=ws)
            qg.qgemv(d["o"], qkv[:QD], residual=x, y=h, ws=ws)
            qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)
            qg.qgemv(d["down"], u, residual=h, y=x, ws=ws)

    token()
    torch.cuda.synchronize()
    eager_out = x.clone()
    step = token
    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            token()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            token()
        step = graph.replay
        step()
        torch.cuda.synchronize()
        if not torch.equal(x, eager_out):
            log("graph replay differs from the eager token; falling back to eager launches")
            step = token
            graph = None
    if not bool(torch.isfinite(x).all()):
        log("non-finite output")
        sys.exit(1)

    # ---- timed steps ------------------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"{args.steps} tokens: {ms * 1e3:.1f} us/token, {gbs:.0f} GB/s, {1e3 / ms:.0f} tok/s")

    # ---- dominant kernel: gate.up SwiGLU, per-launch HIP events ----------------
    sw_bytes = (layers[0]["gate"].nbytes() + layers[0]["up"].nbytes() + H * 4 + H * 2 + FF * 4)
    n_rep = 2
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(len(layers) * n_rep)]
    for i in range(len(evs)):
        d = layers[i % len(layers)]
        qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)  # warm the launch path
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for i, (a, b) in enumerate(evs):
        d = layers[i % len(layers)]
        a.record(stream)
        qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    sw_us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    sw_gbs = sw_bytes / (sw_us * 1e-6) / 1e9

    # traffic: HBM bytes per launch from the committed counter profile, if it
    # was taken on the current kernel source
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_hash") == kernel_hash():
                traffic = tr.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    # ---- measured copy bandwidth (read + write bytes) --------------------------
    nb = 1 << 30
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nb * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    # ---- CPU oracle baseline on a bounded sample --------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(16, os.cpu_count() or 1))
        xh = synth.activations(args.seed, "x0", H, np.float32).astype(np.float64)
        t_start = time.time()
        done_bytes = 0
        nl = 0
        while nl < len(host_layers) and time.time() - t_start < args.cpu_seconds:
            w = host_layers[nl]
            xh = oracle.decoder_layer(w, xh, QD, EPS, nthreads=threads)
            done_bytes += sum(int(m["q"].nbytes + m["scales"].nbytes + m["biases"].nbytes)
                              for m in w.values() if isinstance(m, dict))
            nl += 1
        dt = time.time() - t_start
        cpu = {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{nl} of {len(host_layers)} decoder layers of one token "
                         f"({done_bytes / 1e9:.3f} GB of weights) in {dt:.1f} s, fp64 scalar C",
               "tok_per_s": round(nl / len(host_layers) / dt, 6)}

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode stack, 4-bit g64 planar, M=1",
                   "layers": model["layers"], "hidden": H, "qkv": model["qkv"], "ffn": FF,
                   "bytes_per_token": step_bytes, "graph": graph is not None},
        "tok_per_s": round(1e3 / ms, 2),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "frac_of_copy_peak": round(gbs / copy_gbs, 4),
        "copy_peak_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "kernel": "qswiglu 14336x4096 x2 (gate.up, rmsnorm)",
                     "achieved": round(sw_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(sw_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": sw_bytes, "us_per_launch": round(sw_us, 3)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
