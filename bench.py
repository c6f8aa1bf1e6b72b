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
gate.up SwiGLU launch: 32 back-to-back launches over distinct weights in a
graph, timed with HIP events on the stream that replays it), the
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
KERNEL_SOURCES = ["qg_mv.hip", "qg_common.h", "qg_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dequant_gemv_qgemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


REF_READ_BYTES = 64 << 20  # reference streaming read of known size for counter calibration


def pmc_pass(qg, layers, model, dev):
    import torch
    H, FF = model["hidden"], model["ffn"]
    h = torch.randn(H, device=dev)
    u = torch.empty(FF, dtype=torch.float32, device=dev)
    ws = qg.workspace(qg.QG_OP_SWIGLU, FF, H, 1, 4, 0, 1, dev)
    for i in range(8):
        d = layers[i % len(layers)]
        qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)
    buf = torch.ones(2 * REF_READ_BYTES // 4, dtype=torch.float32, device=dev)
    out = torch.empty(512 * 256, dtype=torch.int32, device=dev)
    for i in range(2):
        qg.qg_probe_read(buf[i * REF_READ_BYTES // 4:(i + 1) * REF_READ_BYTES // 4], out, 512)
    torch.cuda.synchronize()
    log("pmc pass done")


def summarize_pmc(fetch_csv, write_csv):
    """HBM bytes per gate.up SwiGLU launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), scaled by the FETCH_SIZE the reference read of REF_READ_BYTES
    reports (the counter's unit on this device)."""
    import csv
    import re

    def per_kernel(path, counter):
        sw, ref = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if re.search(r"qmv_kernel<4, 0, \d+, \d, 1, 0, \d>", r["Kernel_Name"]):
                sw.append(v)
            elif "probe_read" in r["Kernel_Name"]:
                ref.append(v)
        return sw, ref

    sw_f, ref_f = per_kernel(fetch_csv, "FETCH_SIZE")
    sw_w, _ = per_kernel(write_csv, "WRITE_SIZE")
    scale = REF_READ_BYTES / (sum(ref_f) / len(ref_f))
    fetch = sum(sw_f) / len(sw_f) * scale
    write = sum(sw_w) / len(sw_w) * scale
    out = {"kernel": "qswiglu 14336x4096 x2 (gate.up, rmsnorm)", "kernel_hash": kernel_hash(),
           "counter_scale": round(scale, 4), "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write), "bytes_per_launch": round(fetch + write),
           "launches": len(sw_f)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


def summarize_trace(path):
    """Average duration of each of the four matvec launches of a decode layer
    (qkv, o, gate.up, down: the launch order inside a token) from a rocprofv3
    kernel-trace CSV."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    q = [r for r in rows if "qmv_kernel" in r["Kernel_Name"]]
    names = ["qkv: rmsnorm + 6144x4096", "o: 4096x4096 + residual",
             "gate.up: swiglu 2 x 14336x4096", "down: 4096x14336 + residual"]
    nbytes = [6144 * 4096 * 9 // 16, 4096 * 4096 * 9 // 16, 2 * 14336 * 4096 * 9 // 16,
              4096 * 14336 * 9 // 16]
    dur = [[] for _ in names]
    i = 0
    while i + 3 < len(q):
        # template arguments: bits, fmt, lanes per row, rows, epilogue (1 = SwiGLU), ...
        swi = [q[i + k]["Kernel_Name"].split("<", 1)[1].split(",")[4].strip() == "1"
               for k in range(4)]
        if swi != [False, False, True, False]:
            i += 1
            continue
        for k in range(4):
            dur[k].append(int(q[i + k]["End_Timestamp"]) - int(q[i + k]["Start_Timestamp"]))
        i += 4
    print("| launch | calls | avg us | min us | weight bytes | GB/s at avg |")
    print("|---|---|---|---|---|---|")
    for k, name in enumerate(names):
        v = dur[k]
        avg = sum(v) / len(v) / 1e3
        print(f"| {name} | {len(v)} | {avg:.2f} | {min(v) / 1e3:.2f} | {nbytes[k]} | "
              f"{nbytes[k] / avg / 1e3:.0f} |")


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
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only 8 gate.up SwiGLU launches and 2 reference reads of 64 MiB "
                         "(for rocprofv3 --pmc counter passes)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter CSVs of two --pmc-pass runs into the traffic file")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="per-matvec kernel durations of the decode tokens in a rocprofv3 trace")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return

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

    if args.pmc_pass:
        pmc_pass(qg, layers, model, dev)
        return

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

    # ---- dominant kernel: gate.up SwiGLU ----------------------------------------
    # 32 back-to-back launches (one per layer, distinct weights) captured in a
    # graph and replayed, timed with HIP events on the capturing stream.
    sw_bytes = (layers[0]["gate"].nbytes() + layers[0]["up"].nbytes() + H * 4 + H * 2 + FF * 4)

    def swiglu_all():
        for d in layers:
            qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)

    swiglu_all()
    torch.cuda.synchronize()
    sw_us = None
    if graph is not None:
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            swiglu_all()
        sg.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record()
        for _ in range(reps):
            sg.replay()
        b.record()
        torch.cuda.synchronize()
        sw_us = a.elapsed_time(b) * 1e3 / (reps * len(layers))
    else:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        swiglu_all()
        b.record()
        torch.cuda.synchronize()
        sw_us = a.elapsed_time(b) * 1e3 / len(layers)
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
