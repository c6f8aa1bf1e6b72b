"""Decode-throughput benchmark of the quantized matvec path on one MI355X.

Default (--config stack, 4-bit, M=1): one step = one decode token through
the Llama-3-8B-shaped stack: 32 layers, hidden 4096, each layer = rmsnorm+QKV
matvec (4096->6144), O matvec (4096->4096, + residual), rmsnorm + gate.up
SwiGLU (4096->14336 x2), down matvec (14336->4096, + residual); 4-bit codes,
group 64, fp16 scale + bias, fp32 activations; the attention output is stood
in by the q-slice of the QKV output. Weights are seeded synthetic data of
those shapes (3.93 GB, resident in HBM before timing). The launches of a step
are captured once in a HIP graph and replayed.

Other workloads (each prints its own line): --config stack with --bits 2,
--bits 8, --fmt 1 (16-entry table) or --bits 16 --fmt 2 (dense fp16 weights),
and --m 1..8 activation vectors per step; --config
single (one 2048 x 2048 4-bit matvec, rotating over 256 weight sets);
--config attn (decode attention of 32 Llama-shaped layers against fp16 KV
caches of --ctx positions); --config moe (one 512-expert layer, top-3 + shared expert, 60 chained router
draws per token over the same weights); --config qwen (28-layer hidden-1024
stack + final norm + 151936 x 1024 logits + top-40, three model copies
rotated per token).

Prints ONE JSON line: value = algorithmic bytes per step / time per step
(GB/s), plus equivalent steps/s, the roofline of the dominant kernel
(back-to-back launches over distinct weights in a graph, timed with HIP
events on the stream that replays it), the streaming-read and copy peaks
measured in the same run with the library's own probes (qg_probe_read,
qg_probe_copy), and the CPU oracle's throughput on a bounded sample of the
same workload (all threads the host grants, and one thread).
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
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["qg_mv.hip", "qg_mm.hip", "qg_topk.hip", "qg_moe.hip", "qg_api.hip", "qg_common.h",
                  "qg_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dequant_gemv_qgemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


REF_READ_BYTES = 64 << 20  # reference streaming read of known size for counter calibration
# where a counter pass writes its launch labels (QG_PMC_DIR overrides)
PMC_DIR = os.environ.get("QG_PMC_DIR", os.path.join(ROOT, "pmc_out"))


def traffic_name(args) -> str:
    """File stem of a workload's counter summary under profiles/."""
    if args.config == "stack":
        fmt = {0: f"{args.bits}bit", 1: "lut", 2: "dense_f16"}[args.fmt]
        tp = f"_tp{args.tp}" if getattr(args, "tp", 1) > 1 else ""
        return f"traffic_llama3_8b_stack_{fmt}_m{args.m}{tp}"
    return {"single": "traffic_qgemv_2048x2048_single", "moe": f"traffic_qmoe_512_experts_m{args.m}",
            "qwen": "traffic_qwen3_06b_stack_logits", "attn": "traffic_qattn",
            "phases": "traffic_phases"}[args.config]


def pmc_reference_reads(qg, dev):
    """Two streaming reads of exactly REF_READ_BYTES: the counters' unit."""
    import torch
    buf = torch.ones(2 * REF_READ_BYTES // 4, dtype=torch.float32, device=dev)
    out = torch.empty(512 * 256, dtype=torch.int32, device=dev)
    for i in range(2):
        qg.qg_probe_read(buf[i * REF_READ_BYTES // 4:(i + 1) * REF_READ_BYTES // 4], out, 512)
    torch.cuda.synchronize()


def pmc_pass(args, qg, dev, run_once, labels, nbytes, outputs):
    """Counter pass: two reference reads, then the workload's launches once,
    eagerly, in a known order (labels[i] names product launch i). Writes the
    labels and each launch's algorithmic bytes next to the counter output."""
    import torch
    pmc_reference_reads(qg, dev)
    run_once()
    torch.cuda.synchronize()
    os.makedirs(PMC_DIR, exist_ok=True)
    meta = {"workload": traffic_name(args), "labels": labels, "bytes": nbytes, "outputs": outputs,
            "argv": sys.argv[1:], "kernel_hash": kernel_hash()}
    with open(os.path.join(PMC_DIR, "pmc_labels.json"), "w") as fh:
        json.dump(meta, fh, indent=1)
    log(f"pmc pass done: {len(labels)} launches")


PRODUCT_KERNELS = ("qmv_kernel", "qmm_kernel", "topk_kernel", "sample_kernel", "attn_kernel")


def short_kernel(name: str) -> str:
    """'void qg::(anonymous namespace)::qmv_kernel<4, 0, 64, 1, 0, 0, 2>(qg::MvParams)'
    -> 'qmv_kernel<4, 0, 64, 1, 0, 0, 2>'."""
    import re
    m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
    return m.group(1) if m else name[:60]


def summarize_pmc(fetch_csv, write_csv, labels_json):
    """HBM bytes per launch of a workload from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), scaled by what FETCH_SIZE reports for the reference reads
    of REF_READ_BYTES (the counter's unit on this device); written to
    profiles/<workload>.json and .md next to the algorithmic bytes."""
    import csv
    meta = json.load(open(labels_json))

    def rel(path):
        return os.path.relpath(os.path.abspath(path), ROOT)

    def dispatches(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        ref = [float(r["Counter_Value"]) * 1024.0 for r in rows if "probe_read" in r["Kernel_Name"]]
        ours = [(r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0) for r in rows
                if any(k in r["Kernel_Name"] for k in PRODUCT_KERNELS)]
        return ref, ours

    ref_f, fetch = dispatches(fetch_csv, "FETCH_SIZE")
    _, write = dispatches(write_csv, "WRITE_SIZE")
    labels = meta["labels"]
    if len(fetch) != len(labels) or len(write) != len(labels):
        raise SystemExit(f"{len(fetch)}/{len(write)} product dispatches against {len(labels)} labels")
    scale = REF_READ_BYTES / (sum(ref_f[:2]) / 2)
    per = {}
    for lab, (kn, f), (_, w) in zip(labels, fetch, write):
        d = per.setdefault(lab, {"kernel": short_kernel(kn), "fetch": [], "write": []})
        d["fetch"].append(f * scale)
        d["write"].append(w * scale)
    out = {"workload": meta["workload"], "kernel_hash": meta.get("kernel_hash", kernel_hash()),
           "counter_scale": round(scale, 4),
           "argv": meta["argv"], "launches": {}}
    lines = [f"# HBM traffic per launch: {meta['workload']}", "",
             "Two counter passes, each on its own run (on the MI355X, repository root as $R):", "",
             f"    cd /tmp && timeout -s KILL 150 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "
             f"$R/{rel(os.path.dirname(fetch_csv))} -o run -- python3 $R/bench.py {' '.join(meta['argv'])}",
             f"    cd /tmp && timeout -s KILL 150 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "
             f"$R/{rel(os.path.dirname(write_csv))} -o run -- python3 $R/bench.py {' '.join(meta['argv'])}",
             f"    python bench.py --summarize-pmc {rel(fetch_csv)} {rel(write_csv)} {rel(labels_json)}", "",
             f"The pass first streams two buffers of exactly {REF_READ_BYTES >> 20} MiB with qg_probe_read; "
             f"FETCH_SIZE reports {sum(ref_f[:2]) / 2 / 1024:.0f} KiB for each, so every FETCH_SIZE and "
             f"WRITE_SIZE value is multiplied by {scale:.4f}. Values are averages over the launches "
             "of each kind in one eager pass of the workload.", "",
             "| launch | kernel | n | algorithmic B | HBM fetch B | HBM write B | traffic / algorithmic "
             "| outputs | traffic B per output |", "|---|---|---|---|---|---|---|---|---|"]
    for lab, d in per.items():
        f = sum(d["fetch"]) / len(d["fetch"])
        w = sum(d["write"]) / len(d["write"])
        alg = meta["bytes"][lab]
        n_out = meta["outputs"][lab]
        out["launches"][lab] = {"kernel": d["kernel"], "n": len(d["fetch"]), "algorithmic_bytes": alg,
                                "fetch_bytes": round(f), "write_bytes": round(w),
                                "bytes_per_launch": round(f + w), "ratio": round((f + w) / alg, 4),
                                "outputs": n_out, "bytes_per_output": round((f + w) / n_out, 1)}
        lines.append(f"| {lab} | `{d['kernel']}` | {len(d['fetch'])} | {alg} | {f:.0f} | {w:.0f} | "
                     f"{(f + w) / alg:.3f} | {n_out} | {(f + w) / n_out:.1f} |")
    lines += ["", f"Source hash of the kernels these counters were taken on: `{out['kernel_hash']}` "
              "(bench.py reports a launch's traffic only while the hash matches)."]
    stem = os.path.join(PROFILES, meta["workload"])
    json.dump(out, open(stem + ".json", "w"), indent=1)
    open(stem + ".md", "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_of(args, label):
    """Counter-measured HBM bytes of one launch kind of this workload, or None
    when there are none for the current kernel sources."""
    path = os.path.join(PROFILES, traffic_name(args) + ".json")
    try:
        tr = json.load(open(path))
    except (OSError, ValueError):
        return None
    if tr.get("kernel_hash") != kernel_hash():
        return None
    return tr.get("launches", {}).get(label, {}).get("bytes_per_launch")


def summarize_trace(path):
    """Average duration of each of the four matvec launches of a decode layer
    (qkv, o, gate.up, down: the launch order inside a token) from a rocprofv3
    kernel-trace CSV."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    # M = 1 runs on qmv_kernel<bits, fmt, lanes, rows, epilogue, ...>, M = 2..8 (4- and 2-bit
    # codes, tables) on qmm_kernel<bits, fmt, epilogue>
    mm = not any("qmv_kernel" in r["Kernel_Name"] for r in rows)
    q = [r for r in rows if ("qmm_kernel" if mm else "qmv_kernel") in r["Kernel_Name"]]
    names = ["qkv: rmsnorm + 6144x4096", "o: 4096x4096 + residual",
             "gate.up: swiglu 2 x 14336x4096", "down: 4096x14336 + residual"]
    # stored bytes per weight from the kernel's (bits, fmt) template arguments
    targs = q[0]["Kernel_Name"].split("<", 1)[1].split(",") if q else ["4", "0"]
    bits, fmt = int(targs[0]), int(targs[1])
    per_w = {0: bits / 8 + 4 / 64, 1: bits / 8, 2: 2.0}[fmt]
    lut = 32 if fmt == 1 else 0
    nbytes = [int(n * k * per_w) + n * lut for n, k in
              ((6144, 4096), (4096, 4096), (2 * 14336, 4096), (4096, 14336))]
    dur = [[] for _ in names]
    i = 0
    while i + 3 < len(q):
        # the epilogue argument (1 = SwiGLU): fifth of qmv_kernel's, third of qmm_kernel's
        ep = 2 if mm else 4
        swi = [q[i + k]["Kernel_Name"].split("<", 1)[1].split(">", 1)[0].split(",")[ep].strip() == "1"
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
        if not v:
            print(f"| {name} | 0 | - | - | {nbytes[k]} | - |")
            continue
        avg = sum(v) / len(v) / 1e3
        print(f"| {name} | {len(v)} | {avg:.2f} | {min(v) / 1e3:.2f} | {nbytes[k]} | "
              f"{nbytes[k] / avg / 1e3:.0f} |")


def graph_step(fn, use_graph, out_tensor):
    """Captures fn in a HIP graph (after one eager run) and checks that a
    replay gives bitwise the eager result; returns (step, graph or None)."""
    import torch
    fn()
    torch.cuda.synchronize()
    eager = out_tensor.clone()
    if not use_graph:
        return fn, None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out_tensor, eager):
        log("graph replay differs from the eager run; falling back to eager launches")
        return fn, None
    return g.replay, g


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_launches(fn, n, use_graph, reps=5):
    """us per launch of fn (which issues n launches), replayed from a graph."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
    else:
        a.record()
        for _ in range(reps):
            fn()
        b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * n)


def probe_peaks(qg, dev):
    """Streaming-read and copy bandwidth of this GPU, measured with the
    library's probes over 1 GiB (best of several grid sizes, 10 launches
    each, HIP events), and torch's device copy for reference. Copy figures
    count read + write bytes."""
    import torch
    nb = 1 << 30
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    out = torch.empty(16384 * 256, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn, moved):
        rates = []
        for blocks in (256, 512, 1024, 2048, 4096, 8192, 16384):
            fn(blocks)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                fn(blocks)
            e1.record()
            torch.cuda.synchronize()
            rates.append(moved * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return max(rates)

    read = max(best(lambda b: qg.qg_probe_read(src, out, b), nb),
               best(lambda b: qg.qg_probe_read(src, out, b, cached=True), nb))
    copy = best(lambda b: qg.qg_probe_copy(dst, src, b), 2 * nb)
    tcopy = best(lambda b: dst.copy_(src), 2 * nb)
    del src, dst, out
    torch.cuda.empty_cache()
    return {"read_gbs": round(read, 1), "copy_gbs": round(copy, 1), "torch_copy_gbs": round(tcopy, 1),
            "how": "qg_probe_read / qg_probe_copy over 1 GiB, 16-byte accesses (read: non-temporal "
                   "and cached, copy: non-temporal), best of 256..16384 workgroups of 256 threads, "
                   "10 launches each; copy counts read + write bytes"}


def cpu_sample(work, seconds):
    """Runs work(i) -> bytes for i = 0, 1, ... until `seconds` have passed;
    returns (bytes done, calls, seconds)."""
    t_start = time.time()
    done, n = 0, 0
    while time.time() - t_start < seconds:
        b = work(n)
        if b is None:
            break
        done += b
        n += 1
    dt = time.time() - t_start
    return done, n, dt


def oracle_threads():
    """Threads for the oracle: every core this process may use (the host's
    CPU share when OMP_NUM_THREADS states it)."""
    n = os.cpu_count() or 1
    try:
        n = min(n, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        pass
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(make_work, seconds, describe, extra=None):
    """The oracle timed on the host: make_work(threads) gives work(i) -> bytes
    (None when the sample is exhausted); one leg with every thread the host
    grants, one with a single thread on a fresh sample."""
    th = oracle_threads()
    done, n, dt = cpu_sample(make_work(th), seconds)
    d1, n1, dt1 = cpu_sample(make_work(1), max(seconds / 2, 3.0))
    out = {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
           "sample": describe(n, done, dt) + f", {th} threads",
           "nproc": os.cpu_count(), "cpu_model": cpu_model(),
           "single_thread": {"value": round(d1 / dt1 / 1e9, 4), "unit": "GB/s",
                             "sample": describe(n1, d1, dt1) + ", 1 thread"}}
    if extra:
        out.update(extra(n, done, dt))
    return out


def emit(args, workload, cfg, step_bytes, ms, dom, peaks, cpu, dtype):
    gbs = step_bytes / (ms * 1e-3) / 1e9
    dom["frac_of_read_peak"] = round(dom["achieved"] / peaks["read_gbs"], 4)
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
        "dtype": dtype,
        "data": "synthetic",
        "config": dict({"workload": workload, "bytes_per_step": step_bytes}, **cfg,
                       **({"tune": args.tune} if args.tune else {})),
        "steps_per_s": round(1e3 / ms, 2),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "frac_of_read_peak": round(gbs / peaks["read_gbs"], 4),
        "frac_of_copy_peak": round(gbs / peaks["copy_gbs"], 4),
        "peaks": peaks,
        "roofline": dom,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def arith_dtype(bits, fmt, m):
    """The arithmetic the path computes in: fp16 x fp16 products (codes are
    exact fp16 values, table entries are fp16, x is staged in fp16 after a
    power-of-two range scale) accumulated in fp32."""
    core = "mfma f16xf16->f32" if (m > 1 and bits in (2, 4)) else "f16xf16->f32"
    return f"{core} (x staged in fp16 after a power-of-two scale, fp32 accumulate)"


def roofline(kernel, nbytes, us, traffic=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": nbytes, "us_per_launch": round(us, 3)}


def upload_layer(qg, w, dev):
    import torch
    d = {k: qg.QMat.from_host(v, dev) for k, v in w.items() if isinstance(v, dict)}
    for k in ("g_attn", "g_ffn"):
        d[k] = torch.from_numpy(w[k].view(np.int16)).to(dev)
    return d


def run_stack(args, qg, synth, dev):
    """Llama-3-8B-shaped decode stack; M activation vectors per step."""
    import torch
    bits, fmt, M = args.bits, args.fmt, args.m
    model = synth.tp_shard(synth.LLAMA3_8B, args.tp)
    model["layers"] = args.layers
    H, FF, QD, NQ = model["hidden"], model["ffn"], model["q_dim"], model["qkv"]

    t0 = time.time()
    host_layers, layers = [], []
    for li in range(model["layers"]):
        w = synth.layer_weights(args.seed, model, li, bits, fmt)
        host_layers.append(w)
        layers.append(upload_layer(qg, w, dev))
    torch.cuda.synchronize()
    weight_bytes = sum(m.nbytes() for d in layers for m in d.values() if isinstance(m, qg.QMat))
    log(f"weights: {model['layers']} layers, {weight_bytes / 1e9:.3f} GB in HBM "
        f"({time.time() - t0:.1f} s)")
    # activation traffic per step (fp32 reads/writes of x, qkv, h, u; norm weights)
    act_bytes = model["layers"] * (M * 4 * ((H + NQ) + (QD + H + H) + (H + FF) + (FF + H + H))
                                   + 2 * H * 2)
    step_bytes = weight_bytes + act_bytes
    # algorithmic bytes of each launch of a layer (weights + the vectors it reads and writes)
    d0 = layers[0]
    launch_bytes = {
        "qkv": d0["qkv"].nbytes() + M * 4 * (H + NQ) + H * 2,
        "o": d0["o"].nbytes() + M * 4 * (QD + H + H),
        "gate.up": d0["gate"].nbytes() + d0["up"].nbytes() + M * 4 * (H + FF) + H * 2,
        "down": d0["down"].nbytes() + M * 4 * (FF + H + H),
    }
    launch_outputs = {"qkv": M * NQ, "o": M * H, "gate.up": M * FF, "down": M * H}

    shp = (lambda n: (n,)) if M == 1 else (lambda n: (M, n))
    x0 = torch.from_numpy(synth.activations(args.seed, "x0", M * H, np.float32)
                          .reshape(shp(H))).to(dev)
    x = torch.empty(shp(H), dtype=torch.float32, device=dev)
    qkv = torch.empty(shp(NQ), dtype=torch.float32, device=dev)
    a = torch.empty(shp(QD), dtype=torch.float32, device=dev)
    h = torch.empty(shp(H), dtype=torch.float32, device=dev)
    u = torch.empty(shp(FF), dtype=torch.float32, device=dev)
    ws = qg.workspace(qg.QG_OP_SWIGLU, max(FF, H), max(FF, H), M, bits, fmt, 1, dev)

    def layer_calls(d):
        qg.qgemv_rmsnorm(d["qkv"], x, d["g_attn"], EPS, y=qkv, ws=ws)
        if M == 1:
            att = qkv[:QD]
        else:  # stands in for the attention kernel writing its [M][q_dim] output
            a.copy_(qkv[:, :QD])
            att = a
        qg.qgemv(d["o"], att, residual=x, y=h, ws=ws)
        qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)
        qg.qgemv(d["down"], u, residual=h, y=x, ws=ws)

    def token():
        x.copy_(x0)
        for d in layers:
            layer_calls(d)

    if args.pmc_pass:
        n = min(4, len(layers))

        def once():
            x.copy_(x0)
            for d in layers[:n]:
                layer_calls(d)
        pmc_pass(args, qg, dev, once, ["qkv", "o", "gate.up", "down"] * n, launch_bytes,
                 launch_outputs)
        return

    step, graph = graph_step(token, not args.no_graph, x)
    if not bool(torch.isfinite(x).all()):
        log("non-finite output")
        sys.exit(1)
    ms = time_steps(step, args.steps, args.warmup)
    log(f"{args.steps} steps: {ms * 1e3:.1f} us/step, {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s, "
        f"{1e3 / ms:.0f} steps/s")

    # dominant kernel: gate.up SwiGLU, one launch per layer over distinct weights
    sw_bytes = launch_bytes["gate.up"]

    def swiglu_all():
        for d in layers:
            qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws)

    sw_us = time_launches(swiglu_all, len(layers), graph is not None, reps=10)
    fmt_name = {0: f"{bits}-bit g64 planar", 1: "4-bit 16-entry table per row",
                2: "dense fp16 weights"}[fmt]
    path = "matrix cores" if bits in (2, 4) else "one pass per vector"
    kname = ("qswiglu" if M == 1 else f"qswiglu M={M} ({path})") + \
        f" {FF}x{H} x2 (gate.up, rmsnorm)"
    dom = roofline(kname, sw_bytes, sw_us, traffic_of(args, "gate.up"))
    marginal = None
    if M == 1:
        # The same launch over the first 4096, 8192 and 12288 rows of the same
        # matrices: a least-squares line through the four (bytes, time)
        # points gives the rate of the extra rows and the part of a launch
        # that does not depend on its size.
        pts = [(sw_bytes, sw_us)]
        row_bytes = (d0["gate"].nbytes() + d0["up"].nbytes()) // FF + 4 * M
        sizes = [n for n in (4096, 8192, 12288) if n < FF]
        for n_rows in sizes:
            def rows(m, n=n_rows):
                cut = lambda t: None if t is None else t[:n]
                return qg.QMat(cut(m.q), cut(m.scales), cut(m.biases), cut(m.lut), N=n, K=m.K,
                               bits=m.bits, fmt=m.fmt, group=m.group)

            part = [(rows(d["gate"]), rows(d["up"]), d["g_ffn"]) for d in layers]

            def swiglu_part(part=part, n=n_rows):
                for gt, up, gn in part:
                    qg.qswiglu(gt, up, h, gn, EPS, u=u[:n], ws=ws)

            pts.append((sw_bytes - (FF - n_rows) * row_bytes,
                        time_launches(swiglu_part, len(layers), graph is not None, reps=10)))
        bx = np.array([p[0] for p in pts], np.float64)
        ty = np.array([p[1] for p in pts], np.float64)
        slope, icpt = np.polyfit(bx, ty, 1) if len(pts) > 2 else (0.0, 0.0)  # us per byte, us
        if slope > 0:
            marginal = {"gbs": round(1e-3 / slope, 1), "fixed_us": round(float(icpt), 3),
                        "points_us": {str(int(n)): round(float(t), 3)
                                      for n, t in zip([FF] + sizes, ty)},
                        "how": "the launch at 4096, 8192, 12288 and all 14336 rows of the same "
                               "matrices (graph replays); least-squares line of time against "
                               "bytes: its slope gives the rate of the extra rows, its intercept "
                               "the size-independent part of a launch"}
            dom["marginal"] = marginal
    peaks = probe_peaks(qg, dev)
    if marginal:
        marginal["frac_of_read_peak"] = round(marginal["gbs"] / peaks["read_gbs"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x_start = synth.activations(args.seed, "x0", M * H, np.float32).reshape(M, H).astype(np.float64)
        layer_w = [sum(int(sum(v.nbytes for v in mm.values() if isinstance(v, np.ndarray)))
                       for mm in w.values() if isinstance(mm, dict)) for w in host_layers]

        def make_work(th):
            st = {"x": x_start.copy()}

            def work(i):
                if i >= len(host_layers):
                    return None
                st["x"] = np.stack([oracle.decoder_layer(host_layers[i], st["x"][m], QD, EPS,
                                                         nthreads=th) for m in range(M)])
                return layer_w[i]
            return work

        cpu = cpu_baseline(
            make_work, args.cpu_seconds,
            lambda n, done, dt: (f"{n} of {len(host_layers)} decoder layers of one step ({M} vector(s); "
                                 f"{done / 1e9:.3f} GB of weights) in {dt:.1f} s, fp64 scalar C"),
            lambda n, done, dt: {"steps_per_s": round(n / len(host_layers) / dt, 6)})
    workload = f"llama3-8b-shaped decode stack, {fmt_name}, M={M}"
    if args.tp > 1:
        workload += (f", one GPU's shard at tensor parallelism {args.tp} (qkv {NQ} rows, o {H}x{QD}, "
                     f"gate.up {FF} rows, down {H}x{FF}; no all-reduce)")
    cfg = {"layers": model["layers"], "hidden": H, "qkv": NQ, "ffn": FF, "bits": bits, "fmt": fmt,
           "m": M, "graph": graph is not None, **({"tp": args.tp} if args.tp > 1 else {})}
    emit(args, workload, cfg, step_bytes, ms, dom, peaks, cpu, arith_dtype(bits, fmt, M))


def run_single(args, qg, synth, dev):
    """One 2048 x 2048 4-bit matvec; 256 weight sets rotated (607 MB, more
    than the 256 MB last-level cache)."""
    import torch
    N = K = 2048
    sets = 256
    host = [synth.qmat(args.seed, ("cfg0", i), N, K, 4) for i in range(sets)]
    mats = [qg.QMat.from_host(w, dev) for w in host]
    x = torch.from_numpy(synth.activations(args.seed, "cfg0x", K, np.float16)).to(dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    unit_bytes = mats[0].nbytes() + K * 2 + N * 4

    def all_sets():
        for m in mats:
            qg.qgemv(m, x, y=y)

    if args.pmc_pass:
        def once():
            for m in mats[:16]:
                qg.qgemv(m, x, y=y)
        pmc_pass(args, qg, dev, once, ["qgemv 2048x2048"] * 16, {"qgemv 2048x2048": unit_bytes},
                 {"qgemv 2048x2048": N})
        return
    step, graph = graph_step(all_sets, not args.no_graph, y)
    ms = time_steps(step, args.steps, args.warmup)
    us = ms * 1e3 / sets
    dom = roofline("qgemv 2048x2048 4-bit g64 (x fp16)", unit_bytes, us,
                   traffic_of(args, "qgemv 2048x2048"))
    peaks = probe_peaks(qg, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        xh = synth.activations(args.seed, "cfg0x", K, np.float16)

        def make_work(th):
            def work(i):
                oracle.gemv(host[i % sets], xh, nthreads=th)
                return unit_bytes
            return work

        cpu = cpu_baseline(make_work, args.cpu_seconds,
                           lambda n, done, dt: f"{n} matvecs 2048x2048 in {dt:.1f} s, fp64 scalar C",
                           lambda n, done, dt: {"us_per_matvec": round(dt / n * 1e6, 1)})
    cfg = {"n": N, "k": K, "weight_sets": sets, "us_per_matvec": round(us, 3),
           "graph": graph is not None}
    emit(args, "single 4-bit g64 matvec 2048x2048, M=1, back-to-back over 256 weight sets",
         cfg, unit_bytes * sets, ms, dom, peaks, cpu, arith_dtype(4, 0, 1))


def run_moe(args, qg, synth, dev):
    """One 512-expert layer (gate, up 4096->1024, down 1024->4096, 4-bit),
    top-3 routed + 1 shared expert; a token runs 60 chained layers over the
    same weights with fresh router logits each. With --m M, M tokens run
    through each layer in one batched call; the algorithmic bytes of a layer
    are then the union of the experts the M tokens chose, plus the shared
    one, each counted once."""
    import torch
    M = args.m
    mdl = synth.MOE_397B
    E, F, H, K, L = mdl["experts"], mdl["ffn"], mdl["hidden"], mdl["top_k"], mdl["draws"]
    t0 = time.time()
    gate = synth.qmat(args.seed, "moe_gate_all", E * F, H, 4)
    up = synth.qmat(args.seed, "moe_up_all", E * F, H, 4)
    down = synth.qmat(args.seed, "moe_down_all", E * H, F, 4)
    for W in (gate, up, down):
        W["E"] = E
    shared = tuple(synth.qmat(args.seed, ("moe_shared", n), *nk, 4)
                   for n, nk in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))))
    g = synth.norm_weight(args.seed, "moe_g", H)
    Gd, Ud, Dd = (qg.QMat.from_host(W, dev) for W in (gate, up, down))
    Sd = tuple(qg.QMat.from_host(W, dev) for W in shared)
    gd = torch.from_numpy(g.view(np.int16)).to(dev)
    if M == 1:
        logits = [synth.router_logits(args.seed, ("moe_route", l), E) for l in range(L)]
        x0h = synth.activations(args.seed, "moe_x0", H, np.float32)
    else:
        logits = [synth.router_logits(args.seed, ("moe_route_batch", l), (M, E)) for l in range(L)]
        x0h = synth.activations(args.seed, "moe_x0_batch", (M, H), np.float32)
    lgd = torch.from_numpy(np.stack(logits)).to(dev)
    x0 = torch.from_numpy(x0h).to(dev)
    x = torch.empty_like(x0)
    ws = qg.workspace(qg.QG_OP_MOE, H, F, M, 4, 0, K, dev)
    torch.cuda.synchronize()
    log(f"moe weights {(Gd.nbytes() + Ud.nbytes() + Dd.nbytes()) / 1e9:.2f} GB ({time.time() - t0:.1f} s)")
    expert_bytes = synth.qmat_bytes(F, H) * 2 + synth.qmat_bytes(H, F)
    vec_bytes = M * (E * 4 + H * 4 * 2) + H * 2
    if M == 1:
        layer_bytes = [(K + 1) * expert_bytes + vec_bytes] * L
    else:
        # the experts each layer's tokens choose (largest logits; exact ties do not occur)
        layer_bytes = [(len(set(np.argsort(-lg, axis=1, kind="stable")[:, :K].ravel().tolist())) + 1)
                       * expert_bytes + vec_bytes for lg in logits]

    def token():
        x.copy_(x0)
        for l in range(L):
            if M == 1:
                qg.qmoe_experts(Gd, Ud, Dd, E, Sd, lgd[l], K, x, gd, EPS, y=x, ws=ws)
            else:
                qg.qmoe_experts_batch(Gd, Ud, Dd, E, Sd, lgd[l], K, x, gd, EPS, y=x, ws=ws)

    if args.pmc_pass:
        gu_bytes = (K + 1) * (synth.qmat_bytes(F, H) * 2) + M * (E * 4 + H * 4 + (K + 1) * F * 4) + H * 2
        dn_bytes = (K + 1) * synth.qmat_bytes(H, F) + M * ((K + 1) * F * 4 + H * 8)

        def once():
            x.copy_(x0)
            for l in range(4):
                if M == 1:
                    qg.qmoe_experts(Gd, Ud, Dd, E, Sd, lgd[l], K, x, gd, EPS, y=x, ws=ws)
                else:
                    qg.qmoe_experts_batch(Gd, Ud, Dd, E, Sd, lgd[l], K, x, gd, EPS, y=x, ws=ws)
        labels = ["route + gate.up", "down + combine"]
        pmc_pass(args, qg, dev, once, labels * 4,
                 {labels[0]: gu_bytes, labels[1]: dn_bytes},
                 {labels[0]: M * (K + 1) * F, labels[1]: M * H})
        return
    step, graph = graph_step(token, not args.no_graph, x)
    ms = time_steps(step, args.steps, args.warmup)
    us_layer = ms * 1e3 / L
    kname = ("qmoe_experts (route, gate.up of 4 experts, down + combine)" if M == 1 else
             f"qmoe_experts_batch M={M} (route, gate.up of 4 experts per token, down + combine)")
    parts = [traffic_of(args, "route + gate.up"), traffic_of(args, "down + combine")]
    dom = roofline(kname, sum(layer_bytes) / L, us_layer,
                   None if None in parts else sum(parts))
    peaks = probe_peaks(qg, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        def make_work(th):
            st = {"x": np.atleast_2d(x0h.astype(np.float64))}

            def work(i):
                if i >= L:
                    return None
                lg = np.atleast_2d(logits[i])
                st["x"] = np.stack([oracle.moe_layer(gate, up, down, shared, lg[m], K, st["x"][m], g,
                                                     EPS, nthreads=th)[0] for m in range(M)])
                return layer_bytes[i]
            return work

        cpu = cpu_baseline(make_work, args.cpu_seconds,
                           lambda n, done, dt: (f"{n} of {L} chained expert layers of {M} token(s) in "
                                                f"{dt:.1f} s, fp64 scalar C"),
                           lambda n, done, dt: {"tok_per_s": round(M * n / L / dt, 6)})
    cfg = {"experts": E, "hidden": H, "ffn": F, "top_k": K, "shared": 1, "layers_per_token": L,
           "tokens": M, "us_per_layer": round(us_layer, 3), "graph": graph is not None}
    name = "moe expert layer, 512 experts 4-bit g64, top-3 + shared, 60 chained draws per token"
    if M > 1:
        name += f", {M} tokens per batched call"
    emit(args, name, cfg, sum(layer_bytes), ms, dom, peaks, cpu, arith_dtype(4, 0, 1))


def run_qwen(args, qg, synth, dev):
    """Qwen3-0.6B-shaped stack (28 layers, hidden 1024) + final norm + logits
    151936 x 1024 + top-40 on the GPU; three model copies rotated per token
    (about 1 GB, more than the last-level cache)."""
    import torch
    model = dict(synth.QWEN3_06B)
    H, FF, QD, NQ, V = model["hidden"], model["ffn"], model["q_dim"], model["qkv"], model["vocab"]
    copies, topk = 3, 40
    t0 = time.time()
    hosts, devs = [], []
    for c in range(copies):
        hl = [synth.layer_weights(args.seed + c, model, li) for li in range(model["layers"])]
        head = synth.qmat(args.seed + c, ("qwen_head",), V, H, 4)
        gf = synth.norm_weight(args.seed + c, "qwen_gf", H)
        hosts.append((hl, head, gf))
        devs.append(([upload_layer(qg, w, dev) for w in hl], qg.QMat.from_host(head, dev),
                     torch.from_numpy(gf.view(np.int16)).to(dev)))
    torch.cuda.synchronize()
    stack_bytes = sum(m.nbytes() for d in devs[0][0] for m in d.values() if isinstance(m, qg.QMat))
    head_bytes = devs[0][1].nbytes()
    act_bytes = model["layers"] * (4 * ((H + NQ) + (QD + H + H) + (H + FF) + (FF + H + H)) + 2 * H * 2) \
        + H * 4 + H * 2 + V * 4 * 2 + topk * 8
    step_bytes = stack_bytes + head_bytes + act_bytes
    log(f"qwen: {copies} copies, {step_bytes / 1e6:.1f} MB per token ({time.time() - t0:.1f} s)")
    x0 = torch.from_numpy(synth.activations(args.seed, "qwen_x0", H, np.float32)).to(dev)
    x = torch.empty(H, dtype=torch.float32, device=dev)
    qkv = torch.empty(NQ, dtype=torch.float32, device=dev)
    h = torch.empty(H, dtype=torch.float32, device=dev)
    u = torch.empty(FF, dtype=torch.float32, device=dev)
    z = torch.empty(V, dtype=torch.float32, device=dev)
    idx = torch.empty(topk, dtype=torch.int32, device=dev)
    vals = torch.empty(topk, dtype=torch.float32, device=dev)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, H, 1, 4, 0, topk, dev)
    ws2 = qg.workspace(qg.QG_OP_SWIGLU, FF, FF, 1, 4, 0, 1, dev)

    def token_of(c):
        layers, head, gf = devs[c]

        def token():
            x.copy_(x0)
            for d in layers:
                qg.qgemv_rmsnorm(d["qkv"], x, d["g_attn"], EPS, y=qkv, ws=ws2)
                qg.qgemv(d["o"], qkv[:QD], residual=x, y=h, ws=ws2)
                qg.qswiglu(d["gate"], d["up"], h, d["g_ffn"], EPS, u=u, ws=ws2)
                qg.qgemv(d["down"], u, residual=h, y=x, ws=ws2)
            qg.qlogits_topk(head, x, topk, gf, EPS, logits=z, idx=idx, vals=vals, ws=ws)
        return token

    # the head is one launch (the matvec's workgroups merge their top-k keys)
    # or the matvec and then the top-k kernel
    head_launches = qg.qg_logits_topk_launches(V, H, topk)
    if args.pmc_pass:
        layer_b = {n: devs[0][0][0][k].nbytes() for n, k in (("qkv", "qkv"), ("o", "o"), ("down", "down"))}
        lb = {"qkv": layer_b["qkv"] + 4 * (H + NQ) + H * 2, "o": layer_b["o"] + 4 * (QD + 2 * H),
              "gate.up": devs[0][0][0]["gate"].nbytes() * 2 + 4 * (H + FF) + H * 2,
              "down": layer_b["down"] + 4 * (FF + 2 * H)}
        outs = {"qkv": NQ, "o": H, "gate.up": FF, "down": H}
        labels = ["qkv", "o", "gate.up", "down"] * model["layers"]
        if head_launches == 1:
            lb["logits + top-40 (one launch)"] = head_bytes + H * 4 + H * 2 + V * 4 + topk * 8
            outs["logits + top-40 (one launch)"] = V + topk
            labels.append("logits + top-40 (one launch)")
        else:
            lb["logits (rmsnorm + matvec)"] = head_bytes + H * 4 + H * 2 + V * 4
            lb["top-40"] = V * 4 + topk * 8
            outs["logits (rmsnorm + matvec)"], outs["top-40"] = V, topk
            labels += ["logits (rmsnorm + matvec)", "top-40"]
        pmc_pass(args, qg, dev, token_of(0), labels, lb, outs)
        return
    steps_c, graph = [], None
    for c in range(copies):
        st, graph = graph_step(token_of(c), not args.no_graph, idx)
        steps_c.append(st)
    k = [0]

    def step():
        steps_c[k[0] % copies]()
        k[0] += 1

    ms = time_steps(step, args.steps, args.warmup)

    def heads():
        for c in range(copies):
            qg.qlogits_topk(devs[c][1], x, topk, devs[c][2], EPS, logits=z, idx=idx, vals=vals,
                            ws=ws)

    head_us = time_launches(heads, copies, graph is not None)
    # algorithmic bytes: weights, x, norm weight and logits once, top-k out
    # (the two-launch form reads the logits back)
    head_alg = head_bytes + H * 4 + H * 2 + V * 4 + topk * 8 + (V * 4 if head_launches == 2 else 0)
    parts = ([traffic_of(args, "logits + top-40 (one launch)")] if head_launches == 1 else
             [traffic_of(args, "logits (rmsnorm + matvec)"), traffic_of(args, "top-40")])
    dom = roofline(f"qlogits_topk 151936x1024 4-bit + final norm + top-40 ({head_launches} launch"
                   f"{'es' if head_launches > 1 else ''})", head_alg, head_us,
                   None if None in parts else sum(parts))
    peaks = probe_peaks(qg, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        hl, head, gf = hosts[0]
        per_layer = stack_bytes // model["layers"]

        def make_work(th):
            st = {"x": synth.activations(args.seed, "qwen_x0", H, np.float32).astype(np.float64)}

            def work(i):
                if i < len(hl):
                    st["x"] = oracle.decoder_layer(hl[i], st["x"], QD, EPS, nthreads=th)
                    return per_layer
                if i == len(hl):
                    oracle.logits_topk(head, st["x"], topk, gf, EPS, nthreads=th)
                    return head_bytes
                return None
            return work

        cpu = cpu_baseline(make_work, args.cpu_seconds,
                           lambda n, done, dt: (f"{min(n, len(hl))} of {len(hl)} decoder layers"
                                                f"{' + logits/top-40' if n > len(hl) else ''} of one "
                                                f"token in {dt:.1f} s, fp64 scalar C"))
    cfg = {"layers": model["layers"], "hidden": H, "vocab": V, "top_k": topk, "copies": copies,
           "graph": graph is not None, "head_launches": head_launches}
    emit(args, "qwen3-0.6b-shaped decode stack + logits + top-40, 4-bit g64, M=1", cfg,
         step_bytes, ms, dom, peaks, cpu, arith_dtype(4, 0, 1))


def run_phases(args, qg, synth, dev):
    """The Llama-3-8B-shaped token's matvec byte ranges (qkv, o, gate.up,
    down per layer) read with no arithmetic, three ways: one launch per range
    (the launch-per-matvec design), one launch over every range, and one
    launch with a device-wide barrier between ranges (what a persistent
    whole-token kernel needs, each matvec's x being the previous one's
    output). Prices the launch boundary against the barrier on the same
    bytes; the line's value is the launch-per-range rate."""
    import torch
    model = dict(synth.LLAMA3_8B)
    model["layers"] = args.layers
    H, FF, QD, NQ = model["hidden"], model["ffn"], model["q_dim"], model["qkv"]
    per_layer = [synth.qmat_bytes(NQ, H), synth.qmat_bytes(H, QD), 2 * synth.qmat_bytes(FF, H),
                 synth.qmat_bytes(H, FF)]
    flat, off = [], 0
    for _ in range(model["layers"]):
        for b in per_layer:
            flat += [off, b]
            off += -(-b // 256) * 256
    n, total = len(flat) // 2, off
    src = torch.empty(total, dtype=torch.uint8, device=dev)
    src.fill_(7)
    rng = torch.tensor(flat, dtype=torch.int64, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(2 * cus * 512, dtype=torch.int32, device=dev)
    flags = torch.zeros(2 * cus, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = sum(flat[1::2])
    log(f"phases: {n} ranges, {nbytes / 1e9:.3f} GB")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(3, min(args.steps, 20))

    def timed(launch, prep=None):
        ts = []
        for r in range(reps + 2):
            if prep:
                prep()
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            if r >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    res = {}
    for wg_per_cu in (1, 2):
        blocks = cus * wg_per_cu

        def per_range():
            for q in range(n):
                qg.qg_probe_phases(src, rng[2 * q:], 1, False, out, blocks)

        # one launch per range, replayed from a graph like the decode token
        per_range()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            per_range()
        t_launch = timed(g.replay)
        t_one = timed(lambda: qg.qg_probe_phases(src, rng, n, False, out, blocks))
        err.zero_()
        t_bar = timed(lambda: qg.qg_probe_phases(src, rng, n, True, out, blocks, flags, err),
                      prep=flags.zero_)
        # the barrier with each range's first loads issued before the wait
        t_pre = timed(lambda: qg.qg_probe_phases(src, rng, n, 2, out, blocks, flags, err),
                      prep=flags.zero_)
        torch.cuda.synchronize()
        if int(err.item()):
            raise RuntimeError("phase barrier exceeded its spin limit; timing void")
        res[f"{wg_per_cu}_wg_per_cu"] = {
            "blocks": blocks, "us_launch_per_range": round(t_launch, 1),
            "us_one_launch": round(t_one, 1), "us_one_launch_barrier": round(t_bar, 1),
            "us_one_launch_barrier_prefetch": round(t_pre, 1),
            "us_per_launch_boundary": round((t_launch - t_one) / (n - 1), 3),
            "us_per_barrier": round((t_bar - t_one) / (n - 1), 3),
            "us_per_barrier_prefetch": round((t_pre - t_one) / (n - 1), 3),
            "gbs_launch_per_range": round(nbytes / (t_launch * 1e-6) / 1e9, 1),
            "gbs_one_launch": round(nbytes / (t_one * 1e-6) / 1e9, 1),
            "gbs_one_launch_barrier": round(nbytes / (t_bar * 1e-6) / 1e9, 1),
            "gbs_one_launch_barrier_prefetch": round(nbytes / (t_pre * 1e-6) / 1e9, 1)}
        log(f"phases {wg_per_cu} wg/cu: {res[f'{wg_per_cu}_wg_per_cu']}")
    best = min(res.values(), key=lambda r: r["us_launch_per_range"])
    us = best["us_launch_per_range"]
    dom = roofline(f"probe_phases_kernel ({n} ranges, one launch each)", nbytes / n, us / n)
    peaks = probe_peaks(qg, dev)
    cfg = {"layers": model["layers"], "ranges": n, "phases": res}
    emit(args, "llama3-8b-shaped token byte ranges, read only (launch boundary vs grid barrier)",
         cfg, nbytes, us * 1e-3, dom, peaks, None, "u32 (xor of the bytes read)")


def run_attn(args, qg, synth, dev):
    """Decode attention of a Llama-3-8B-shaped model (32 query heads, 8 kv
    heads, head dimension 128) at context length --ctx: one step is the
    attention of all layers at position ctx-1 (the new k/v rows are written
    there first), each layer with its own fp16 cache, so a step reads more
    than the 256 MB last-level cache holds for ctx >= 4096."""
    import torch
    H, Hkv, d, L, T = 32, 8, 128, args.layers, args.ctx
    pos = T - 1
    scale = 1.0 / float(np.sqrt(d))
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    kc = [torch.randn(Hkv, T, d, generator=gen, device=dev).half() for _ in range(L)]
    vc = [torch.randn(Hkv, T, d, generator=gen, device=dev).half() for _ in range(L)]
    q = torch.randn(L, H, d, generator=gen, device=dev)
    kn = torch.randn(L, Hkv, d, generator=gen, device=dev)
    vn = torch.randn(L, Hkv, d, generator=gen, device=dev)
    out = torch.empty(L, H, d, device=dev)
    ws = qg.workspace(qg.QG_OP_ATTN, H, T, Hkv, k=d, device=dev)
    layer_bytes = 2 * Hkv * (pos + 1) * d * 2 + 2 * H * d * 4 + 2 * Hkv * d * (4 + 2)

    def step():
        for l in range(L):
            qg.qattn_decode(q[l], kc[l], vc[l], pos, scale, kn[l], vn[l], out=out[l], ws=ws)

    run, graph = graph_step(step, not args.no_graph, out)
    ms = time_steps(run, args.steps, args.warmup)
    us = time_launches(step, L, not args.no_graph)
    dom = roofline(f"qattn_decode H32/Hkv8/d128, {pos + 1} positions", layer_bytes, us)
    peaks = probe_peaks(qg, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        hk = [kc[l].cpu().numpy() for l in range(2)]
        hv = [vc[l].cpu().numpy() for l in range(2)]
        hq = q[:2].double().cpu().numpy()

        def make_work(th):  # the attention oracle runs on one thread
            def work(i):
                if th > 1:
                    return None
                oracle.attention(hq[i % 2], hk[i % 2], hv[i % 2], pos + 1, scale)
                return layer_bytes
            return work

        done, n, dt = cpu_sample(make_work(1), args.cpu_seconds)
        cpu = {"value": round(done / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} layers of attention over {pos + 1} positions in {dt:.1f} s, "
                         "fp64 scalar C, one thread", "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    cfg = {"layers": L, "heads": H, "kv_heads": Hkv, "head_dim": d, "context": pos + 1,
           "graph": graph is not None}
    emit(args, f"llama3-8b-shaped decode attention, {L} layers, fp16 KV cache, context {pos + 1}",
         cfg, layer_bytes * L, ms, dom, peaks, cpu, "f16 cache x f32 query, f32 accumulate")


def tune_arg(text):
    """KNOB=VALUE with small non-negative integers (checked again by qg_tune)."""
    import argparse
    parts = text.split("=")
    if len(parts) != 2 or not all(p.strip().isdigit() for p in parts) or int(parts[0]) > 15:
        raise argparse.ArgumentTypeError(f"--tune expects KNOB=VALUE (integers), got {text!r}")
    return f"{int(parts[0])}={int(parts[1])}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="stack",
                    choices=["stack", "single", "moe", "qwen", "attn", "phases"])
    ap.add_argument("--ctx", type=int, default=8192, help="attn: context length (positions)")
    ap.add_argument("--bits", type=int, default=4, choices=[2, 4, 8, 16],
                    help="stack: code width (16 = dense fp16 weights, with --fmt 2)")
    ap.add_argument("--fmt", type=int, default=0, choices=[0, 1, 2],
                    help="stack: 0 = scale + bias per group, 1 = 16-entry table per row (4-bit), "
                         "2 = dense fp16 weights (--bits 16)")
    ap.add_argument("--m", type=int, default=1,
                    help="stack: activation vectors per step; moe: tokens per batched call (1..8)")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--tp", type=int, default=1, choices=[1, 2, 4, 8],
                    help="stack, M = 1: the layers of one GPU's shard under tensor parallelism "
                         "TP (qkv and gate/up rows, o and down inputs divided by TP; the "
                         "all-reduces are not run)")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--tune", action="append", default=[], metavar="KNOB=VALUE", type=tune_arg,
                    help="qg_tune override applied before the run (repeatable), e.g. 6=1 for staged "
                         "scale/bias rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="two reference reads of 64 MiB, then the workload's launches once, eagerly "
                         "(for rocprofv3 --pmc counter passes; writes pmc_labels.json under $QG_PMC_DIR, "
                         "default pmc_out/)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "LABELS_JSON"),
                    help="turn the counter CSVs of two --pmc-pass runs into profiles/traffic_*.{json,md}")
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
        print("bench.py: the library runs on one GPU; --gpus above 1 is not supported "
              "(the sharding plan is described in the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.fmt == 1 and args.bits != 4:
        print("bench.py: the table format has 4-bit codes", file=sys.stderr)
        sys.exit(2)
    if (args.fmt == 2) != (args.bits == 16):
        print("bench.py: dense fp16 weights are --bits 16 --fmt 2", file=sys.stderr)
        sys.exit(2)
    if not 1 <= args.m <= 8:
        print("bench.py: --m must be 1..8", file=sys.stderr)
        sys.exit(2)
    if args.tp > 1 and (args.config != "stack" or args.m != 1):
        print("bench.py: --tp is for --config stack with --m 1", file=sys.stderr)
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
    for t in args.tune:
        knob, value = (int(v) for v in t.split("="))
        qg.qg_tune(knob, value)
    {"stack": run_stack, "single": run_single, "moe": run_moe, "qwen": run_qwen,
     "attn": run_attn, "phases": run_phases}[args.config](args, qg, synth, dev)


if __name__ == "__main__":
    main()
