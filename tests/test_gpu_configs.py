"""GPU parity of whole workloads, call by call: the Llama-3-8B-shaped
32-layer stack (4-bit), the same layer shapes with 2-bit codes and with
16-entry tables, the Qwen3-0.6B-shaped 28-layer stack with its logits head
and top-40, and a token of 60 chained 512-expert MoE layers. Every call is compared with the oracle applied to
that call's own GPU input (a chained stack amplifies fp32 rounding in
tokens that cancel, so end-to-end equality is not a fair bar for one call);
top-k indices and routing decisions are compared bit-exact."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"
EPS = 1e-5


@pytest.fixture(scope="module")
def qg():
    import os

    import dequant_gemv_qgemv_amd as qg
    if not os.path.exists(qg.LIB_PATH):
        from dequant_gemv_qgemv_amd import build
        build.build()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()
    yield qg


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def close(got, ref, tol=TOL, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    bound = tol * max(np.max(np.abs(ref)) if ref.size else 0.0, 1e-30)
    assert err <= bound, f"{what}: max err {err:.3e} > {bound:.3e}"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rows_of(W, rows):
    out = dict(W)
    out["N"] = len(rows)
    for k in ("q", "scales", "biases", "lut"):
        if W.get(k) is not None:
            out[k] = W[k][rows]
    return out


def sample_rows(N, n=160, seed=0):
    if N <= n:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n - 2, replace=False)]))


def check_layer(qg, w, x, QD, ws, li, n_rows=160):
    """Runs one decoder layer through the four fused calls on the GPU and
    checks each call against the oracle on that call's own GPU input (sampled
    rows). Returns the layer's output (device)."""
    d = {n: qg.QMat.from_host(w[n], DEV) for n in ("qkv", "o", "gate", "up", "down")}
    qkv = qg.qgemv_rmsnorm(d["qkv"], x, to_dev(w["g_attn"]), EPS, ws=ws)
    h = qg.qgemv(d["o"], qkv[:QD], residual=x, ws=ws)
    u = qg.qswiglu(d["gate"], d["up"], h, to_dev(w["g_ffn"]), EPS, ws=ws)
    y = qg.qgemv(d["down"], u, residual=h, ws=ws)
    torch.cuda.synchronize()
    xc, qc, hc, uc, yc = (t.cpu().numpy() for t in (x, qkv, h, u, y))
    H = len(xc)
    rq, rh, rf = (sample_rows(len(qc), n_rows, li), sample_rows(H, n_rows, li + 1),
                  sample_rows(len(uc), n_rows, li + 2))
    close(qc[rq], oracle.rmsnorm_gemv(rows_of(w["qkv"], rq), xc, w["g_attn"], EPS),
          what=f"layer {li} qkv")
    close(hc[rh], oracle.gemv(rows_of(w["o"], rh), qc[:QD], xc[rh]), what=f"layer {li} o")
    close(uc[rf], oracle.rmsnorm_swiglu(rows_of(w["gate"], rf), rows_of(w["up"], rf), hc,
                                        w["g_ffn"], EPS), what=f"layer {li} gate.up")
    close(yc[rh], oracle.gemv(rows_of(w["down"], rh), uc, hc[rh]), what=f"layer {li} down")
    return y


def test_llama_stack_32_layers(qg):
    """The Llama-3-8B-shaped stack at M = 1, 4-bit g64, all 32 layers chained
    on the GPU (the residual grows by orders of magnitude along the chain):
    every call of every layer against the oracle."""
    model = synth.LLAMA3_8B
    H, QD = model["hidden"], model["q_dim"]
    seed = 1234
    say("llama stack: 32 layers, 4-bit")
    x = torch.from_numpy(synth.activations(seed, "x0", H, np.float32)).to(DEV)
    ws = qg.workspace(qg.QG_OP_SWIGLU, model["ffn"], model["ffn"], 1, 4, 0, 1, DEV)
    scale0 = float(x.abs().max())
    for li in range(model["layers"]):
        x = check_layer(qg, synth.layer_weights(seed, model, li), x, QD, ws, li)
    # the chain really grows: the fp32 residual ends orders of magnitude above x0
    assert float(x.abs().max()) > 1e3 * scale0


@pytest.mark.parametrize("bits,fmt", [(2, synth.AFFINE), (4, synth.LUT)])
def test_llama_layers_2bit_and_table(qg, bits, fmt):
    """The 2-bit and 16-entry-table variants of the Llama layer shapes at
    M = 1 through the fused calls (rmsnorm + QKV, O + residual, rmsnorm +
    gate.up SwiGLU, down + residual), four chained layers, call by call."""
    model = dict(synth.LLAMA3_8B)
    H, QD = model["hidden"], model["q_dim"]
    seed = 2024
    say(f"llama layers bits={bits} fmt={fmt}")
    x = torch.from_numpy(synth.activations(seed, "x0", H, np.float32)).to(DEV)
    ws = qg.workspace(qg.QG_OP_SWIGLU, model["ffn"], model["ffn"], 1, bits, fmt, 1, DEV)
    for li in range(4):
        x = check_layer(qg, synth.layer_weights(seed, model, li, bits, fmt), x, QD, ws, li)


def test_qwen_stack_and_head(qg):
    """28 layers at hidden 1024 (QKV 1024->4096, O 2048->1024, gate/up
    1024->3072, down 3072->1024) + final norm + 151936 x 1024 logits +
    top-40, chained on the GPU."""
    model = synth.QWEN3_06B
    H, QD, V, k = model["hidden"], model["q_dim"], model["vocab"], 40
    seed = 4321
    say("qwen stack: 28 layers + head")
    x = torch.from_numpy(synth.activations(seed, "x0", H, np.float32)).to(DEV)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, H, 1, 4, 0, k, DEV)
    ws2 = qg.workspace(qg.QG_OP_SWIGLU, model["ffn"], model["ffn"], 1, 4, 0, 1, DEV)
    for li in range(model["layers"]):
        w = synth.layer_weights(seed, model, li)
        d = {n: qg.QMat.from_host(w[n], DEV) for n in ("qkv", "o", "gate", "up", "down")}
        qkv = qg.qgemv_rmsnorm(d["qkv"], x, to_dev(w["g_attn"]), EPS, ws=ws2)
        h = qg.qgemv(d["o"], qkv[:QD], residual=x, ws=ws2)
        u = qg.qswiglu(d["gate"], d["up"], h, to_dev(w["g_ffn"]), EPS, ws=ws2)
        y = qg.qgemv(d["down"], u, residual=h, ws=ws2)
        torch.cuda.synchronize()
        xc, qc, hc, uc, yc = (t.cpu().numpy() for t in (x, qkv, h, u, y))
        rq, rh, rf = sample_rows(len(qc)), sample_rows(H), sample_rows(len(uc))
        close(qc[rq], oracle.rmsnorm_gemv(rows_of(w["qkv"], rq), xc, w["g_attn"], EPS),
              what=f"layer {li} qkv")
        close(hc[rh], oracle.gemv(rows_of(w["o"], rh), qc[:QD], xc[rh]), what=f"layer {li} o")
        close(uc[rf], oracle.rmsnorm_swiglu(rows_of(w["gate"], rf), rows_of(w["up"], rf), hc,
                                            w["g_ffn"], EPS), what=f"layer {li} gate.up")
        close(yc[rh], oracle.gemv(rows_of(w["down"], rh), uc, hc[rh]), what=f"layer {li} down")
        x = y
    head = synth.qmat(seed, ("qwen_head",), V, H, 4)
    gf = synth.norm_weight(seed, "qwen_gf", H)
    say("qwen head: logits + top-40")
    z, idx, vals = qg.qlogits_topk(qg.QMat.from_host(head, DEV), x, k, to_dev(gf), EPS, ws=ws)
    torch.cuda.synchronize()
    zc, xc = z.cpu().numpy(), x.cpu().numpy()
    rv = sample_rows(V, 512)
    close(zc[rv], oracle.gemv(rows_of(head, rv), oracle.rmsnorm(xc, gf, EPS)), what="logits")
    ridx, rvals = oracle.topk(zc, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(vals.cpu().numpy(), rvals.astype(np.float32))


def test_moe_token_60_layers(qg):
    """512 experts (gate, up 4096->1024, down 1024->4096) + shared expert,
    top-3, 60 chained layers with their own router draws over one layer's
    weights."""
    E, F, H, K, L = 512, 1024, 4096, 3, 60
    seed = 99
    say("moe token: 60 chained expert layers")
    gate = synth.qmat(seed, "gate_all", E * F, H, 4)
    up = synth.qmat(seed, "up_all", E * F, H, 4)
    down = synth.qmat(seed, "down_all", E * H, F, 4)
    for W in (gate, up, down):
        W["E"] = E
    shared = (synth.qmat(seed, "sh_gate", F, H, 4), synth.qmat(seed, "sh_up", F, H, 4),
              synth.qmat(seed, "sh_down", H, F, 4))
    g = synth.norm_weight(seed, "g", H)
    Gd, Ud, Dd = (qg.QMat.from_host(W, DEV) for W in (gate, up, down))
    Sd = tuple(qg.QMat.from_host(W, DEV) for W in shared)
    gd = to_dev(g)
    ws = qg.workspace(qg.QG_OP_MOE, H, F, 1, 4, 0, K, DEV)
    x = torch.from_numpy(synth.activations(seed, "x0", H, np.float32)).to(DEV)
    ids = torch.empty(K, dtype=torch.int32, device=DEV)
    wts = torch.empty(K, dtype=torch.float32, device=DEV)
    for l in range(L):
        lg = synth.router_logits(seed, ("route", l), E)
        xin = x.cpu().numpy()
        y = qg.qmoe_experts(Gd, Ud, Dd, E, Sd, to_dev(lg), K, x, gd, EPS, sel_ids=ids, sel_w=wts,
                            ws=ws)
        torch.cuda.synchronize()
        yref, rid, rw = oracle.moe_layer(gate, up, down, shared, lg, K, xin, g, EPS, nthreads=8)
        assert np.array_equal(ids.cpu().numpy(), rid), f"layer {l} routing"
        close(wts.cpu().numpy(), rw, tol=1e-6, what=f"layer {l} routing weights")
        close(y.cpu().numpy(), yref, what=f"layer {l}")
        x = y
