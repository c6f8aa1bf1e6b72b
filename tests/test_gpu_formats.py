"""GPU parity of the Q8 (8-bit codes, four per word) and dense fp16 matvec
formats against the CPU oracle: plain, RMSNorm-fused, gate.up SwiGLU, logits +
top-k and (Q8) MoE experts, with the probes that make unpacking bit-exact.

Bars as for the 2- and 4-bit formats: codes and top-k indices bit-exact;
floating outputs within max|y_gpu - y_ref| <= 2e-3 * max|y_ref|."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"


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
    for k in range(4):
        qg.qg_tune(k, 0)


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


def sample_rows(N, n=256, seed=0):
    if N <= n:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n - 2, replace=False)]))


FORMATS = {"q8": (8, synth.AFFINE), "f16": (16, synth.DENSE)}


def mat(seed, tag, N, K, name):
    bits, fmt = FORMATS[name]
    return synth.qmat(seed, (tag, name), N, K, bits, fmt)


def ws(qg, op, N, K, name, k=1):
    bits, fmt = FORMATS[name]
    return qg.workspace(op, N, K, 1, bits, fmt, k, DEV)


SHAPES = [(1, 64), (7, 128), (300, 1024), (1000, 3072), (513, 4096), (64, 14336), (2048, 2048)]


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_qgemv_formats(qg, name, N, K, xdt):
    say(f"qgemv {name} N={N} K={K} x={xdt}")
    W = mat(21, "gemv", N, K, name)
    x = synth.activations(21, ("x", K), K, np.float16 if xdt == "f16" else np.float32)
    y = qg.qgemv(qg.QMat.from_host(W, DEV), to_dev(x), ws=ws(qg, qg.QG_OP_GEMV, N, K, name))
    torch.cuda.synchronize()
    close(y.cpu().numpy(), oracle.gemv(W, x.astype(np.float64), nthreads=8), what=name)


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("lpr", [16, 32, 64])
@pytest.mark.parametrize("rows,splits", [(1, 1), (2, 1), (1, 3)])
def test_qgemv_formats_variants(qg, name, lpr, rows, splits):
    N, K = 333, 3072
    say(f"qgemv {name} variant lpr={lpr} rows={rows} splits={splits}")
    W = mat(22, "var", N, K, name)
    x = synth.activations(22, "varx", K, np.float32)
    r = synth.activations(22, "varr", N, np.float32)
    w = ws(qg, qg.QG_OP_GEMV, N, K, name)
    qg.qg_tune(2, lpr)
    qg.qg_tune(1, rows)
    qg.qg_tune(0, splits)
    try:
        Wd = qg.QMat.from_host(W, DEV)
        y = qg.qgemv(Wd, to_dev(x), residual=to_dev(r), ws=w)
        y2 = qg.qgemv(Wd, to_dev(x), residual=to_dev(r), ws=w)
        torch.cuda.synchronize()
    finally:
        for k in range(3):
            qg.qg_tune(k, 0)
    close(y.cpu().numpy(), oracle.gemv(W, x, r, nthreads=8), what="variant")
    assert torch.equal(y, y2), "not deterministic"


def test_q8_unpack_bit_exact(qg):
    """s=1, b=0: x = e_k gives code[n][k]; x = 256^j at three columns spells
    three codes per launch (every partial sum is an integer below 2^24)."""
    N, K = 96, 512
    say("q8 unpack probe")
    W = synth.qmat(23, "unpack8", N, K, 8)
    W["scales"][:] = 1
    W["biases"][:] = 0
    codes = oracle.unpack(W)
    Wd = qg.QMat.from_host(W, DEV)
    for k in [0, 1, 2, 3, 4, 15, 16, 31, 63, 64, 100, 255, 256, 511]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        assert np.array_equal(y, codes[:, k].astype(np.float32)), f"column {k}"
    cols = [6, 200, 509]
    x = np.zeros(K, np.float32)
    for j, c in enumerate(cols):
        x[c] = float(256 ** j)
    y = qg.qgemv(Wd, to_dev(x)).cpu().numpy().astype(np.int64)
    for j, c in enumerate(cols):
        assert np.array_equal((y >> (8 * j)) & 255, codes[:, c])


@pytest.mark.parametrize("name", ["q8", "f16"])
def test_one_hot_single_rounding_bit_exact(qg, name):
    """x = e_k gives y_n = fl32(W[n][k]): code*s needs at most 19 bits, so
    code*s + b is rounded once; a dense weight comes back unchanged."""
    N, K = 64, 512
    W = mat(24, "onehot", N, K, name)
    dense = oracle.dequant(W)
    Wd = qg.QMat.from_host(W, DEV)
    for k in [0, 3, 64, 129, 255, 256, 511]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        assert np.array_equal(y, dense[:, k].astype(np.float32)), f"column {k}"


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("N,K", [(6144, 4096), (2048, 1024), (100, 14336)])
def test_qgemv_rmsnorm_formats(qg, name, N, K):
    say(f"qgemv_rmsnorm {name} N={N} K={K}")
    W = mat(25, "rn", N, K, name)
    g = synth.norm_weight(25, ("g", K), K)
    x = synth.activations(25, ("x", K), K, np.float32) * 3.0
    r = synth.activations(25, ("r", N), N, np.float32)
    rows = sample_rows(N)
    y = qg.qgemv_rmsnorm(qg.QMat.from_host(W, DEV), to_dev(x), to_dev(g), 1e-5, residual=to_dev(r),
                         ws=ws(qg, qg.QG_OP_GEMV_RMSNORM, N, K, name))
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_gemv(rows_of(W, rows), x, g, 1e-5, r[rows])
    close(y.cpu().numpy()[rows], ref, what="rmsnorm")


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("F,K,norm", [(14336, 4096, True), (3072, 1024, True), (1000, 2048, False),
                                      (8, 64, True)])
def test_qswiglu_formats(qg, name, F, K, norm):
    say(f"qswiglu {name} F={F} K={K} norm={norm}")
    Wg = mat(26, ("gate", F, K), F, K, name)
    Wu = mat(26, ("up", F, K), F, K, name)
    g = synth.norm_weight(26, ("g", K), K) if norm else None
    x = synth.activations(26, ("x", K), K, np.float32)
    rows = sample_rows(F)
    u = qg.qswiglu(qg.QMat.from_host(Wg, DEV), qg.QMat.from_host(Wu, DEV), to_dev(x),
                   None if g is None else to_dev(g), 1e-5, ws=ws(qg, qg.QG_OP_SWIGLU, F, K, name))
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_swiglu(rows_of(Wg, rows), rows_of(Wu, rows), x, g, 1e-5)
    close(u.cpu().numpy()[rows], ref, what="swiglu")


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("V,K,k", [(151936, 1024, 40), (1000, 256, 1)])
def test_qlogits_topk_formats(qg, name, V, K, k):
    say(f"qlogits_topk {name} V={V} K={K} k={k}")
    W = mat(27, ("lm", V, K), V, K, name)
    g = synth.norm_weight(27, "gf", K)
    x = synth.activations(27, "x", K, np.float32) * 5.0
    z, idx, vals = qg.qlogits_topk(qg.QMat.from_host(W, DEV), to_dev(x), k, to_dev(g), 1e-5,
                                   ws=ws(qg, qg.QG_OP_LOGITS_TOPK, V, K, name, k))
    torch.cuda.synchronize()
    zc = z.cpu().numpy()
    rows = sample_rows(V)
    close(zc[rows], oracle.gemv(rows_of(W, rows), oracle.rmsnorm(x, g)), what="logits")
    ridx, rvals = oracle.topk(zc, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(vals.cpu().numpy(), rvals.astype(np.float32))


@pytest.mark.parametrize("E,F,H,top_k", [(16, 128, 256, 3), (16, 1024, 4096, 3)])
def test_qmoe_experts_q8(qg, E, F, H, top_k):
    say(f"qmoe_experts q8 E={E} F={F} H={H}")
    gate = synth.qmat(28, "gate_all", E * F, H, 8)
    up = synth.qmat(28, "up_all", E * F, H, 8)
    down = synth.qmat(28, "down_all", E * H, F, 8)
    for Wt in (gate, up, down):
        Wt["E"] = E
    sh = (synth.qmat(28, "sh_gate", F, H, 8), synth.qmat(28, "sh_up", F, H, 8),
          synth.qmat(28, "sh_down", H, F, 8))
    g = synth.norm_weight(28, "g", H)
    x = synth.activations(28, "x", H, np.float32)
    Gd, Ud, Dd = (qg.QMat.from_host(m, DEV) for m in (gate, up, down))
    shd = tuple(qg.QMat.from_host(m, DEV) for m in sh)
    w_ = qg.workspace(qg.QG_OP_MOE, H, F, 1, 8, 0, top_k, DEV)
    for draw in range(2):
        lg = synth.router_logits(28, ("route", draw), E)
        ids = torch.empty(top_k, dtype=torch.int32, device=DEV)
        w = torch.empty(top_k, dtype=torch.float32, device=DEV)
        y = qg.qmoe_experts(Gd, Ud, Dd, E, shd, to_dev(lg), top_k, to_dev(x), to_dev(g), 1e-5,
                            sel_ids=ids, sel_w=w, ws=w_)
        torch.cuda.synchronize()
        yref, rid, rw = oracle.moe_layer(gate, up, down, sh, lg, top_k, x, g, nthreads=8)
        assert np.array_equal(ids.cpu().numpy(), rid)
        close(y.cpu().numpy(), yref, what="moe q8")


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("M", [2, 5, 8])
@pytest.mark.parametrize("N,K", [(300, 1024), (1000, 4096), (64, 14336)])
def test_several_vectors(qg, name, M, N, K):
    """M activation vectors in one call (plain with residual, RMSNorm-fused
    and gate.up SwiGLU): each vector against the oracle, and each equal bit
    for bit to the one-vector call."""
    say(f"several vectors {name} M={M} N={N} K={K}")
    W = mat(34, ("mv", N, K), N, K, name)
    Wu = mat(34, ("mvu", N, K), N, K, name)
    X = synth.activations(34, ("x", M, K), (M, K), np.float32)
    R = synth.activations(34, ("r", M, N), (M, N), np.float32)
    g = synth.norm_weight(34, ("g", K), K)
    w = ws(qg, qg.QG_OP_SWIGLU, N, K, name)
    Wd, Wud = qg.QMat.from_host(W, DEV), qg.QMat.from_host(Wu, DEV)
    Xd, Rd, gd = to_dev(X), to_dev(R), to_dev(g)
    y = qg.qgemv(Wd, Xd, residual=Rd, ws=w)
    yn = qg.qgemv_rmsnorm(Wd, Xd, gd, 1e-5, ws=w)
    u = qg.qswiglu(Wd, Wud, Xd, gd, 1e-5, ws=w)
    X16 = to_dev(X.astype(np.float16))
    y16 = qg.qgemv(Wd, X16, ws=w)
    torch.cuda.synchronize()
    rows = sample_rows(N)
    for m in range(M):
        close(y.cpu().numpy()[m], oracle.gemv(W, X[m], R[m], nthreads=8), what=f"gemv vector {m}")
        close(yn.cpu().numpy()[m][rows], oracle.rmsnorm_gemv(rows_of(W, rows), X[m], g, 1e-5),
              what=f"rmsnorm vector {m}")
        close(u.cpu().numpy()[m][rows], oracle.rmsnorm_swiglu(rows_of(W, rows), rows_of(Wu, rows), X[m],
                                                               g, 1e-5), what=f"swiglu vector {m}")
        close(y16.cpu().numpy()[m], oracle.gemv(W, X[m].astype(np.float16).astype(np.float64),
                                                nthreads=8), what=f"fp16 x vector {m}")
        one = qg.qgemv_rmsnorm(Wd, Xd[m].contiguous(), gd, 1e-5, ws=w)
        torch.cuda.synchronize()
        assert torch.equal(one, yn[m]), f"vector {m} differs from the one-vector call"


@pytest.mark.parametrize("name", ["q8", "f16"])
@pytest.mark.parametrize("K", [20480, 65536])
@pytest.mark.parametrize("norm", [False, True])
def test_long_k_formats(qg, name, K, norm):
    """Long rows: the one-chunk-per-thread staging loops over several chunks
    per thread, and K beyond one LDS slice is split across workgroups."""
    N = 200
    say(f"long K {name} K={K} norm={norm}")
    W = mat(32, ("longk", K), N, K, name)
    x = synth.activations(32, ("x", K), K, np.float32)
    g = synth.norm_weight(32, ("g", K), K) if norm else None
    w = ws(qg, qg.QG_OP_GEMV_RMSNORM, N, K, name)
    Wd = qg.QMat.from_host(W, DEV)
    if norm:
        y = qg.qgemv_rmsnorm(Wd, to_dev(x), to_dev(g), 1e-5, ws=w)
        ref = oracle.rmsnorm_gemv(W, x, g, 1e-5, nthreads=8)
    else:
        y = qg.qgemv(Wd, to_dev(x), ws=w)
        ref = oracle.gemv(W, x, nthreads=8)
    torch.cuda.synchronize()
    close(y.cpu().numpy(), ref, what="long K")


def test_graph_replay_several_vectors_and_batched_moe(qg):
    """Q8 with four vectors and a four-token batched MoE layer captured in one
    HIP graph, replayed several times with eager work between the replays;
    every replay equals the eager run bit for bit."""
    M, N, K = 4, 1000, 4096
    E, F, H, top_k = 16, 128, 256, 3
    W = mat(35, "graph", N, K, "q8")
    Wd = qg.QMat.from_host(W, DEV)
    g = to_dev(synth.norm_weight(35, "g", K))
    X = to_dev(synth.activations(35, "x", (M, K), np.float32))
    gate = synth.qmat(35, "gate_all", E * F, H, 8)
    up = synth.qmat(35, "up_all", E * F, H, 8)
    down = synth.qmat(35, "down_all", E * H, F, 8)
    Gd, Ud, Dd = (qg.QMat.from_host(m, DEV) for m in (gate, up, down))
    sh = tuple(qg.QMat.from_host(synth.qmat(35, n, r, c, 8), DEV)
               for n, r, c in (("sh_gate", F, H), ("sh_up", F, H), ("sh_down", H, F)))
    gm = to_dev(synth.norm_weight(35, "gm", H))
    lg = to_dev(synth.router_logits(35, "route", (M, E)))
    xm0 = to_dev(synth.activations(35, "xm", (M, H), np.float32))
    wsv = ws(qg, qg.QG_OP_SWIGLU, N, K, "q8")
    wsm = qg.workspace(qg.QG_OP_MOE, H, F, M, 8, 0, top_k, DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    xm = torch.empty_like(xm0)

    def step():
        qg.qgemv_rmsnorm(Wd, X, g, 1e-5, y=y, ws=wsv)
        xm.copy_(xm0)
        for _ in range(3):
            qg.qmoe_experts_batch(Gd, Ud, Dd, E, sh, lg, top_k, xm, gm, 1e-5, y=xm, ws=wsm)

    step()
    torch.cuda.synchronize()
    ey, ex = y.clone(), xm.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(4):
        y.zero_()
        xm.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ey), f"replay {rep}: several vectors differ"
        assert torch.equal(xm, ex), f"replay {rep}: batched MoE differs"
        step()  # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,K", [("q8", 65536), ("f16", 32768)])
def test_several_vectors_beyond_one_slice_unsupported(qg, name, K):
    """Several vectors keep each vector's K in one LDS slice; a K that would
    need split-K is refused before anything is enqueued."""
    W = mat(36, ("big", K), 16, K, name)
    X = to_dev(synth.activations(36, ("x", K), (2, K), np.float32))
    w = ws(qg, qg.QG_OP_GEMV, 16, K, name)
    with pytest.raises(qg.QgError) as e:
        qg.qgemv(qg.QMat.from_host(W, DEV), X, ws=w)
    assert e.value.status == qg.QG_EUNSUPPORTED
    # one vector of the same matrix splits K and runs
    y = qg.qgemv(qg.QMat.from_host(W, DEV), X[0].contiguous(), ws=w)
    torch.cuda.synchronize()
    close(y.cpu().numpy(), oracle.gemv(W, X[0].cpu().numpy(), nthreads=8), what="one vector")
