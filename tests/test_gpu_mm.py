"""GPU parity of the small-M path (M = 2..8 activation vectors, matrix-core
kernels) against the CPU oracle on the same seeded inputs.

Bars as for M = 1: unpacking bit-exact (one-hot probes), floating outputs
within max|y_gpu - y_ref| <= 2e-3 * max|y_ref| for each output vector."""

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
    for k in range(7):
        qg.qg_tune(k, 0)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def close(got, ref, tol=TOL, what=""):
    """The bar per output vector: for [M][N] outputs each row m is checked
    against its own max|y_ref[m]|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if got.ndim == 2:
        for m in range(got.shape[0]):
            close(got[m], ref[m], tol, f"{what} vector {m}")
        return
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


def sample_rows(N, n=192, seed=0):
    if N <= n:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n - 2, replace=False)]))


def acts(seed, tag, M, K, dtype):
    return synth.activations(seed, tag, M * K, dtype).reshape(M, K)


FMTS = [(4, synth.AFFINE), (2, synth.AFFINE), (4, synth.LUT)]
# shapes span one band, ragged bands, several workgroups, and 1, 2 and 4 K slices
SHAPES = [(16, 512), (17, 512), (300, 1024), (1000, 4096), (513, 4608), (64, 14336)]


@pytest.mark.parametrize("bits,fmt", FMTS)
@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("M", [2, 3, 8])
def test_qgemv_m(qg, bits, fmt, N, K, M):
    say(f"qgemv M={M} bits={bits} fmt={fmt} N={N} K={K}")
    W = synth.qmat(21, ("mm", bits, fmt, N, K), N, K, bits, fmt)
    x = acts(21, ("x", M, K), M, K, np.float16)
    r = acts(21, ("r", M, N), M, N, np.float32)
    ws = qg.workspace(qg.QG_OP_GEMV, N, K, M, bits, fmt, 1, DEV)
    Wd = qg.QMat.from_host(W, DEV)
    y = qg.qgemv(Wd, to_dev(x), residual=to_dev(r), ws=ws)
    y2 = qg.qgemv(Wd, to_dev(x), residual=to_dev(r), ws=ws)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, N)
    close(y.cpu().numpy(), oracle.gemv(W, x, r, nthreads=8), what="qgemv M>1")
    assert torch.equal(y, y2), "not deterministic"


@pytest.mark.parametrize("M", [2, 4, 8])
def test_qgemv_m_f32_and_in_place(qg, M):
    N, K = 777, 8192
    say(f"qgemv M={M} fp32 x, in-place residual, N={N} K={K}")
    W = synth.qmat(22, "f32", N, K, 4)
    x = acts(22, "x", M, K, np.float32) * 7.0
    r = acts(22, "r", M, N, np.float32)
    ws = qg.workspace(qg.QG_OP_GEMV, N, K, M, 4, 0, 1, DEV)
    yd = to_dev(r.copy())
    qg.qgemv(qg.QMat.from_host(W, DEV), to_dev(x), residual=yd, y=yd, ws=ws)
    torch.cuda.synchronize()
    close(yd.cpu().numpy(), oracle.gemv(W, x, r, nthreads=8), what="in place")


def test_qgemv_m_token_scales(qg):
    """Tokens of very different magnitude, a zero token and a single spike:
    each token carries its own power-of-two scale."""
    M, N, K = 6, 200, 4096
    W = synth.qmat(23, "scales", N, K, 4)
    x = acts(23, "x", M, K, np.float32)
    x[0] *= 1e-6
    x[1] *= 3e4
    x[2] = 0.0
    x[3, :] = 0.0
    x[3, 1234] = 2.5
    x[4, :2048] *= 1e-5  # one half of K tiny, the other N(0,1)
    ws = qg.workspace(qg.QG_OP_GEMV, N, K, M, 4, 0, 1, DEV)
    y = qg.qgemv(qg.QMat.from_host(W, DEV), to_dev(x), ws=ws).cpu().numpy()
    ref = oracle.gemv(W, x, nthreads=8)
    for m in range(M):
        if m == 2:
            assert np.all(y[m] == 0.0)
            continue
        close(y[m], ref[m], what=f"token {m}")


@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_bit_exact_m(qg, bits):
    """s=1, b=0, token m = e_{k_m}: y[m][n] is code[n][k_m] exactly; token
    rows holding 16^j at four columns decode four codes at once."""
    N, K, M = 80, 1024, 8
    W = synth.qmat(24, ("unpack", bits), N, K, bits)
    W["scales"][:] = 1
    W["biases"][:] = 0
    codes = oracle.unpack(W)
    Wd = qg.QMat.from_host(W, DEV)
    cols = [0, 1, 2, 7, 8, 15, 16, 31, 33, 63, 64, 100, 255, 256, 511, 512, 777, 1023]
    for i in range(0, len(cols), M):
        cs = cols[i:i + M]
        x = np.zeros((len(cs), K), np.float32)
        for m, c in enumerate(cs):
            x[m, c] = 1.0
        if len(cs) == 1:
            x = np.vstack([x, np.zeros((1, K), np.float32)])
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        for m, c in enumerate(cs):
            assert np.array_equal(y[m], codes[:, c].astype(np.float32)), f"column {c}"
    groups = [[5, 70, 200, 511], [3, 4, 5, 6], [600, 601, 1000, 1023]]
    x = np.zeros((len(groups), K), np.float32)
    for m, g in enumerate(groups):
        for j, c in enumerate(g):
            x[m, c] = float(16 ** j)
    y = qg.qgemv(Wd, to_dev(x)).cpu().numpy().astype(np.int64)
    for m, g in enumerate(groups):
        for j, c in enumerate(g):
            assert np.array_equal((y[m] >> (4 * j)) & 15, codes[:, c]), f"token {m} column {c}"


def test_dequant_single_rounding_bit_exact_m(qg):
    """token m = e_{k_m} gives y[m][n] = fl32(code*s + b), one rounding."""
    N, K = 64, 512
    W = synth.qmat(25, "dq", N, K, 4)
    dense = oracle.dequant(W)
    cols = [0, 3, 64, 129, 255, 300, 448, 511]
    x = np.zeros((len(cols), K), np.float32)
    for m, c in enumerate(cols):
        x[m, c] = 1.0
    y = qg.qgemv(qg.QMat.from_host(W, DEV), to_dev(x)).cpu().numpy()
    for m, c in enumerate(cols):
        assert np.array_equal(y[m], dense[:, c].astype(np.float32)), f"column {c}"


def test_lut_one_hot_bit_exact_m(qg):
    N, K = 48, 512
    W = synth.qmat(26, "lut1h", N, K, 4, synth.LUT)
    dense = oracle.dequant(W)
    cols = [0, 1, 31, 32, 200, 255, 256, 511]
    x = np.zeros((len(cols), K), np.float32)
    for m, c in enumerate(cols):
        x[m, c] = 1.0
    y = qg.qgemv(qg.QMat.from_host(W, DEV), to_dev(x)).cpu().numpy()
    for m, c in enumerate(cols):
        assert np.array_equal(y[m], dense[:, c].astype(np.float32)), f"column {c}"


@pytest.mark.parametrize("bits,fmt", FMTS)
@pytest.mark.parametrize("N,K", [(6144, 4096), (300, 8192), (40, 512)])
def test_qgemv_rmsnorm_m(qg, bits, fmt, N, K):
    M = 4
    say(f"qgemv_rmsnorm M={M} bits={bits} fmt={fmt} N={N} K={K}")
    W = synth.qmat(27, ("rn", bits, fmt, N, K), N, K, bits, fmt)
    g = synth.norm_weight(27, ("g", K), K)
    x = acts(27, ("x", K), M, K, np.float32) * 3.0
    r = acts(27, ("r", N), M, N, np.float32)
    ws = qg.workspace(qg.QG_OP_GEMV_RMSNORM, N, K, M, bits, fmt, 1, DEV)
    rows = sample_rows(N)
    y = qg.qgemv_rmsnorm(qg.QMat.from_host(W, DEV), to_dev(x), to_dev(g), 1e-5,
                         residual=to_dev(r), ws=ws)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_gemv(rows_of(W, rows), x, g, 1e-5, r[:, rows], nthreads=8)
    close(y.cpu().numpy()[:, rows], ref, what="rmsnorm M>1")


@pytest.mark.parametrize("bits,fmt", FMTS)
@pytest.mark.parametrize("F,K,norm", [(14336, 4096, True), (1000, 2048, False), (24, 8192, True)])
def test_qswiglu_m(qg, bits, fmt, F, K, norm):
    M = 8
    say(f"qswiglu M={M} bits={bits} fmt={fmt} F={F} K={K} norm={norm}")
    Wg = synth.qmat(28, ("gate", bits, fmt, F, K), F, K, bits, fmt)
    Wu = synth.qmat(28, ("up", bits, fmt, F, K), F, K, bits, fmt)
    g = synth.norm_weight(28, ("g", K), K) if norm else None
    x = acts(28, ("x", K), M, K, np.float16)
    ws = qg.workspace(qg.QG_OP_SWIGLU, F, K, M, bits, fmt, 1, DEV)
    rows = sample_rows(F)
    u = qg.qswiglu(qg.QMat.from_host(Wg, DEV), qg.QMat.from_host(Wu, DEV), to_dev(x),
                   None if g is None else to_dev(g), 1e-5, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_swiglu(rows_of(Wg, rows), rows_of(Wu, rows), x, g, 1e-5, nthreads=8)
    close(u.cpu().numpy()[:, rows], ref, what="swiglu M>1")


@pytest.mark.parametrize("bits,fmt", [(2, synth.AFFINE), (4, synth.LUT)])
def test_llama_layer_m8(qg, bits, fmt):
    """One Llama-3-8B-shaped decode layer for 8 activation vectors through the
    four fused calls, in the 2-bit and the table format. Each call is checked
    against the oracle applied to that call's own GPU input: with these
    synthetic weights some tokens cancel strongly inside the layer, so the
    end-to-end result of such a token amplifies any rounding of its inputs
    and is not a fair bar for one call."""
    M = 8
    say(f"llama layer M={M} bits={bits} fmt={fmt}")
    model = synth.LLAMA3_8B
    w = synth.layer_weights(77, model, 0, bits, fmt)
    H, Q = model["hidden"], model["q_dim"]
    x = acts(77, "h0", M, H, np.float32)
    d = {k: qg.QMat.from_host(w[k], DEV) for k in ("qkv", "o", "gate", "up", "down")}
    F = w["gate"]["N"]
    ws = qg.workspace(qg.QG_OP_SWIGLU, max(F, w["qkv"]["N"]), max(F, H), M, bits, fmt, 1, DEV)
    xd = to_dev(x)
    qkv = qg.qgemv_rmsnorm(d["qkv"], xd, to_dev(w["g_attn"]), 1e-5, ws=ws)
    a = qkv[:, :Q].contiguous()
    h = qg.qgemv(d["o"], a, residual=xd, ws=ws)
    u = qg.qswiglu(d["gate"], d["up"], h, to_dev(w["g_ffn"]), 1e-5, ws=ws)
    y = qg.qgemv(d["down"], u, residual=h, ws=ws)
    torch.cuda.synchronize()
    qkv, a, h, u, y = (t.cpu().numpy() for t in (qkv, a, h, u, y))
    rq = sample_rows(w["qkv"]["N"])
    rh = sample_rows(H)
    rf = sample_rows(F)
    for m in range(M):
        close(qkv[m, rq], oracle.rmsnorm_gemv(rows_of(w["qkv"], rq), x[m], w["g_attn"], 1e-5),
              what=f"qkv token {m}")
        close(h[m, rh], oracle.gemv(rows_of(w["o"], rh), a[m], x[m, rh]), what=f"o token {m}")
        close(u[m, rf], oracle.rmsnorm_swiglu(rows_of(w["gate"], rf), rows_of(w["up"], rf), h[m],
                                              w["g_ffn"], 1e-5), what=f"gate.up token {m}")
        close(y[m, rh], oracle.gemv(rows_of(w["down"], rh), u[m], h[m, rh]), what=f"down token {m}")
