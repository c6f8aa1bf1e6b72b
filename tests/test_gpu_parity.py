"""GPU parity: every entry point of the HIP library against the CPU oracle on
the same seeded inputs.

Bars: code unpacking and top-k indices bit-exact; floating outputs within
max|y_gpu - y_ref| <= 2e-3 * max|y_ref| per output vector (fp32 accumulation
against the fp64 oracle). Large shapes are checked on sampled rows that the
oracle computes one by one."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def qg():
    import dequant_gemv_qgemv_amd as qg
    import os
    if not os.path.exists(qg.LIB_PATH):
        from dequant_gemv_qgemv_amd import build
        build.build()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()
    yield qg
    for k in range(7):
        qg.qg_tune(k, 0)


# the logits top-k: one launch (the matvec's workgroups merge their rows'
# keys) or the matvec and then the top-k kernel (knob 5 = 1)
TOPK_PATHS = ["one_launch", "two_launch"]


def set_topk_path(qg, path):
    qg.qg_tune(5, 1 if path == "two_launch" else 0)


DEV = "cuda"


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


def dev_mat(qg, W):
    return qg.QMat.from_host(W, DEV)


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a).to(DEV)


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
    r = np.unique(np.concatenate([[0, N - 1], rng.choice(N, n - 2, replace=False)]))
    return r


def ws_for(qg, op, N, K, k=1):
    return qg.workspace(op, N, K, 1, 4, 0, k, DEV)


# ---------------------------------------------------------------------------
SHAPES = [(1, 64), (7, 128), (300, 1024), (1000, 3072), (513, 4096), (64, 14336), (2048, 2048),
          (10001, 1792)]  # rows of 56 chunks past 8192 rows: 16 lanes, ragged last band


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_qgemv_4bit(qg, N, K, xdt):
    say(f"qgemv 4-bit N={N} K={K} x={xdt}")
    W = synth.qmat(11, ("g4", N, K), N, K, 4)
    x = synth.activations(11, ("x", K), K, np.float16 if xdt == "f16" else np.float32)
    ws = ws_for(qg, qg.QG_OP_GEMV, N, K)
    y = qg.qgemv(dev_mat(qg, W), to_dev(x), ws=ws)
    torch.cuda.synchronize()
    close(y.cpu().numpy(), oracle.gemv(W, x.astype(np.float64), nthreads=8), what="qgemv")


def test_qgemv_config0(qg):
    """N=K=2048, 4-bit g64, x fp16 N(0,1), y fp32: the single-matvec workload."""
    say("qgemv config0 2048x2048")
    W = synth.qmat(1234, "cfg0", 2048, 2048, 4)
    x = synth.activations(1234, "cfg0", 2048, np.float16)
    y = qg.qgemv(dev_mat(qg, W), to_dev(x))
    torch.cuda.synchronize()
    close(y.cpu().numpy(), oracle.gemv(W, x, nthreads=8), what="cfg0")


@pytest.mark.parametrize("lpr", [16, 32, 64])
@pytest.mark.parametrize("rows", [1, 2])
@pytest.mark.parametrize("splits", [1, 3])
def test_qgemv_variants(qg, lpr, rows, splits):
    N, K = 333, 3072
    say(f"qgemv variant lpr={lpr} rows={rows} splits={splits}")
    W = synth.qmat(5, "var", N, K, 4)
    x = synth.activations(5, "varx", K, np.float32)
    r = synth.activations(5, "varr", N, np.float32)
    ws = ws_for(qg, qg.QG_OP_GEMV, N, K)
    qg.qg_tune(2, lpr)
    qg.qg_tune(1, rows)
    qg.qg_tune(0, splits)
    try:
        y = qg.qgemv(dev_mat(qg, W), to_dev(x), residual=to_dev(r), ws=ws)
        y2 = qg.qgemv(dev_mat(qg, W), to_dev(x), residual=to_dev(r), ws=ws)
        torch.cuda.synchronize()
    finally:
        for k in range(3):
            qg.qg_tune(k, 0)
    ref = oracle.gemv(W, x, r, nthreads=8)
    close(y.cpu().numpy(), ref, what="variant")
    assert torch.equal(y, y2), "not deterministic"


@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_bit_exact(qg, bits):
    """s=1, b=0 and x = e_k: y_n is code[n][k] exactly (any summation order)."""
    N, K = 96, 512
    say(f"unpack probe bits={bits}")
    W = synth.qmat(3, ("unpack", bits), N, K, bits)
    W["scales"][:] = 1
    W["biases"][:] = 0
    codes = oracle.unpack(W)
    Wd = dev_mat(qg, W)
    for k in [0, 1, 2, 7, 8, 15, 16, 31, 33, 63, 64, 100, 255, 256, 511]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        assert np.array_equal(y, codes[:, k].astype(np.float32)), f"column {k}"
    # 16^j at four columns (fp32): decodes four codes per launch, exactly
    cols = [5, 70, 200, 511]
    x = np.zeros(K, np.float32)
    for j, c in enumerate(cols):
        x[c] = float(16 ** j)
    y = qg.qgemv(Wd, to_dev(x)).cpu().numpy().astype(np.int64)
    for j, c in enumerate(cols):
        assert np.array_equal((y >> (4 * j)) & 15, codes[:, c])


def test_dequant_single_rounding_bit_exact(qg):
    """x = e_k gives y_n = fl32(code*s + b) with one rounding."""
    N, K = 64, 256
    W = synth.qmat(4, "dq", N, K, 4)
    dense = oracle.dequant(W)
    Wd = dev_mat(qg, W)
    for k in [0, 3, 64, 129, 255]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        assert np.array_equal(y, dense[:, k].astype(np.float32)), f"column {k}"


def test_lut_one_hot_bit_exact(qg):
    N, K = 48, 256
    W = synth.qmat(6, "lut1h", N, K, 4, synth.LUT)
    dense = oracle.dequant(W)
    Wd = dev_mat(qg, W)
    for k in [0, 1, 31, 32, 200]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y = qg.qgemv(Wd, to_dev(x)).cpu().numpy()
        assert np.array_equal(y, dense[:, k].astype(np.float32)), f"column {k}"


@pytest.mark.parametrize("bits,fmt", [(2, synth.AFFINE), (4, synth.LUT)])
@pytest.mark.parametrize("N,K", [(5, 64), (777, 1024), (640, 4096), (96, 14336)])
def test_qgemv_2bit_and_lut(qg, bits, fmt, N, K):
    say(f"qgemv bits={bits} fmt={fmt} N={N} K={K}")
    W = synth.qmat(8, ("b", bits, fmt, N, K), N, K, bits, fmt)
    x = synth.activations(8, ("x", K), K, np.float16)
    ws = ws_for(qg, qg.QG_OP_GEMV, N, K)
    y = qg.qgemv(dev_mat(qg, W), to_dev(x), ws=ws)
    torch.cuda.synchronize()
    close(y.cpu().numpy(), oracle.gemv(W, x, nthreads=8), what="2bit/lut")


FMTS = [(4, synth.AFFINE), (2, synth.AFFINE), (4, synth.LUT)]


def fmt_tag(bits, fmt):
    return () if (bits, fmt) == (4, synth.AFFINE) else (bits, fmt)


@pytest.mark.parametrize("bits,fmt", FMTS)
@pytest.mark.parametrize("N,K", [(6144, 4096), (2048, 1024), (100, 14336)])
def test_qgemv_rmsnorm(qg, N, K, bits, fmt):
    """Includes the Llama QKV shape (6144 x 4096) in every format: the 2-bit
    and table-format stacks run exactly this launch."""
    say(f"qgemv_rmsnorm N={N} K={K} bits={bits} fmt={fmt}")
    W = synth.qmat(9, ("rn", N, K) + fmt_tag(bits, fmt), N, K, bits, fmt)
    g = synth.norm_weight(9, ("g", K), K)
    x = synth.activations(9, ("x", K), K, np.float32) * 3.0
    r = synth.activations(9, ("r", N), N, np.float32)
    ws = ws_for(qg, qg.QG_OP_GEMV_RMSNORM, N, K)
    rows = sample_rows(N)
    y = qg.qgemv_rmsnorm(dev_mat(qg, W), to_dev(x), to_dev(g), 1e-5, residual=to_dev(r), ws=ws)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_gemv(rows_of(W, rows), x, g, 1e-5, r[rows])
    close(y.cpu().numpy()[rows], ref, what="rmsnorm")


@pytest.mark.parametrize("bits,fmt", FMTS)
@pytest.mark.parametrize("F,K,norm", [(14336, 4096, True), (3072, 1024, True), (1000, 2048, False),
                                      (8, 64, True)])
def test_qswiglu(qg, F, K, norm, bits, fmt):
    """Includes the Llama gate.up shape (2 x 14336 x 4096, normed) in every
    format: the 2-bit and table-format stacks run exactly this launch."""
    say(f"qswiglu F={F} K={K} norm={norm} bits={bits} fmt={fmt}")
    Wg = synth.qmat(10, ("gate", F, K) + fmt_tag(bits, fmt), F, K, bits, fmt)
    Wu = synth.qmat(10, ("up", F, K) + fmt_tag(bits, fmt), F, K, bits, fmt)
    g = synth.norm_weight(10, ("g", K), K) if norm else None
    x = synth.activations(10, ("x", K), K, np.float32)
    ws = ws_for(qg, qg.QG_OP_SWIGLU, F, K)
    rows = sample_rows(F)
    u = qg.qswiglu(dev_mat(qg, Wg), dev_mat(qg, Wu), to_dev(x),
                   None if g is None else to_dev(g), 1e-5, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm_swiglu(rows_of(Wg, rows), rows_of(Wu, rows), x, g, 1e-5)
    close(u.cpu().numpy()[rows], ref, what="swiglu")


def test_residual_in_place(qg):
    N, K = 4096, 4096
    W = synth.qmat(12, "inplace", N, K, 4)
    x = synth.activations(12, "x", K, np.float32)
    r = synth.activations(12, "r", N, np.float32)
    rows = sample_rows(N)
    yd = to_dev(r.copy())
    qg.qgemv(dev_mat(qg, W), to_dev(x), residual=yd, y=yd)
    torch.cuda.synchronize()
    close(yd.cpu().numpy()[rows], oracle.gemv(rows_of(W, rows), x, r[rows]), what="in-place")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path", TOPK_PATHS)
def test_topk_ties_bit_exact(qg, path):
    """s = 0 and x = 1 make logit_n = 64 * b_n exactly; duplicate b give ties
    (and -0 ties +0: order by index, the value comes back with its sign)."""
    set_topk_path(qg, path)
    V, K, k = 5000, 64, 40
    W = synth.qmat(13, "ties", V, K, 4)
    W["scales"][:] = 0
    rng = np.random.default_rng(1)
    W["biases"][:, 0] = rng.choice(np.array([0.5, 0.25, -0.0, 0.0, 0.125], np.float16), V)
    x = np.ones(K, np.float32)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k, DEV)
    z, idx, vals = qg.qlogits_topk(dev_mat(qg, W), to_dev(x), k, ws=ws)
    torch.cuda.synchronize()
    zc = z.cpu().numpy()
    assert np.array_equal(zc, (64.0 * W["biases"][:, 0].astype(np.float64)).astype(np.float32))
    ridx, rvals = oracle.topk(zc, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32),
                          rvals.astype(np.float32).view(np.uint32))
    qg.qg_tune(5, 0)


@pytest.mark.parametrize("path", TOPK_PATHS)
@pytest.mark.parametrize("V,K,k,norm", [(151936, 1024, 40, True), (1000, 256, 1, False),
                                        (40, 128, 40, True), (9000, 64, 1024, False),
                                        (1, 64, 1, False), (151936, 1024, 64, False)])
def test_qlogits_topk(qg, V, K, k, norm, path):
    say(f"qlogits_topk V={V} K={K} k={k} {path}")
    set_topk_path(qg, path)
    W = synth.qmat(14, ("lm", V, K), V, K, 4)
    g = synth.norm_weight(14, "gf", K) if norm else None
    x = synth.activations(14, "x", K, np.float32) * 5.0
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k, DEV)
    z, idx, vals = qg.qlogits_topk(dev_mat(qg, W), to_dev(x), k,
                                   None if g is None else to_dev(g), 1e-5, ws=ws)
    torch.cuda.synchronize()
    zc = z.cpu().numpy()
    rows = sample_rows(V)
    ref = oracle.gemv(rows_of(W, rows), oracle.rmsnorm(x, g) if norm else x)
    close(zc[rows], ref, what="logits")
    ridx, rvals = oracle.topk(zc, k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(vals.cpu().numpy(), rvals.astype(np.float32))
    # a second call on the same workspace gives the same answer
    _, idx2, _ = qg.qlogits_topk(dev_mat(qg, W), to_dev(x), k,
                                 None if g is None else to_dev(g), 1e-5, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    qg.qg_tune(5, 0)


@pytest.mark.parametrize("op,N,K,bits,splits", [
    ("gemv", 4096, 14336, 4, 0), ("swiglu", 14336, 4096, 4, 0), ("rmsnorm", 6144, 4096, 2, 0),
    ("gemv", 1024, 3072, 4, 0), ("swiglu", 3072, 1024, 4, 0), ("gemv", 4096, 4096, 4, 2),
    ("gemv", 2048, 4096, 8, 0), ("swiglu", 1000, 2048, 2, 0), ("gemv", 1000, 4160, 4, 0),
    ("gemv", 3001, 14336, 4, 0)])
def test_staged_scale_rows_equal_per_pass_loads(qg, op, N, K, bits, splits):
    """Scale/bias rows staged in LDS per band (knob 6, 16-byte aligned rows)
    and the per-pass 2-byte loads give the same bits; both are the oracle's
    result within the bar. Includes two rows per lane (K = 14336), a second
    K slice starting mid-row, 2- and 8-bit codes and a K whose rows are not
    16-byte aligned (per-pass loads on both sides)."""
    say(f"staged scale rows {op} N={N} K={K} bits={bits} splits={splits}")
    W = synth.qmat(16, ("sbl", op, N, K, bits), N, K, bits)
    W2 = synth.qmat(16, ("sbl2", op, N, K, bits), N, K, bits) if op == "swiglu" else None
    g = synth.norm_weight(16, ("sblg", K), K)
    x = synth.activations(16, ("sblx", K), K, np.float32) * 2.0
    ws = ws_for(qg, qg.QG_OP_SWIGLU, N, K)
    Wd, W2d = dev_mat(qg, W), (dev_mat(qg, W2) if W2 is not None else None)
    xd, gd = to_dev(x), to_dev(g)
    outs = []
    qg.qg_tune(0, splits)
    try:
        for knob in (0, 1, 0):
            qg.qg_tune(6, knob)
            if op == "gemv":
                outs.append(qg.qgemv(Wd, xd, ws=ws))
            elif op == "rmsnorm":
                outs.append(qg.qgemv_rmsnorm(Wd, xd, gd, 1e-5, ws=ws))
            else:
                outs.append(qg.qswiglu(Wd, W2d, xd, gd, 1e-5, ws=ws))
    finally:
        qg.qg_tune(6, 0)
        qg.qg_tune(0, 0)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    rows = sample_rows(N, 200, 3)
    y = outs[0].cpu().numpy()
    if op == "gemv":
        ref = oracle.gemv(rows_of(W, rows), x)
    elif op == "rmsnorm":
        ref = oracle.rmsnorm_gemv(rows_of(W, rows), x, g, 1e-5)
    else:
        ref = oracle.rmsnorm_swiglu(rows_of(W, rows), rows_of(W2, rows), x, g, 1e-5)
    close(y[rows], ref, what=op)


def test_staged_scale_rows_moe_layer(qg):
    """The MoE layer (routed gate.up with staged rows of the chosen experts
    and the shared expert) gives the same bits with and without staging."""
    E, F, H, K = 64, 1024, 4096, 3
    say("staged scale rows: moe layer")
    gate, up, down, shared = moe_weights(17, E, F, H)
    g = synth.norm_weight(17, "g", H)
    lg = synth.router_logits(17, "route", E)
    x = synth.activations(17, "x", H, np.float32)
    Gd, Ud, Dd = (dev_mat(qg, W) for W in (gate, up, down))
    Sd = tuple(dev_mat(qg, W) for W in shared)
    ws = qg.workspace(qg.QG_OP_MOE, H, F, 1, 4, 0, K, DEV)
    ys = []
    try:
        for knob in (0, 1):
            qg.qg_tune(6, knob)
            ys.append(qg.qmoe_experts(Gd, Ud, Dd, E, Sd, to_dev(lg), K, to_dev(x), to_dev(g), 1e-5,
                                      ws=ws))
    finally:
        qg.qg_tune(6, 0)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    yref, _, _ = oracle.moe_layer(gate, up, down, shared, lg, K, x, g, 1e-5, nthreads=8)
    close(ys[1].cpu().numpy(), yref, what="moe")


def test_handoff_under_alternating_inputs(qg):
    """The hand-off between workgroups of one launch (split-K partials and
    their tickets; the one-launch top-k's lists, tickets and logit reloads)
    uses agent-coherent stores and loads and relaxed integer tickets. Two
    inputs alternate over 48 calls replayed from a graph: the partials, lists
    and tickets sit at the same workspace addresses in every call, so a read
    that saw the previous call's data instead of its own would change that
    call's result. Every call must give the same bits as the first call on
    its input."""
    say("hand-off stress: split-K and one-launch top-k, alternating inputs")
    N, K = 4096, 16384
    W = dev_mat(qg, synth.qmat(18, "handoff", N, K, 4))
    xs = [to_dev(synth.activations(18, ("hox", i), K, np.float32)) for i in range(2)]
    ws = ws_for(qg, qg.QG_OP_SWIGLU, N, K)
    V, KH, k = 151936, 1024, 40
    H = dev_mat(qg, synth.qmat(18, "handoff_head", V, KH, 4))
    hx = [to_dev(synth.activations(18, ("hhx", i), KH, np.float32) * 4.0) for i in range(2)]
    wsh = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, KH, 1, 4, 0, k, DEV)
    n = 48
    ys = [torch.empty(N, dtype=torch.float32, device=DEV) for _ in range(n)]
    zs = [torch.empty(V, dtype=torch.float32, device=DEV) for _ in range(n)]
    ids = [torch.empty(k, dtype=torch.int32, device=DEV) for _ in range(n)]
    vs = [torch.empty(k, dtype=torch.float32, device=DEV) for _ in range(n)]
    try:
        def calls():
            for i in range(n):
                qg.qg_tune(0, 4)  # the matvec in four K slices (planned at the call)
                qg.qgemv(W, xs[i % 2], y=ys[i], ws=ws)
                qg.qg_tune(0, 0)  # the head in one launch
                qg.qlogits_topk(H, hx[i % 2], k, logits=zs[i], idx=ids[i], vals=vs[i], ws=wsh)
        calls()
        torch.cuda.synchronize()
        refs = [(ys[j].clone(), ids[j].clone(), vs[j].clone(), zs[j].clone()) for j in range(2)]
        for i in range(n):
            r = refs[i % 2]
            assert torch.equal(ys[i], r[0]) and torch.equal(ids[i], r[1]) and torch.equal(vs[i], r[2])
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            calls()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            for i in range(n):
                r = refs[i % 2]
                assert torch.equal(ys[i], r[0]), f"replay {rep} call {i}: split-K result"
                assert torch.equal(ids[i], r[1]) and torch.equal(vs[i], r[2]), f"replay {rep} call {i}: top-k"
                assert torch.equal(zs[i], r[3]), f"replay {rep} call {i}: logits"
    finally:
        qg.qg_tune(0, 0)
    assert not torch.equal(refs[0][0], refs[1][0]) and not torch.equal(refs[0][1], refs[1][1])
    ridx, _ = oracle.topk(refs[0][3].cpu().numpy(), k)
    assert np.array_equal(refs[0][1].cpu().numpy(), ridx)
    assert qg.qg_logits_topk_launches(V, KH, k, W=H) == 1


def test_topk_launch_count(qg):
    """One launch for the Qwen-shaped head at k <= 64, two past 64 keys, for
    more rows per wave than a key list holds, and under knob 5."""
    assert qg.qg_logits_topk_launches(151936, 1024, 40) == 1
    assert qg.qg_logits_topk_launches(151936, 1024, 64) == 1
    assert qg.qg_logits_topk_launches(151936, 1024, 65) == 2
    assert qg.qg_logits_topk_launches(300007, 64, 8) == 2
    qg.qg_tune(5, 1)
    try:
        assert qg.qg_logits_topk_launches(151936, 1024, 40) == 2
    finally:
        qg.qg_tune(5, 0)


@pytest.mark.parametrize("bits,fmt", FMTS + [(8, synth.AFFINE), (16, synth.DENSE)])
@pytest.mark.parametrize("V,K,k", [(20011, 512, 64), (300007, 64, 8), (4099, 4096, 17)])
def test_topk_one_launch_equals_two(qg, bits, fmt, V, K, k):
    """Every weight format, ragged vocabularies: the one-launch head gives the
    same logits, indices and values, bit for bit, as the matvec followed by
    the separate top-k, and its indices are the oracle's top-k of those
    logits. 300007 x 64 has more rows per wave than one key list holds, so it
    takes the two-launch form on both sides."""
    say(f"topk one vs two launches V={V} K={K} k={k} bits={bits} fmt={fmt}")
    W = dev_mat(qg, synth.qmat(15, ("tk1", V, K) + fmt_tag(bits, fmt), V, K, bits, fmt))
    x = to_dev(synth.activations(15, ("tk1x", K), K, np.float32) * 3.0)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, bits, fmt, k, DEV)
    out = []
    for path in ("one_launch", "two_launch", "one_launch"):
        set_topk_path(qg, path)
        out.append(qg.qlogits_topk(W, x, k, ws=ws))
    qg.qg_tune(5, 0)
    torch.cuda.synchronize()
    for (z, i, v) in out[1:]:
        assert torch.equal(z, out[0][0]) and torch.equal(i, out[0][1]) and torch.equal(v, out[0][2])
    zc = out[0][0].cpu().numpy()
    ridx, rvals = oracle.topk(zc, k)
    assert np.array_equal(out[0][1].cpu().numpy(), ridx)
    assert np.array_equal(out[0][2].cpu().numpy(), rvals.astype(np.float32))


# ---------------------------------------------------------------------------
def moe_weights(seed, E, F, H):
    gate = synth.qmat(seed, "gate_all", E * F, H, 4)
    up = synth.qmat(seed, "up_all", E * F, H, 4)
    down = synth.qmat(seed, "down_all", E * H, F, 4)
    for Wt in (gate, up, down):
        Wt["E"] = E
    shared = (synth.qmat(seed, "sh_gate", F, H, 4), synth.qmat(seed, "sh_up", F, H, 4),
              synth.qmat(seed, "sh_down", H, F, 4))
    return gate, up, down, shared


@pytest.mark.parametrize("E,F,H,top_k,shared", [(16, 128, 256, 3, True), (8, 64, 128, 1, False),
                                                (512, 1024, 4096, 3, True), (16, 128, 256, 8, True),
                                                (12, 64, 192, 8, False), (3, 8192, 256, 3, True)])
def test_qmoe_experts(qg, E, F, H, top_k, shared):
    """Includes top_k = 8 with the shared expert (nine gathered matrices in one
    launch) and F = 8192 with three routed experts + the shared one, whose
    K-concatenated down projection (32768 codes) is split across workgroups."""
    say(f"qmoe_experts E={E} F={F} H={H} top_k={top_k}")
    gate, up, down, sh = moe_weights(15, E, F, H)
    g = synth.norm_weight(15, "g", H)
    x = synth.activations(15, "x", H, np.float32)
    Gd, Ud, Dd = dev_mat(qg, gate), dev_mat(qg, up), dev_mat(qg, down)
    shd = tuple(dev_mat(qg, m) for m in sh) if shared else None
    ws = qg.workspace(qg.QG_OP_MOE, H, F, 1, 4, 0, top_k, DEV)
    for draw in range(3):
        lg = synth.router_logits(15, ("route", draw), E)
        ids = torch.empty(top_k, dtype=torch.int32, device=DEV)
        w = torch.empty(top_k, dtype=torch.float32, device=DEV)
        y = qg.qmoe_experts(Gd, Ud, Dd, E, shd, to_dev(lg), top_k, to_dev(x), to_dev(g), 1e-5,
                            sel_ids=ids, sel_w=w, ws=ws)
        torch.cuda.synchronize()
        yref, rid, rw = oracle.moe_layer(gate, up, down, sh if shared else None, lg, top_k, x, g,
                                         nthreads=8)
        assert np.array_equal(ids.cpu().numpy(), rid)
        close(w.cpu().numpy(), rw, tol=1e-6, what="routing weights")
        close(y.cpu().numpy(), yref, what="moe")


# ---------------------------------------------------------------------------
def test_llama_layer_full_size(qg):
    """One Llama-3-8B-shaped decode layer through the four fused calls."""
    say("llama layer full size")
    model = synth.LLAMA3_8B
    w = synth.layer_weights(1234, model, 0)
    H = model["hidden"]
    x = synth.activations(1234, "x0", H, np.float32)
    d = {k: dev_mat(qg, v) for k, v in w.items() if isinstance(v, dict)}
    ws = qg.workspace(qg.QG_OP_SWIGLU, model["ffn"], H, 1, 4, 0, 1, DEV)
    xd = to_dev(x)
    qkv = qg.qgemv_rmsnorm(d["qkv"], xd, to_dev(w["g_attn"]), 1e-5, ws=ws)
    h = qg.qgemv(d["o"], qkv[:model["q_dim"]], residual=xd, ws=ws)
    u = qg.qswiglu(d["gate"], d["up"], h, to_dev(w["g_ffn"]), 1e-5, ws=ws)
    y = qg.qgemv(d["down"], u, residual=h, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.decoder_layer(w, x, model["q_dim"], 1e-5, nthreads=8)
    close(y.cpu().numpy(), ref, what="layer")


@pytest.mark.parametrize("tp", [2, 8])
def test_llama_tp_shard_layer(qg, tp):
    """One GPU's shard of the Llama-3-8B-shaped layer under tensor
    parallelism (qkv 6144/tp rows, o 4096 x 4096/tp, gate.up 14336/tp rows,
    down 4096 x 14336/tp): the four fused calls at those shapes, each against
    the oracle on its own input (the all-reduces are outside the path)."""
    say(f"llama tp{tp} shard layer")
    model = synth.tp_shard(synth.LLAMA3_8B, tp)
    w = synth.layer_weights(1234, model, 0)
    H, QD = model["hidden"], model["q_dim"]
    x = synth.activations(1234, ("x0", tp), H, np.float32)
    d = {k: dev_mat(qg, v) for k, v in w.items() if isinstance(v, dict)}
    ws = qg.workspace(qg.QG_OP_SWIGLU, max(model["ffn"], H), H, 1, 4, 0, 1, DEV)
    xd = to_dev(x)
    qkv = qg.qgemv_rmsnorm(d["qkv"], xd, to_dev(w["g_attn"]), 1e-5, ws=ws)
    h = qg.qgemv(d["o"], qkv[:QD], residual=xd, ws=ws)
    u = qg.qswiglu(d["gate"], d["up"], h, to_dev(w["g_ffn"]), 1e-5, ws=ws)
    y = qg.qgemv(d["down"], u, residual=h, ws=ws)
    torch.cuda.synchronize()
    qkv_h, h_h, u_h = qkv.cpu().numpy(), h.cpu().numpy(), u.cpu().numpy()
    close(qkv_h, oracle.rmsnorm_gemv(w["qkv"], x, w["g_attn"], 1e-5, nthreads=8), what="qkv")
    close(h_h, oracle.gemv(w["o"], qkv_h[:QD].astype(np.float64), x, nthreads=8), what="o")
    close(u_h, oracle.rmsnorm_swiglu(w["gate"], w["up"], h_h.astype(np.float64), w["g_ffn"], 1e-5,
                                     nthreads=8), what="gate.up")
    close(y.cpu().numpy(), oracle.gemv(w["down"], u_h.astype(np.float64), h_h, nthreads=8),
          what="down")


def test_graph_replay_matches_eager(qg):
    """Two Llama-shaped layers captured in a HIP graph, replayed several times
    with eager work between the replays; every replay equals the eager run."""
    model = dict(synth.LLAMA3_8B)
    H, QD = model["hidden"], model["q_dim"]
    ws_ = [synth.layer_weights(77, model, li) for li in range(2)]
    layers = []
    for w in ws_:
        d = {k: dev_mat(qg, v) for k, v in w.items() if isinstance(v, dict)}
        d["ga"], d["gf"] = to_dev(w["g_attn"]), to_dev(w["g_ffn"])
        layers.append(d)
    ws = ws_for(qg, qg.QG_OP_SWIGLU, model["ffn"], H)
    x0 = to_dev(synth.activations(77, "x0", H, np.float32))
    x = torch.empty_like(x0)
    qkv = torch.empty(model["qkv"], dtype=torch.float32, device=DEV)
    h = torch.empty(H, dtype=torch.float32, device=DEV)
    u = torch.empty(model["ffn"], dtype=torch.float32, device=DEV)

    def token():
        x.copy_(x0)
        for d in layers:
            qg.qgemv_rmsnorm(d["qkv"], x, d["ga"], 1e-5, y=qkv, ws=ws)
            qg.qgemv(d["o"], qkv[:QD], residual=x, y=h, ws=ws)
            qg.qswiglu(d["gate"], d["up"], h, d["gf"], 1e-5, u=u, ws=ws)
            qg.qgemv(d["down"], u, residual=h, y=x, ws=ws)

    token()
    torch.cuda.synchronize()
    eager = x.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        token()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        token()
    for rep in range(4):
        x.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, eager), f"replay {rep}"
        token()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(x, eager)


@pytest.mark.parametrize("bits,fmt", [(4, synth.AFFINE), (2, synth.AFFINE), (4, synth.LUT)])
@pytest.mark.parametrize("K", [20480, 65536])
@pytest.mark.parametrize("norm", [False, True])
def test_long_k_staging_rounds(qg, bits, fmt, K, norm):
    """K beyond 512 quarter units per slice: x is staged in several uniform
    rounds, and beyond the LDS slice K is split across workgroups."""
    N = 300
    say(f"long K bits={bits} fmt={fmt} K={K} norm={norm}")
    W = synth.qmat(31, ("longk", bits, fmt, K), N, K, bits, fmt)
    x = synth.activations(31, ("x", K), K, np.float32)
    g = synth.norm_weight(31, ("g", K), K) if norm else None
    ws = qg.workspace(qg.QG_OP_GEMV_RMSNORM, N, K, 1, bits, fmt, 1, DEV)
    Wd = dev_mat(qg, W)
    if norm:
        y = qg.qgemv_rmsnorm(Wd, to_dev(x), to_dev(g), 1e-5, ws=ws)
        ref = oracle.rmsnorm_gemv(W, x, g, 1e-5, nthreads=8)
    else:
        y = qg.qgemv(Wd, to_dev(x), ws=ws)
        ref = oracle.gemv(W, x, nthreads=8)
    torch.cuda.synchronize()
    close(y.cpu().numpy(), ref, what="long K")


@pytest.mark.parametrize("E,F,H,top_k,M,shared,bits,seed", [(16, 128, 256, 3, 5, True, 4, 33),
                                                            (16, 128, 256, 8, 3, True, 4, 33),
                                                            (8, 64, 128, 1, 2, False, 4, 33),
                                                            (512, 1024, 4096, 3, 8, True, 4, 33),
                                                            (16, 1024, 4096, 3, 4, True, 8, 28)])
def test_qmoe_experts_batch(qg, E, F, H, top_k, M, shared, bits, seed):
    """M tokens in one call: each token's output is bitwise that of the
    single-token call, and its routing, weights and output match the oracle's
    MoE layer for that token alone. (The 8-bit case uses the input family of
    the single-token 8-bit test: token 1 of the seed-33 family cancels its
    experts' contributions down to 1/60 of the other tokens' outputs and
    lands at 2.3e-3 in one call as in the batch.)"""
    say(f"qmoe_experts_batch E={E} F={F} H={H} top_k={top_k} M={M} bits={bits}")
    gate = synth.qmat(seed, "gate_all", E * F, H, bits)
    up = synth.qmat(seed, "up_all", E * F, H, bits)
    down = synth.qmat(seed, "down_all", E * H, F, bits)
    for Wt in (gate, up, down):
        Wt["E"] = E
    sh = (synth.qmat(seed, "sh_gate", F, H, bits), synth.qmat(seed, "sh_up", F, H, bits),
          synth.qmat(seed, "sh_down", H, F, bits))
    g = synth.norm_weight(seed, "g", H)
    X = synth.activations(seed, "xb", (M, H), np.float32)
    lg = synth.router_logits(seed, "routeb", (M, E))
    Gd, Ud, Dd = dev_mat(qg, gate), dev_mat(qg, up), dev_mat(qg, down)
    shd = tuple(dev_mat(qg, m) for m in sh) if shared else None
    ws = qg.workspace(qg.QG_OP_MOE, H, F, M, bits, 0, top_k, DEV)
    ids = torch.empty((M, top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((M, top_k), dtype=torch.float32, device=DEV)
    y = qg.qmoe_experts_batch(Gd, Ud, Dd, E, shd, to_dev(lg), top_k, to_dev(X), to_dev(g), 1e-5,
                              sel_ids=ids, sel_w=w, ws=ws)
    torch.cuda.synchronize()
    yc, ic, wc = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    for m in range(M):
        ys = qg.qmoe_experts(Gd, Ud, Dd, E, shd, to_dev(lg[m]), top_k, to_dev(X[m]), to_dev(g), 1e-5,
                             ws=ws)
        assert torch.equal(ys, y[m]), f"token {m}: batch differs from the single-token call"
    for m in range(M):
        yref, rid, rw = oracle.moe_layer(gate, up, down, sh if shared else None, lg[m], top_k, X[m],
                                         g, nthreads=8)
        assert np.array_equal(ic[m], rid), f"token {m} routing"
        close(wc[m], rw, tol=1e-6, what=f"token {m} routing weights")
        close(yc[m], yref, what=f"token {m} moe")
    # in place (y is x), and token 0 alone through qmoe_experts gives the same bits
    xin = to_dev(X)
    qg.qmoe_experts_batch(Gd, Ud, Dd, E, shd, to_dev(lg), top_k, xin, to_dev(g), 1e-5, y=xin, ws=ws)
    y0 = qg.qmoe_experts(Gd, Ud, Dd, E, shd, to_dev(lg[0]), top_k, to_dev(X[0]), to_dev(g), 1e-5,
                         ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(xin, y), "in-place batch differs"
    assert torch.equal(y0, y[0]), "token 0 alone differs"


def test_qmoe_batch_refused_enqueues_nothing(qg):
    """A batch whose concatenated down projection needs split-K is refused
    (QG_EUNSUPPORTED) before either launch is enqueued: the routing outputs
    keep their previous contents."""
    E, F, H, top_k, M = 3, 8192, 256, 3, 2
    say("qmoe_experts_batch refused case")
    gate, up, down, sh = moe_weights(16, E, F, H)
    Gd, Ud, Dd = dev_mat(qg, gate), dev_mat(qg, up), dev_mat(qg, down)
    shd = tuple(dev_mat(qg, m) for m in sh)
    X = synth.activations(16, "xb", (M, H), np.float32)
    lg = synth.router_logits(16, "routeb", (M, E))
    ws = qg.workspace(qg.QG_OP_MOE, H, F, M, 4, 0, top_k, DEV)
    ids = torch.full((M, top_k), -7, dtype=torch.int32, device=DEV)
    w = torch.full((M, top_k), -7.0, dtype=torch.float32, device=DEV)
    xd = to_dev(X)
    y = torch.full((M, H), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(qg.QgError) as ei:
        qg.qmoe_experts_batch(Gd, Ud, Dd, E, shd, to_dev(lg), top_k, xd, None, 1e-5, y=y,
                              sel_ids=ids, sel_w=w, ws=ws)
    assert ei.value.status == qg.QG_EUNSUPPORTED
    torch.cuda.synchronize()
    assert bool((ids == -7).all()) and bool((w == -7.0).all()) and bool((y == 3.0).all())
