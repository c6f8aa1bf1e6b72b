"""Pins for the CPU oracle: every check compares it with something other than
itself (hand-computed values, closed forms, invariants, library routines,
brute force on tiny inputs). CPU only."""

import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Independent packer: field j of each word holds codes[..., j]."""
    per = 32 // bits
    c = codes.astype(np.uint64).reshape(codes.shape[0], -1, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    return (c << shifts).sum(axis=-1).astype(np.uint32)


def make_mat(codes, bits, scales=None, biases=None, lut=None, group=64):
    N, K = codes.shape
    fmt = synth.LUT if lut is not None else synth.AFFINE
    return {"N": N, "K": K, "bits": bits, "fmt": fmt, "group": group,
            "q": pack_codes(codes, bits),
            "scales": None if scales is None else np.asarray(scales, np.float16),
            "biases": None if biases is None else np.asarray(biases, np.float16),
            "lut": None if lut is None else np.asarray(lut, np.float16)}


def const_mat(N, K, bits, word, scale, bias, group=64):
    per_row = K * bits // 32
    return {"N": N, "K": K, "bits": bits, "fmt": synth.AFFINE, "group": group,
            "q": np.full((N, per_row), word, np.uint32),
            "scales": np.full((N, K // group), scale, np.float16),
            "biases": np.full((N, K // group), bias, np.float16), "lut": None}


# ---------------------------------------------------------------------------
def test_half_decoder_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (got == ref))
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


@pytest.mark.parametrize("case", GOLDEN["unpack"])
def test_unpack_hand_words(case):
    bits = case["bits"]
    per = 32 // bits
    W = const_mat(1, 64, bits, int(case["word"], 16), 1.0, 0.0)
    codes = oracle.unpack(W)[0]
    for w in range(64 // per):
        assert list(codes[w * per:(w + 1) * per]) == case["codes"]


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_unpack_roundtrip_independent_packer(bits):
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 1 << bits, size=(5, 192), dtype=np.uint8)
    W = make_mat(codes, bits, np.ones((5, 3)), np.zeros((5, 3)))
    assert np.array_equal(oracle.unpack(W), codes)
    # and the other way: random words survive unpack -> pack
    W2 = synth.qmat(3, "rt", 4, 256, bits)
    assert np.array_equal(pack_codes(oracle.unpack(W2), bits), W2["q"])


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_dequant_special_cases(bits):
    rng = np.random.default_rng(11)
    N, K = 6, 256
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = synth.uniform(rng, (N, K // 64), 0.005, 0.02)
    b = synth.uniform(rng, (N, K // 64), -0.1, 0.1)
    ones = np.ones((N, K // 64), np.float16)
    zeros = np.zeros((N, K // 64), np.float16)
    # s=1, b=0: the weights are the codes
    assert np.array_equal(oracle.dequant(make_mat(codes, bits, ones, zeros)), codes)
    # s=0: every weight of a group is its bias (64 consecutive k of one row)
    Wb = oracle.dequant(make_mat(codes, bits, zeros, b))
    assert np.array_equal(Wb, np.repeat(b.astype(np.float64), 64, axis=1))
    # codes all 1, b=0: every weight of a group is its scale
    Ws = oracle.dequant(make_mat(np.ones_like(codes), bits, s, zeros))
    assert np.array_equal(Ws, np.repeat(s.astype(np.float64), 64, axis=1))
    # the affine form is additive in (s, b) and exact in double
    W = oracle.dequant(make_mat(codes, bits, s, b))
    W0 = oracle.dequant(make_mat(codes, bits, s, zeros))
    assert np.array_equal(W, W0 + Wb)
    # round trip: the codes are recovered from the dequantized weights
    rec = np.rint((W - np.repeat(b.astype(np.float64), 64, 1)) / np.repeat(s.astype(np.float64), 64, 1))
    assert np.array_equal(rec, codes)


def test_dequant_lut():
    rng = np.random.default_rng(12)
    N, K = 3, 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    ident = np.tile(np.arange(16, dtype=np.float16), (N, 1))
    assert np.array_equal(oracle.dequant(make_mat(codes, 4, lut=ident)), codes)
    lut = synth.normal(rng, (N, 16), 0.0, 0.02)
    W = oracle.dequant(make_mat(codes, 4, lut=lut))
    for n in range(N):
        for k in range(K):
            assert W[n, k] == float(lut[n, codes[n, k]])


@pytest.mark.parametrize("case", GOLDEN["gemv"])
def test_gemv_hand_cases(case):
    W = const_mat(1, case["K"], case["bits"], int(case["word"], 16), case["scale"], case["bias"])
    x = np.ones(case["K"]) if case["x"] == "ones" else np.tile([1.0, -1.0], case["K"] // 2)
    assert oracle.gemv(W, x)[0] == case["y"]


def dense_mat(K, word, N=1):
    return {"N": N, "K": K, "bits": 16, "fmt": synth.DENSE, "group": 64,
            "q": np.full((N, K // 2), word, np.uint32), "scales": None, "biases": None, "lut": None}


@pytest.mark.parametrize("case", GOLDEN["dense"])
def test_dense_hand_cases(case):
    x = np.ones(case["K"]) if case["x"] == "ones" else np.tile([1.0, -1.0], case["K"] // 2)
    assert oracle.gemv(dense_mat(case["K"], int(case["word"], 16)), x)[0] == case["y"]


def test_dense_matches_numpy_fp16():
    """The dense format's weights are numpy's own reading of the row bytes as
    little-endian fp16, and the matvec is numpy's matmul of them."""
    W = synth.qmat(5, "dense", 29, 192, 16, synth.DENSE)
    ref = W["q"].view(np.float16).astype(np.float64)
    assert ref.shape == (29, 192)
    assert np.array_equal(oracle.dequant(W), ref)
    X = synth.activations(5, "densex", (2, 192), np.float32)
    np.testing.assert_allclose(oracle.gemv(W, X), X.astype(np.float64) @ ref.T, rtol=1e-12, atol=1e-12)
    # every fp16 pattern of one word decodes as numpy does (field 0 = low half)
    pats = np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xC000, 0xFBFF], np.uint16)
    words = pats[::2].astype(np.uint32) | (pats[1::2].astype(np.uint32) << 16)
    D = {"N": 1, "K": 8, "bits": 16, "fmt": synth.DENSE, "group": 64, "q": words[None, :],
         "scales": None, "biases": None, "lut": None}
    assert np.array_equal(oracle.dequant(D)[0], pats.view(np.float16).astype(np.float64))


def test_dense_rejects_codes_and_other_widths():
    W = synth.qmat(1, "dbad", 2, 64, 16, synth.DENSE)
    with pytest.raises(ValueError):
        oracle.unpack(W)
    W["bits"] = 8
    with pytest.raises(ValueError):
        oracle.gemv(W, np.ones(64))


def test_gemv_power256_probe_decodes_8bit_codes():
    """s=1, b=0 and x = 256^j at three columns: y_n spells out three 8-bit
    codes (every partial sum is an integer below 2^24)."""
    W = synth.qmat(9, "p256", 40, 192, 8)
    W["scales"][:] = 1
    W["biases"][:] = 0
    codes = oracle.unpack(W)
    cols = [5, 64, 191]
    x = np.zeros(192)
    for j, c in enumerate(cols):
        x[c] = 256.0 ** j
    y = oracle.gemv(W, x).astype(np.int64)
    for j, c in enumerate(cols):
        assert np.array_equal((y >> (8 * j)) & 255, codes[:, c])


@pytest.mark.parametrize("bits,fmt", [(4, synth.AFFINE), (2, synth.AFFINE), (4, synth.LUT),
                                      (8, synth.AFFINE)])
def test_gemv_matches_library_matmul(bits, fmt):
    W = synth.qmat(5, ("mm", bits, fmt), 37, 320, bits, fmt)
    X = synth.activations(5, "mmx", (3, 320), np.float32)
    dense = oracle.dequant(W)
    ref = np.matmul(X.astype(np.float64), dense.T)
    got = oracle.gemv(W, X)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # rows are independent of the thread split
    assert np.array_equal(oracle.gemv(W, X, nthreads=4), got)
    # each activation vector alone gives the same row
    for m in range(3):
        assert np.array_equal(oracle.gemv(W, X[m]), got[m])


def test_gemv_power16_probe_decodes_codes():
    """s=1, b=0 and x = 16^j at four columns: y_n spells out the four codes."""
    W = synth.qmat(9, "p16", 50, 128, 4)
    W["scales"][:] = 1
    W["biases"][:] = 0
    codes = oracle.unpack(W)
    cols = [3, 64, 70, 127]
    x = np.zeros(128)
    for j, c in enumerate(cols):
        x[c] = 16.0 ** j
    y = oracle.gemv(W, x).astype(np.int64)
    for j, c in enumerate(cols):
        assert np.array_equal((y >> (4 * j)) & 15, codes[:, c])


def test_gemv_all_ones_closed_form():
    W = synth.qmat(4, "ones", 20, 256, 4)
    codes = oracle.unpack(W).astype(np.float64)
    s = W["scales"].astype(np.float64)
    b = W["biases"].astype(np.float64)
    gsum = codes.reshape(20, 4, 64).sum(-1)
    ref = (s * gsum + 64 * b).sum(-1)
    np.testing.assert_allclose(oracle.gemv(W, np.ones(256)), ref, rtol=1e-13)


def test_gemv_zero_scale_is_bias_times_group_sums():
    W = synth.qmat(4, "s0", 10, 256, 4)
    W["scales"][:] = 0
    x = synth.activations(4, "s0x", 256, np.float32).astype(np.float64)
    ref = (W["biases"].astype(np.float64) * x.reshape(4, 64).sum(-1)).sum(-1)
    np.testing.assert_allclose(oracle.gemv(W, x), ref, rtol=1e-12, atol=1e-14)


def test_gemv_residual_and_linearity():
    W = synth.qmat(6, "lin", 16, 128, 4)
    x1 = synth.activations(6, "x1", 128, np.float32).astype(np.float64)
    x2 = synth.activations(6, "x2", 128, np.float32).astype(np.float64)
    r = synth.activations(6, "r", 16, np.float32).astype(np.float64)
    y1, y2 = oracle.gemv(W, x1), oracle.gemv(W, x2)
    np.testing.assert_allclose(oracle.gemv(W, x1 + x2), y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.gemv(W, x1, r), y1 + r, rtol=1e-15, atol=1e-15)


def test_oracle_rejects_bad_shapes():
    W = synth.qmat(1, "bad", 4, 128, 4)
    W["K"] = 100
    with pytest.raises(ValueError):
        oracle.gemv(W, np.ones(100))
    W = synth.qmat(1, "bad", 4, 128, 4)
    W["bits"] = 3
    with pytest.raises(ValueError):
        oracle.gemv(W, np.ones(128))


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", GOLDEN["rmsnorm"])
def test_rmsnorm_hand_case(case):
    got = oracle.rmsnorm(case["x"], np.asarray(case["g"], np.float16), case["eps"])
    np.testing.assert_allclose(got, case["y"], rtol=1e-15)


def test_rmsnorm_closed_forms():
    g = synth.norm_weight(2, "g", 64)
    c = 0.37
    got = oracle.rmsnorm(np.full(64, c), g, 1e-5)
    np.testing.assert_allclose(got, g.astype(np.float64) * c / np.sqrt(c * c + 1e-5), rtol=1e-14)
    x = synth.activations(2, "x", 333, np.float32).astype(np.float64)
    out = oracle.rmsnorm(x, np.ones(333, np.float16), 0.0)
    assert abs(np.mean(out ** 2) - 1.0) < 1e-13
    assert np.array_equal(np.sign(out), np.sign(x))


def test_silu_library():
    for z in [-30.0, -3.5, -1.0, -1e-3, 0.0, 1e-3, 0.5, 2.0, 17.0]:
        assert oracle.silu(z) == pytest.approx(z * scipy.special.expit(z), rel=1e-15, abs=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_swiglu_closed_forms():
    K, F = 128, 12
    x = synth.activations(3, "x", K, np.float32).astype(np.float64)
    Wg = synth.qmat(3, "g", F, K, 4)
    Wu = synth.qmat(3, "u", F, K, 4)
    # zero gate weights: silu(0) = 0 kills every output
    Z = dict(Wg, scales=np.zeros_like(Wg["scales"]), biases=np.zeros_like(Wg["biases"]))
    assert np.array_equal(oracle.swiglu(Z, Wu, x), np.zeros(F))
    # constant gate weight b: a_j = b * sum(x) for every row
    C = dict(Wg, scales=np.zeros_like(Wg["scales"]), biases=np.full_like(Wg["biases"], 0.25))
    a = 0.25 * x.sum()
    c = oracle.gemv(Wu, x)
    np.testing.assert_allclose(oracle.swiglu(C, Wu, x), a * scipy.special.expit(a) * c, rtol=1e-12)
    # general: silu of one pinned matvec times another
    ref = oracle.gemv(Wg, x)
    np.testing.assert_allclose(oracle.swiglu(Wg, Wu, x), ref * scipy.special.expit(ref) * c,
                               rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", GOLDEN["topk"])
def test_topk_hand_cases(case):
    idx, _ = oracle.topk(case["z"], case["k"])
    assert list(idx) == case["idx"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 300))
    z = rng.integers(-5, 6, size=V).astype(np.float64)  # many ties
    k = int(rng.integers(1, V + 1))
    order = np.lexsort((np.arange(V), -z))
    idx, vals = oracle.topk(z, k)
    assert np.array_equal(idx, order[:k])
    assert np.array_equal(vals, z[order[:k]])


def test_topk_nan_last():
    idx, _ = oracle.topk([np.nan, 1.0, -np.inf, np.nan], 4)
    assert list(idx) == [1, 2, 0, 3]


def test_route_equal_and_softmax():
    ids, w = oracle.route(np.zeros(512), 3)
    assert list(ids) == [0, 1, 2]
    np.testing.assert_allclose(w, [1 / 3] * 3, rtol=1e-15)
    lg = synth.router_logits(1, "r", 512).astype(np.float64)
    ids, w = oracle.route(lg, 3)
    assert np.array_equal(ids, np.lexsort((np.arange(512), -lg))[:3])
    np.testing.assert_allclose(w, scipy.special.softmax(lg[ids]), rtol=1e-14)
    assert abs(w.sum() - 1) < 1e-15


# ---------------------------------------------------------------------------
def _experts(seed, E, F, H):
    gate = synth.qmat(seed, "gate", E * F, H, 4)
    up = synth.qmat(seed, "up", E * F, H, 4)
    down = synth.qmat(seed, "down", E * H, F, 4)
    for W in (gate, up, down):
        W["E"] = E
    return gate, up, down


def test_moe_zero_experts_is_identity():
    E, F, H = 6, 64, 128
    gate, up, down = _experts(1, E, F, H)
    down["scales"][:] = 0
    down["biases"][:] = 0
    x = synth.activations(1, "x", H, np.float32).astype(np.float64)
    lg = synth.router_logits(1, "l", E)
    y, ids, w = oracle.moe_layer(gate, up, down, None, lg, 3, x, None)
    assert np.array_equal(y, x)


def test_moe_k_concatenation_identity():
    """sum_e w_e D_e u_e equals one matvec over the K-concatenated experts."""
    E, F, H = 5, 64, 128
    gate, up, down = _experts(2, E, F, H)
    shared = tuple(synth.qmat(2, ("sh", t), *s, 4) for t, s in
                   (("g", (F, H)), ("u", (F, H)), ("d", (H, F))))
    x = synth.activations(2, "x", H, np.float32).astype(np.float64)
    g = synth.norm_weight(2, "g", H)
    lg = synth.router_logits(2, "l", E)
    y, ids, w = oracle.moe_layer(gate, up, down, shared, lg, 3, x, g)
    xn = oracle.rmsnorm(x, g)
    parts, mats = [], []
    for e, we in zip(ids, w):
        u = oracle.swiglu(oracle.expert_slice(gate, e), oracle.expert_slice(up, e), xn)
        parts.append(we * u)
        mats.append(oracle.expert_slice(down, e))
    parts.append(oracle.swiglu(shared[0], shared[1], xn))
    mats.append(shared[2])
    cat = {"N": H, "K": F * len(mats), "bits": 4, "fmt": synth.AFFINE, "group": 64,
           "q": np.hstack([m["q"] for m in mats]),
           "scales": np.hstack([m["scales"] for m in mats]),
           "biases": np.hstack([m["biases"] for m in mats]), "lut": None}
    ref = x + oracle.gemv(cat, np.concatenate(parts))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_moe_single_expert_closed_form():
    E, F, H = 4, 64, 128
    gate, up, down = _experts(3, E, F, H)
    x = synth.activations(3, "x", H, np.float32).astype(np.float64)
    lg = np.array([0.1, 2.0, -1.0, 0.3])
    y, ids, w = oracle.moe_layer(gate, up, down, None, lg, 1, x, None)
    assert list(ids) == [1] and w[0] == 1.0
    u = oracle.swiglu(oracle.expert_slice(gate, 1), oracle.expert_slice(up, 1), x)
    np.testing.assert_allclose(y, x + oracle.gemv(oracle.expert_slice(down, 1), u), rtol=1e-14)


def test_decoder_layer_zero_weights_identity():
    model = dict(name="tiny", layers=1, hidden=128, qkv=192, q_dim=128, o_in=128, ffn=256)
    w = synth.layer_weights(1, model, 0)
    for name in ("o", "down"):
        w[name]["scales"][:] = 0
        w[name]["biases"][:] = 0
    x = synth.activations(1, "x", 128, np.float32).astype(np.float64)
    assert np.array_equal(oracle.decoder_layer(w, x, 128), x)


def _rowconst(N, K, b):
    """N x K 4-bit matrix with scale 0 and bias b[n] in every group: W.v = b_n sum(v)."""
    b = np.broadcast_to(np.asarray(b, np.float64), (N,))
    return {"N": N, "K": K, "bits": 4, "fmt": synth.AFFINE, "group": 64,
            "q": synth.words(synth.stream(0, "rowconst", N, K), (N, K * 4 // 32)),
            "scales": np.zeros((N, K // 64), np.float16),
            "biases": np.repeat(b[:, None], K // 64, axis=1).astype(np.float16), "lut": None}


def _two_level_x(H, lo, hi):
    return np.where(np.arange(H) < H // 2, lo, hi).astype(np.float64)


def test_decoder_layer_hand_case():
    """The whole layer against the hand derivation in the golden file: a wrong
    q-slice, the FFN reading x instead of h, swapped norm weights or a dropped
    residual each move the answer."""
    c = GOLDEN["decoder_layer"]
    H, QD, F = c["hidden"], c["q_dim"], c["ffn"]
    b_qkv = np.concatenate([np.full(QD, c["b_q"]), np.full(c["qkv_rows"] - QD, c["b_kv"])])
    w = {"qkv": _rowconst(c["qkv_rows"], H, b_qkv), "o": _rowconst(H, QD, c["b_o"]),
         "gate": _rowconst(F, H, c["b_gate"]), "up": _rowconst(F, H, c["b_up"]),
         "down": _rowconst(H, F, c["b_down"]),
         "g_attn": np.full(H, c["g_attn"], np.float16), "g_ffn": np.full(H, c["g_ffn"], np.float16)}
    x = _two_level_x(H, 1.0, 7.0)
    h = _two_level_x(H, 1.8, 7.8)
    S = 614.4 / np.sqrt(32.04)
    expect = h + (S / 64) / (1 + np.exp(-S / 64)) * S / 128
    np.testing.assert_allclose(oracle.decoder_layer(w, x, QD, c["eps"]), expect, rtol=1e-13)


def test_rmsnorm_gemv_closed_form():
    """W . rmsnorm(x; g) + r with rows of constant weight: b_n * sum(g x) / rms(x) + r_n."""
    H, N = 128, 5
    b = np.array([1, -2, 3, 0.5, 0.25]) / 64
    W = _rowconst(N, H, b)
    x = _two_level_x(H, 1.0, 7.0)  # rms 5
    g = np.full(H, 2.0, np.float16)
    r = np.arange(N, dtype=np.float64)
    y = oracle.rmsnorm_gemv(W, x, g, 0.0, r)
    np.testing.assert_allclose(y, b * (2 * 64 * 8 / 5) + r, rtol=1e-14)
    # scale invariance of the norm: 10 x gives the same output
    np.testing.assert_allclose(oracle.rmsnorm_gemv(W, 10 * x, g, 0.0, r), y, rtol=1e-14)


def test_rmsnorm_swiglu_closed_form():
    """gate rows 1/64 and up rows 1/128 of constant weight after the norm:
    u = silu(S/64) * S/128 with S = sum(g x) / rms(x) = 102.4."""
    H, F = 64, 3
    x = _two_level_x(H, 1.0, 7.0)
    g = np.full(H, 2.0, np.float16)
    u = oracle.rmsnorm_swiglu(_rowconst(F, H, 1 / 64), _rowconst(F, H, 1 / 128), x, g, 0.0)
    np.testing.assert_allclose(u, np.full(F, 0.8 * 1.6 / (1 + np.exp(-1.6))), rtol=1e-14)


def test_logits_topk_closed_form():
    """Rows of constant weight b_n: z_n = b_n * sum(g x) / rms(x), the same for
    x and 10 x; the top-k follows the order of b (ties by lower index)."""
    H = 64
    b = np.array([0.5, -1, 2, 2, 0.25, 1]) / 32
    W = _rowconst(len(b), H, b)
    x = _two_level_x(H, 1.0, 7.0)
    g = np.full(H, 0.5, np.float16)
    for scale in (1.0, 10.0):
        z, idx, vals = oracle.logits_topk(W, scale * x, 4, g, 0.0)
        np.testing.assert_allclose(z, b * (0.5 * 32 * 8 / 5), rtol=1e-14)
        assert list(idx) == [2, 3, 5, 0]


def test_moe_expert_rows_closed_form():
    """Expert e's rows are rows [e*N, (e+1)*N) of the stacked tensors: expert
    e's down weight is the constant (e+1)/64, gate/up constants give one known
    u; the routed expert's number shows in the output."""
    E, F, H = 5, 64, 64
    gate = _rowconst(E * F, H, 1 / 64)
    up = _rowconst(E * F, H, 1 / 128)
    down = _rowconst(E * H, F, np.repeat((np.arange(E) + 1) / 64, H))
    for W in (gate, up, down):
        W["E"] = E
    x = _two_level_x(H, 1.0, 7.0)
    a = x.sum() / 64  # gate_j (no norm: x' = x), 4.0
    c = x.sum() / 128  # up_j, 2.0
    u = a / (1 + np.exp(-a)) * c
    for e in range(E):
        lg = np.full(E, -1.0)
        lg[e] = 3.0
        y, ids, w = oracle.moe_layer(gate, up, down, None, lg, 1, x, None)
        assert list(ids) == [e] and w[0] == 1.0
        np.testing.assert_allclose(y, x + (e + 1) / 64 * F * u, rtol=1e-14)


def test_expert_bytes_match_page():
    """The page's per-expert size pins 4-bit codes + fp16 scale + fp16 bias per 64."""
    c = GOLDEN["expert_bytes"]
    H, F = c["hidden"], c["ffn"]
    mats = [synth.qmat(0, "e", F, H), synth.qmat(0, "e", F, H), synth.qmat(0, "e", H, F)]
    nbytes = sum(m["q"].nbytes + m["scales"].nbytes + m["biases"].nbytes for m in mats)
    assert nbytes == c["bytes"]
    assert nbytes / 2 ** 20 == c["mib"]


# ---------------------------------------------------------------------------
# sampling after top-k: the counter-based generator and the draw

# Outputs 0..3 of SplitMix64 started from state 0 (the reference
# implementation accompanying Steele, Lea and Flood, OOPSLA 2014; the first
# two are also java.util.SplittableRandom(0).nextLong() = -2152535657050944081
# and 7960286522194355700).
SPLITMIX64_STATE0 = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]


def test_splitmix64_published_outputs():
    assert [oracle.splitmix64(0, c) for c in range(4)] == SPLITMIX64_STATE0
    assert oracle.splitmix64(0, 0) - 2**64 == -2152535657050944081
    assert oracle.splitmix64(0, 1) == 7960286522194355700


def test_splitmix64_seed_is_a_state_offset():
    # starting from state s = 0 + j*gamma gives the generator's outputs from
    # position j on: the counter form is the sequential generator
    gamma = 0x9E3779B97F4A7C15
    for j in range(3):
        for c in range(3):
            assert oracle.splitmix64((j * gamma) % 2**64, c) == oracle.splitmix64(0, j + c)


def test_uniform_range_and_moments():
    n = 200000
    u = np.array([oracle.uniform(1234, c) for c in range(n)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 0.002
    for c in (0, 1, 77):
        assert oracle.uniform(99, c) == (oracle.splitmix64(99, c) >> 11) / 2.0**53


def test_sample_greedy_at_zero_temperature():
    idx = np.array([7, 3, 9], np.int32)
    for u in (0.0, 0.5, 0.999999):
        assert oracle.sample([2.0, 1.0, 0.5], idx, 0.0, 1.0, u) == 7


def test_sample_inverse_cdf_closed_forms():
    # two candidates with weights 1 and 1/3: probabilities 3/4 and 1/4
    v2, i2 = [0.0, -np.log(3.0)], np.array([11, 22], np.int32)
    assert oracle.sample(v2, i2, 1.0, 1.0, 0.0) == 11
    assert oracle.sample(v2, i2, 1.0, 1.0, 0.7499) == 11
    assert oracle.sample(v2, i2, 1.0, 1.0, 0.7501) == 22
    assert oracle.sample(v2, i2, 1.0, 1.0, 0.999) == 22
    # three candidates with weights 4:2:1: cumulative 4/7, 6/7, 1
    v3, i3 = np.log([4.0, 2.0, 1.0]), np.array([5, 6, 7], np.int32)
    assert oracle.sample(v3, i3, 1.0, 1.0, 0.5) == 5
    assert oracle.sample(v3, i3, 1.0, 1.0, 0.6) == 6
    assert oracle.sample(v3, i3, 1.0, 1.0, 0.85) == 6
    assert oracle.sample(v3, i3, 1.0, 1.0, 0.86) == 7


def test_sample_temperature_scales_the_logits():
    rng = np.random.default_rng(5)
    v = np.sort(rng.normal(size=8))[::-1]
    idx = np.arange(8, dtype=np.int32)
    for u in np.linspace(0.0, 0.99, 34):
        assert oracle.sample(2.0 * v, idx, 2.0, 1.0, u) == oracle.sample(v, idx, 1.0, 1.0, u)
        assert oracle.sample(v, idx, 0.5, 1.0, u) == oracle.sample(2.0 * v, idx, 1.0, 1.0, u)
    # a very low temperature is greedy
    assert oracle.sample(v, idx, 1e-3, 1.0, 0.999) == 0


def test_sample_top_p_prefix():
    v3, i3 = np.log([4.0, 2.0, 1.0]), np.array([5, 6, 7], np.int32)
    for u in (0.0, 0.5, 0.99):  # 4/7 >= 0.5: only the first candidate is kept
        assert oracle.sample(v3, i3, 1.0, 0.5, u) == 5
    # top_p 0.8 keeps the first two (6/7 >= 0.8 > 4/7), renormalized 2/3, 1/3
    assert oracle.sample(v3, i3, 1.0, 0.8, 0.66) == 5
    assert oracle.sample(v3, i3, 1.0, 0.8, 0.67) == 6
    assert oracle.sample(v3, i3, 1.0, 0.8, 0.99) == 6


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_sample_frequencies_match_softmax(top_p):
    rng = np.random.default_rng(11)
    v = np.sort(rng.normal(scale=0.8, size=5))[::-1]
    idx = np.arange(5, dtype=np.int32)
    T = 0.7
    p = scipy.special.softmax(v / T)
    keep = int(np.searchsorted(np.cumsum(p), top_p * (1 - 1e-12)) + 1)
    q = np.zeros(5)
    q[:keep] = p[:keep] / p[:keep].sum()
    n = 40000
    counts = np.bincount([oracle.sample(v, idx, T, top_p, oracle.uniform(2024, c)) for c in range(n)],
                         minlength=5)
    sigma = np.sqrt(n * q * (1 - q)) + 1e-9
    assert np.all(np.abs(counts - n * q) < 5 * sigma + 1), (counts, n * q)


def test_sample_rejects_bad_arguments():
    v, i = [1.0, 0.0], np.array([0, 1], np.int32)
    for T, tp, u in ((-1.0, 1.0, 0.5), (1.0, 0.0, 0.5), (1.0, 1.5, 0.5), (1.0, 1.0, 1.0),
                     (1.0, 1.0, -0.1), (float("nan"), 1.0, 0.5)):
        with pytest.raises(Exception):
            oracle.sample(v, i, T, tp, u)


# ---------------------------------------------------------------------------
# decode attention over a [Hkv][T_max][d] fp16 cache

def _cache(rng, Hkv, T_max, d):
    return (rng.normal(size=(Hkv, T_max, d)).astype(np.float16),
            rng.normal(size=(Hkv, T_max, d)).astype(np.float16))


def test_attention_one_position_is_v():
    rng = np.random.default_rng(1)
    Kc, Vc = _cache(rng, 2, 5, 16)
    q = rng.normal(size=(4, 16))
    out = oracle.attention(q, Kc, Vc, 1, 0.25)
    for h in range(4):
        assert np.array_equal(out[h], Vc[h // 2, 0].astype(np.float64))


def test_attention_equal_keys_average_v():
    rng = np.random.default_rng(2)
    Kc, Vc = _cache(rng, 1, 9, 8)
    Kc[:] = Kc[:, :1]  # every position has the same key
    q = rng.normal(size=(3, 8))
    out = oracle.attention(q, Kc, Vc, 7, 0.3)
    ref = Vc[0, :7].astype(np.float64).mean(axis=0)
    assert np.allclose(out, ref[None, :], rtol=0, atol=1e-12)


@pytest.mark.parametrize("H,Hkv,d,n", [(4, 4, 16, 13), (8, 2, 32, 50), (6, 1, 8, 3)])
def test_attention_matches_library_softmax(H, Hkv, d, n):
    rng = np.random.default_rng(H * 100 + n)
    Kc, Vc = _cache(rng, Hkv, n + 5, d)
    q = rng.normal(size=(H, d))
    scale = 1 / np.sqrt(d)
    out = oracle.attention(q, Kc, Vc, n, scale)
    G = H // Hkv
    for h in range(H):
        Kg = Kc[h // G, :n].astype(np.float64)
        Vg = Vc[h // G, :n].astype(np.float64)
        p = scipy.special.softmax(scale * (Kg @ q[h]))
        assert np.allclose(out[h], p @ Vg, rtol=1e-12, atol=1e-12)


def test_attention_gqa_groups_are_independent_caches():
    rng = np.random.default_rng(4)
    Kc, Vc = _cache(rng, 2, 20, 16)
    q = rng.normal(size=(8, 16))
    both = oracle.attention(q, Kc, Vc, 17, 0.2)
    for g in range(2):
        one = oracle.attention(q[4 * g:4 * g + 4], Kc[g:g + 1], Vc[g:g + 1], 17, 0.2)
        assert np.array_equal(both[4 * g:4 * g + 4], one)


def test_attention_scale_and_one_hot():
    rng = np.random.default_rng(5)
    Kc, Vc = _cache(rng, 1, 12, 16)
    q = rng.normal(size=(2, 16))
    assert np.allclose(oracle.attention(q, Kc, Vc, 12, 0.5), oracle.attention(q * 0.5, Kc, Vc, 12, 1.0),
                       rtol=1e-12, atol=1e-12)
    # a query far along one key picks that position's value
    q1 = 200.0 * Kc[0, 7:8].astype(np.float64)
    Kn = Kc.copy()
    Kn[0] /= np.linalg.norm(Kn[0].astype(np.float64), axis=1, keepdims=True).astype(np.float16)
    q1 = 200.0 * Kn[0, 7:8].astype(np.float64)
    out = oracle.attention(q1, Kn, Vc, 12, 1.0)
    assert np.allclose(out[0], Vc[0, 7].astype(np.float64), atol=1e-3)


def test_attention_rejects_bad_shapes():
    rng = np.random.default_rng(6)
    Kc, Vc = _cache(rng, 2, 4, 8)
    with pytest.raises(Exception):
        oracle.attention(rng.normal(size=(3, 8)), Kc, Vc, 2, 1.0)  # H not a multiple of Hkv
    with pytest.raises(Exception):
        oracle.attention(rng.normal(size=(4, 8)), Kc, Vc, 5, 1.0)  # n > T_max
