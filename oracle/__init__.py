"""CPU oracle for the quantized decode matrix-vector product and its fusions.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the GPU library and the GPU library never imports it.

The arithmetic lives in ``qg_oracle.c`` (plain scalar C, double precision).
This module loads it with ctypes and composes the whole decode steps from its
primitives in the pages' order:

* decoder layer: qkv = Wqkv . rmsnorm(x; g_attn); the attention output is read
  as the first q_dim entries of qkv (attention itself is outside the path);
  h = x + Wo . a; u = swiglu(rmsnorm(h; g_ffn)); x' = h + Wdown . u.
  ("Booster la vitesse d'inference sur Apple Silicon", section 1: rmsnorm
  fused into the QKV matvec, residual + norm, gate.up SwiGLU.)
* MoE expert layer: route the top-k of the router logits, softmax over the
  chosen ones, run each chosen expert's SwiGLU FFN on rmsnorm(x) and combine
  with the routing weights, add the always-on shared expert with weight 1
  and the residual. (GeekNews item on the 397B MoE engine: "Architecture du
  modele", "Deferred GPU Expert Compute".)
* decode attention: one query per head against a [Hkv][T][d] fp16 KV cache,
  softmax over the positions, GQA head grouping ("Booster la vitesse
  d'inference sur Apple Silicon", section 2 "KV cache").
* logits head: z = Wlm . rmsnorm(x; g_final), then the top-k of z, and
  optionally one token drawn from the top-k (temperature, top-p, a uniform
  number from the counter-based SplitMix64 generator).

Parity status of each function: see the ``PINS`` table at the bottom.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qg_oracle.c")
# QG_ORACLE_LIB lets the mutation tests load a deliberately broken build.
_LIB_PATH = os.environ.get("QG_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

AFFINE = 0
LUT = 1
DENSE = 2


def build(force: bool = True) -> str:
    """Compile qg_oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                        "-Wall", "-Wextra", "-fPIC", "-shared", "-o", tmp, _SRC,
                        "-lm", "-lpthread"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _QMat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("lut", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int), ("group", ctypes.c_int),
                ("bits", ctypes.c_int), ("fmt", ctypes.c_int)]


_lib = None
_lock = threading.Lock()


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            L = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            L.og_half_to_double.argtypes = [ctypes.c_uint16]
            L.og_half_to_double.restype = ctypes.c_double
            L.og_unpack.argtypes = [ctypes.POINTER(_QMat), P]
            L.og_dequant.argtypes = [ctypes.POINTER(_QMat), P]
            L.og_gemv.argtypes = [ctypes.POINTER(_QMat), I, P, P, P, I]
            L.og_rmsnorm.argtypes = [P, I, P, ctypes.c_double, P]
            L.og_silu.argtypes = [ctypes.c_double]
            L.og_silu.restype = ctypes.c_double
            L.og_swiglu.argtypes = [ctypes.POINTER(_QMat), ctypes.POINTER(_QMat), I, P, P, I]
            L.og_topk.argtypes = [P, I, I, P, P]
            L.og_route.argtypes = [P, I, I, P, P]
            D = ctypes.c_double
            U64 = ctypes.c_uint64
            L.og_sample.argtypes = [P, P, I, D, D, D, P]
            L.og_attention.argtypes = [P, P, P, I, I, I, I, I, D, P]
            L.og_splitmix64.argtypes = [U64, U64]
            L.og_splitmix64.restype = U64
            L.og_uniform.argtypes = [U64, U64]
            L.og_uniform.restype = D
            for f in ("og_unpack", "og_dequant", "og_gemv", "og_rmsnorm", "og_swiglu",
                      "og_topk", "og_route", "og_sample", "og_attention"):
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Mat:
    """Keeps the contiguous arrays alive while C holds pointers into them."""

    def __init__(self, W: dict):
        self.q = _c(W["q"], np.uint32)
        self.s = _c(W.get("scales"), np.float16)
        self.b = _c(W.get("biases"), np.float16)
        self.l = _c(W.get("lut"), np.float16)
        self.N, self.K = int(W["N"]), int(W["K"])
        self.st = _QMat(_ptr(self.q), _ptr(self.s), _ptr(self.b), _ptr(self.l),
                        self.N, self.K, int(W.get("group", 64)), int(W["bits"]),
                        int(W["fmt"]))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


# ---------------------------------------------------------------------------
# primitives

def half_to_double(bits: int) -> float:
    return lib().og_half_to_double(int(bits) & 0xFFFF)


def unpack(W: dict) -> np.ndarray:
    m = _Mat(W)
    out = np.empty((m.N, m.K), np.uint8)
    _check(lib().og_unpack(ctypes.byref(m.st), out.ctypes.data), "unpack")
    return out


def dequant(W: dict) -> np.ndarray:
    m = _Mat(W)
    out = np.empty((m.N, m.K), np.float64)
    _check(lib().og_dequant(ctypes.byref(m.st), out.ctypes.data), "dequant")
    return out


def gemv(W: dict, x, residual=None, nthreads: int = 1) -> np.ndarray:
    """y[m] = residual[m] + W x[m]; x is [K] or [M][K]; returns float64."""
    m = _Mat(W)
    x = np.asarray(x)
    one = x.ndim == 1
    X = _c(np.atleast_2d(x), np.float64)
    M = X.shape[0]
    if X.shape[1] != m.K:
        raise ValueError("x length != K")
    R = None if residual is None else _c(np.atleast_2d(residual), np.float64)
    y = np.empty((M, m.N), np.float64)
    _check(lib().og_gemv(ctypes.byref(m.st), M, X.ctypes.data, _ptr(R), y.ctypes.data,
                         int(nthreads)), "gemv")
    return y[0] if one else y


def rmsnorm(x, g, eps: float = 1e-5) -> np.ndarray:
    X = _c(x, np.float64)
    G = _c(g, np.float16)
    out = np.empty_like(X)
    _check(lib().og_rmsnorm(X.ctypes.data, X.size, G.ctypes.data, float(eps),
                            out.ctypes.data), "rmsnorm")
    return out


def silu(z: float) -> float:
    return lib().og_silu(float(z))


def swiglu(Wg: dict, Wu: dict, x, nthreads: int = 1) -> np.ndarray:
    mg, mu = _Mat(Wg), _Mat(Wu)
    x = np.asarray(x)
    one = x.ndim == 1
    X = _c(np.atleast_2d(x), np.float64)
    M = X.shape[0]
    u = np.empty((M, mg.N), np.float64)
    _check(lib().og_swiglu(ctypes.byref(mg.st), ctypes.byref(mu.st), M, X.ctypes.data,
                           u.ctypes.data, int(nthreads)), "swiglu")
    return u[0] if one else u


def topk(z, k: int):
    """(idx int32[k], vals float64[k]): larger first, ties by lower index."""
    Z = _c(z, np.float64)
    idx = np.empty(k, np.int32)
    vals = np.empty(k, np.float64)
    _check(lib().og_topk(Z.ctypes.data, Z.size, int(k), idx.ctypes.data, vals.ctypes.data),
           "topk")
    return idx, vals


def route(logits, k: int):
    """(ids int32[k], weights float64[k]) of the top-k experts."""
    Lg = _c(logits, np.float64)
    ids = np.empty(k, np.int32)
    w = np.empty(k, np.float64)
    _check(lib().og_route(Lg.ctypes.data, Lg.size, int(k), ids.ctypes.data, w.ctypes.data),
           "route")
    return ids, w


def sample(vals, idx, temperature: float, top_p: float, u: float) -> int:
    """One token from a top-k list (vals larger first) for the uniform draw u."""
    V = _c(vals, np.float64)
    Ix = _c(idx, np.int32)
    tok = np.empty(1, np.int32)
    _check(lib().og_sample(V.ctypes.data, Ix.ctypes.data, V.size, float(temperature),
                           float(top_p), float(u), tok.ctypes.data), "sample")
    return int(tok[0])


def attention(q, k_cache, v_cache, n: int, scale: float):
    """out[H][d] of one decode step: q [H][d] (float64), caches [Hkv][T_max][d]
    fp16, attending positions 0..n-1."""
    Q = _c(q, np.float64)
    Kc = np.ascontiguousarray(k_cache, np.float16)
    Vc = np.ascontiguousarray(v_cache, np.float16)
    H, d = Q.shape
    Hkv, T_max, d2 = Kc.shape
    assert d2 == d and Vc.shape == Kc.shape
    out = np.empty((H, d), np.float64)
    _check(lib().og_attention(Q.ctypes.data, Kc.ctypes.data, Vc.ctypes.data, H, Hkv, d, T_max,
                              int(n), float(scale), out.ctypes.data), "attention")
    return out


def splitmix64(seed: int, counter: int) -> int:
    """Output number `counter` of the SplitMix64 generator started at `seed`."""
    return int(lib().og_splitmix64(seed & (2**64 - 1), counter & (2**64 - 1)))


def uniform(seed: int, counter: int) -> float:
    """The draw in [0, 1) for (seed, counter): top 53 bits of splitmix64."""
    return float(lib().og_uniform(seed & (2**64 - 1), counter & (2**64 - 1)))


# ---------------------------------------------------------------------------
# composed steps

def rmsnorm_gemv(W: dict, x, g, eps: float = 1e-5, residual=None, nthreads: int = 1):
    """W . rmsnorm(x; g) (+ residual), per activation vector."""
    x = np.asarray(x, np.float64)
    X = np.atleast_2d(x)
    Xn = np.stack([rmsnorm(row, g, eps) for row in X])
    y = gemv(W, Xn, residual, nthreads)
    return y[0] if x.ndim == 1 else y


def rmsnorm_swiglu(Wg: dict, Wu: dict, x, g=None, eps: float = 1e-5, nthreads: int = 1):
    x = np.asarray(x, np.float64)
    X = np.atleast_2d(x)
    Xn = X if g is None else np.stack([rmsnorm(row, g, eps) for row in X])
    u = swiglu(Wg, Wu, Xn, nthreads)
    return u[0] if x.ndim == 1 else u


def decoder_layer(w: dict, x, q_dim: int, eps: float = 1e-5, nthreads: int = 1):
    """One decode layer with the attention output stood in by the q-slice."""
    x = np.asarray(x, np.float64)
    qkv = rmsnorm_gemv(w["qkv"], x, w["g_attn"], eps, None, nthreads)
    a = qkv[:q_dim]
    h = gemv(w["o"], a, x, nthreads)
    u = rmsnorm_swiglu(w["gate"], w["up"], h, w["g_ffn"], eps, nthreads)
    return gemv(w["down"], u, h, nthreads)


def expert_slice(W_all: dict, e: int) -> dict:
    """Expert e of a stacked [E*N][...] quantized tensor."""
    N = W_all["N"] // W_all["E"]
    out = dict(W_all)
    out["N"] = N
    for key in ("q", "scales", "biases", "lut"):
        if W_all.get(key) is not None:
            out[key] = W_all[key][e * N:(e + 1) * N]
    return out


def moe_layer(gate_all: dict, up_all: dict, down_all: dict, shared: tuple, logits, top_k: int,
              x, g=None, eps: float = 1e-5, nthreads: int = 1):
    """y = x + sum_{e in top_k} w_e D_e swiglu_e(x') + D_sh swiglu_sh(x'),
    x' = rmsnorm(x; g) (or x when g is None). Returns (y, ids, weights)."""
    x = np.asarray(x, np.float64)
    xn = x if g is None else rmsnorm(x, g, eps)
    ids, wts = route(logits, top_k)
    y = x.copy()
    for e, we in zip(ids, wts):
        u = swiglu(expert_slice(gate_all, e), expert_slice(up_all, e), xn, nthreads)
        y = y + we * gemv(expert_slice(down_all, e), u, None, nthreads)
    if shared is not None:
        u = swiglu(shared[0], shared[1], xn, nthreads)
        y = y + gemv(shared[2], u, None, nthreads)
    return y, ids, wts


def logits_topk(W: dict, x, k: int, g=None, eps: float = 1e-5, nthreads: int = 1):
    """(z, idx, vals): z = W . rmsnorm(x; g) and its top-k."""
    x = np.asarray(x, np.float64)
    xn = x if g is None else rmsnorm(x, g, eps)
    z = gemv(W, xn, None, nthreads)
    idx, vals = topk(z, k)
    return z, idx, vals


# What pins each function to something other than itself (tests/test_oracle.py).
PINS = {
    "half_to_double": "all 65536 fp16 patterns against numpy's fp16 conversion",
    "unpack": "hand words 0x76543210 / 0xFEDCBA98 / 0xE4E4E4E4 / 0x03020100 / 0xFFC08001; "
              "independent packer round trip (2-, 4- and 8-bit)",
    "dequant": "matrices built from chosen codes, scales and biases; one-hot, 16^j and 256^j "
               "probes; dense fp16 fields against numpy's fp16 reading of the row bytes",
    "gemv": "hand-computed tiny cases (2-, 4-, 8-bit and dense); all-ones closed form; numpy "
            "matmul of the dense weights",
    "rmsnorm": "constant-vector closed form; hand case [3,4]; unit mean square for eps=0",
    "silu": "z * scipy.special.expit(z)",
    "swiglu": "one-hot and zero-weight closed forms; composition of pinned gemv and silu",
    "topk": "numpy lexsort brute force with forced ties, signed zeros and NaN",
    "route": "equal logits give 1/k each; scipy.special.softmax over the chosen logits",
    "moe_layer": "zero experts give y = x; single-expert closed form; K-concatenation identity",
    "decoder_layer": "composition of pinned primitives; zero weights give identity",
    "logits_topk": "composition of pinned gemv, rmsnorm and topk",
    "splitmix64": "published first output for state 0 (0xE220A8397B1DCDAF); Python big-int "
                  "arithmetic of the published mixing steps over random seeds",
    "uniform": "range [0, 1); mean and variance of 200000 draws; top-53-bit mapping",
    "attention": "one position gives V exactly; equal keys give the mean of V; scipy softmax "
                 "times V brute force; GQA head mapping against per-group calls; scale "
                 "invariance",
    "sample": "greedy at temperature 0; two- and three-candidate closed forms of the inverse "
              "CDF at chosen u; temperature scaling invariance; top-p prefix cut; empirical "
              "frequencies of 40000 counter draws against softmax probabilities",
}
