"""Python binding of libqgemv.so, the gfx950 quantized decode matvec library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/qgemv.h. PyTorch provides device
memory and the current stream. The functions carry the C names:

  qgemv, qgemv_rmsnorm, qswiglu, qmoe_experts, qmoe_experts_batch, qlogits_topk, qlogits_sample,
  qg_sample_topk,
  qattn_decode,
  qg_workspace_bytes, qg_workspace_init, qg_status_str, qg_tune

Import fails loudly when the library has not been built; there is no CPU
fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

# status codes and enums (include/qgemv.h)
QG_OK, QG_EINVAL, QG_EUNSUPPORTED, QG_EWORKSPACE, QG_ELAUNCH, QG_EDEVICE = 0, -1, -2, -3, -4, -5
QG_AFFINE, QG_LUT, QG_DENSE = 0, 1, 2
QG_F16, QG_F32 = 0, 1
QG_OP_GEMV, QG_OP_GEMV_RMSNORM, QG_OP_SWIGLU, QG_OP_MOE, QG_OP_LOGITS_TOPK, QG_OP_ATTN = 0, 1, 2, 3, 4, 5
QG_MAX_TOPK = 1024

EXPORTED = ("qg_status_str", "qg_workspace_bytes", "qg_workspace_init", "qg_tune", "qgemv",
            "qgemv_rmsnorm", "qswiglu", "qmoe_experts", "qmoe_experts_batch", "qlogits_topk",
            "qlogits_topk_noalloc", "qg_logits_topk_launches", "qlogits_sample",
            "qg_sample_topk", "qattn_decode", "qg_probe_read",
            "qg_probe_copy", "qg_probe_phases")


class QgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {qg_status_str(status)} ({status})")


class qg_qmat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("lut", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        Q = ctypes.POINTER(qg_qmat)
        L.qg_status_str.argtypes = [I]
        L.qg_status_str.restype = ctypes.c_char_p
        L.qg_workspace_bytes.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(S)]
        L.qg_workspace_init.argtypes = [P, S, P]
        L.qg_tune.argtypes = [I, I]
        L.qgemv.argtypes = [Q, I, I, I, I, I, I, P, I, P, P, P, S, P]
        L.qgemv_rmsnorm.argtypes = [Q, I, I, I, I, I, I, P, I, P, F, P, P, P, S, P]
        L.qswiglu.argtypes = [Q, Q, I, I, I, I, I, I, P, I, P, F, P, P, S, P]
        L.qmoe_experts.argtypes = [Q, Q, Q, I, I, I, I, I, I, Q, P, I, P, F, P, P, P, P, P, S, P]
        L.qmoe_experts_batch.argtypes = [Q, Q, Q, I, I, I, I, I, I, I, Q, P, I, P, F, P, P, P, P, P,
                                         S, P]
        L.qlogits_topk.argtypes = [Q, I, I, I, I, I, P, I, P, F, P, I, P, P, P, S, P]
        L.qlogits_topk_noalloc.argtypes = [Q, I, I, I, I, I, P, I, P, F, P, I, P, P, P]
        L.qg_logits_topk_launches.argtypes = [Q, I, I, I, I, I, I, ctypes.POINTER(I)]
        U64 = ctypes.c_uint64
        L.qlogits_sample.argtypes = [Q, I, I, I, I, I, P, I, P, F, P, I, P, P, F, F, U64, P, P,
                                     P, S, P]
        L.qg_sample_topk.argtypes = [P, P, I, F, F, U64, P, P, P]
        L.qattn_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, P, S, P]
        L.qg_probe_read.argtypes = [P, S, P, I, I, P]
        L.qg_probe_copy.argtypes = [P, P, S, I, P]
        L.qg_probe_phases.argtypes = [P, S, P, I, I, P, P, P, I, I, P]
        for name in EXPORTED:
            if name != "qg_status_str":
                getattr(L, name).restype = I
        _lib = L
    return _lib


def qg_status_str(status: int) -> str:
    return lib().qg_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != QG_OK:
        raise QgError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, n: int, name: str, dtypes=None):
    """A tensor handed to the library by pointer must be contiguous, of one of
    `dtypes` (torch dtypes) when given, and hold at least n elements: the
    C-ABI cannot see its size, so an undersized buffer is refused here."""
    if t is None:
        return
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements, needs at least {n}")


def _f32():
    import torch
    return (torch.float32,)


def _f16():
    """fp16 data, as float16 or as its raw 16-bit patterns"""
    import torch
    return (torch.float16, torch.int16)


def _i32():
    import torch
    return (torch.int32,)


def _x_for(x, W_K: int, name: str = "x"):
    """M of an activation tensor [K] or [M, K] whose row length is W_K."""
    import torch
    M = 1 if x.dim() == 1 else x.shape[0]
    _need(x, M * W_K, name, (torch.float16, torch.float32))
    if x.shape[-1] != W_K or x.dim() > 2:
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected [{W_K}] or [M, {W_K}]")
    return M


def _xdtype(x):
    import torch
    if x.dtype == torch.float16:
        return QG_F16
    if x.dtype == torch.float32:
        return QG_F32
    raise TypeError("activations must be float16 or float32")


class QMat:
    """A planar quantized N x K matrix on the device (see include/qgemv.h).

    q: int32 tensor [N, K*bits/32] holding the uint32 code words (dense
    format: the fp16 matrix [N, K] read as words);
    scales, biases: float16 [N, K/64] (affine) or None;
    lut: float16 [N, 16] (LUT format) or None."""

    def __init__(self, q, scales=None, biases=None, lut=None, *, N: int, K: int, bits: int = 4,
                 fmt: int = QG_AFFINE, group: int = 64):
        self.q, self.scales, self.biases, self.lut = q, scales, biases, lut
        self.N, self.K, self.bits, self.fmt, self.group = N, K, bits, fmt, group
        words = N * (K * (16 if fmt == QG_DENSE else bits) // 32)
        _need(q, words, "q")
        if fmt == QG_AFFINE:
            _need(scales, N * (K // max(group, 1)), "scales", _f16())
            _need(biases, N * (K // max(group, 1)), "biases", _f16())
        if fmt == QG_LUT:
            _need(lut, N * 16, "lut", _f16())
        self.c = qg_qmat(q.data_ptr() if q is not None else None,
                         scales.data_ptr() if scales is not None else None,
                         biases.data_ptr() if biases is not None else None,
                         lut.data_ptr() if lut is not None else None)

    @classmethod
    def from_host(cls, W: dict, device="cuda"):
        """Uploads a host matrix given as a dict of numpy arrays (q uint32,
        scales/biases/lut float16) with N, K, bits, fmt, group."""
        import torch

        def up(a, dt):
            if a is None:
                return None
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        return cls(up(W["q"], np.int32), up(W.get("scales"), np.float16),
                   up(W.get("biases"), np.float16), up(W.get("lut"), np.float16),
                   N=int(W["N"]), K=int(W["K"]), bits=int(W["bits"]), fmt=int(W["fmt"]),
                   group=int(W.get("group", 64)))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.q, self.scales, self.biases,
                                                           self.lut) if t is not None)


def qg_workspace_bytes(op: int, N: int, K: int, M: int = 1, bits: int = 4, fmt: int = QG_AFFINE,
                       k: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().qg_workspace_bytes(op, N, K, M, bits, fmt, k, ctypes.byref(out)),
           "qg_workspace_bytes")
    return out.value


def qg_workspace_init(ws, stream=None):
    _check(lib().qg_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qg_workspace_init")


def workspace(op: int, N: int, K: int, M: int = 1, bits: int = 4, fmt: int = QG_AFFINE, k: int = 1,
              device="cuda", stream=None):
    """Allocates (through torch) and clears a workspace for `op`."""
    import torch
    n = max(qg_workspace_bytes(op, N, K, M, bits, fmt, k), 256)
    ws = torch.empty((n + 3) // 4, dtype=torch.int32, device=device)
    qg_workspace_init(ws, stream)
    return ws


def qg_tune(knob: int, value: int):
    _check(lib().qg_tune(knob, value), "qg_tune")


def qg_logits_topk_launches(V: int, K: int, k: int, bits: int = 4, fmt: int = QG_AFFINE,
                            group: int = 64, W=None) -> int:
    """Kernels (1 or 2) that qlogits_topk enqueues for this head (W: its QMat,
    or None) on the current device."""
    out = ctypes.c_int(0)
    _check(lib().qg_logits_topk_launches(None if W is None else ctypes.byref(W.c), V, K, group,
                                         bits, fmt, k, ctypes.byref(out)),
           "qg_logits_topk_launches")
    return out.value


def qg_probe_read(src, out, blocks: int, cached: bool = False, stream=None):
    """Streams src once (read-only bandwidth probe); out: int32 [blocks*256]."""
    _check(lib().qg_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(out), blocks,
                               1 if cached else 0, _stream(stream)), "qg_probe_read")


def qg_probe_copy(dst, src, blocks: int, stream=None):
    """Copies src to dst (copy bandwidth probe)."""
    _check(lib().qg_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(), blocks,
                               _stream(stream)), "qg_probe_copy")


def qg_probe_phases(src, ranges, nphases: int, barrier, out, blocks: int, flags=None,
                    err=None, spin_limit: int = 1 << 20, stream=None):
    """Streams nphases byte ranges of src (ranges: int64 [2*nphases] device
    tensor of offset, count) in one launch, with or without a grid barrier
    between them (phase probe). barrier: False / True (= 1), or 2 for the
    barrier with the next range's first loads issued before the wait."""
    mode = int(barrier)
    _check(lib().qg_probe_phases(_ptr(src), src.numel() * src.element_size(), _ptr(ranges),
                                 nphases, mode, _ptr(flags), _ptr(out), _ptr(err),
                                 blocks, spin_limit, _stream(stream)), "qg_probe_phases")


def _ws_args(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def qgemv(W: QMat, x, residual=None, y=None, ws=None, stream=None):
    """y = residual + W x  (x: [K] or [M, K] fp16/fp32; y fp32)."""
    import torch
    M = _x_for(x, W.K)
    if y is None:
        y = torch.empty((W.N,) if x.dim() == 1 else (M, W.N), dtype=torch.float32, device=x.device)
    _need(y, M * W.N, "y", _f32())
    _need(residual, M * W.N, "residual", _f32())
    wp, wn = _ws_args(ws)
    _check(lib().qgemv(ctypes.byref(W.c), W.N, W.K, M, W.group, W.bits, W.fmt, _ptr(x),
                       _xdtype(x), _ptr(residual), _ptr(y), wp, wn, _stream(stream)), "qgemv")
    return y


def qgemv_rmsnorm(W: QMat, x, norm_w, eps: float = 1e-5, residual=None, y=None, ws=None,
                  stream=None):
    """y = residual + W rmsnorm(x; norm_w, eps)."""
    import torch
    M = _x_for(x, W.K)
    if y is None:
        y = torch.empty((W.N,) if x.dim() == 1 else (M, W.N), dtype=torch.float32, device=x.device)
    _need(y, M * W.N, "y", _f32())
    _need(residual, M * W.N, "residual", _f32())
    _need(norm_w, W.K, "norm_w", _f16())
    wp, wn = _ws_args(ws)
    _check(lib().qgemv_rmsnorm(ctypes.byref(W.c), W.N, W.K, M, W.group, W.bits, W.fmt, _ptr(x),
                               _xdtype(x), _ptr(norm_w), float(eps), _ptr(residual), _ptr(y), wp,
                               wn, _stream(stream)), "qgemv_rmsnorm")
    return y


def qswiglu(Wgate: QMat, Wup: QMat, x, norm_w=None, eps: float = 1e-5, u=None, ws=None,
            stream=None):
    """u = silu(Wgate x') * (Wup x'), x' = rmsnorm(x) when norm_w is given."""
    import torch
    M = _x_for(x, Wgate.K)
    if u is None:
        u = torch.empty((Wgate.N,) if x.dim() == 1 else (M, Wgate.N), dtype=torch.float32,
                        device=x.device)
    _need(u, M * Wgate.N, "u", _f32())
    _need(norm_w, Wgate.K, "norm_w", _f16())
    wp, wn = _ws_args(ws)
    _check(lib().qswiglu(ctypes.byref(Wgate.c), ctypes.byref(Wup.c), Wgate.N, Wgate.K, M,
                         Wgate.group, Wgate.bits, Wgate.fmt, _ptr(x), _xdtype(x), _ptr(norm_w),
                         float(eps), _ptr(u), wp, wn, _stream(stream)), "qswiglu")
    return u


def qmoe_experts(gate_all: QMat, up_all: QMat, down_all: QMat, n_experts: int, shared3,
                 router_logits, top_k: int, x, norm_w=None, eps: float = 1e-5, y=None,
                 sel_ids=None, sel_w=None, ws=None, stream=None):
    """One MoE expert layer (routing, SwiGLU experts, weighted combine, residual).
    gate_all/up_all are (n_experts*F) x H, down_all is (n_experts*H) x F;
    shared3 = (gate, up, down) QMats of the always-on expert, or None."""
    import torch
    F = gate_all.N // n_experts
    H = gate_all.K
    _need(x, H, "x", _f32())
    if y is None:
        y = torch.empty_like(x)
    _need(y, H, "y", _f32())
    _need(router_logits, n_experts, "router_logits", _f32())
    _need(norm_w, H, "norm_w", _f16())
    _need(sel_ids, top_k, "sel_ids", _i32())
    _need(sel_w, top_k, "sel_w", _f32())
    sh = None
    if shared3 is not None:
        arr = (qg_qmat * 3)(shared3[0].c, shared3[1].c, shared3[2].c)
        sh = ctypes.cast(arr, ctypes.POINTER(qg_qmat))
    wp, wn = _ws_args(ws)
    _check(lib().qmoe_experts(ctypes.byref(gate_all.c), ctypes.byref(up_all.c),
                              ctypes.byref(down_all.c), n_experts, F, H, gate_all.group,
                              gate_all.bits, gate_all.fmt, sh, _ptr(router_logits), top_k,
                              _ptr(norm_w), float(eps), _ptr(x), _ptr(y), _ptr(sel_ids),
                              _ptr(sel_w), wp, wn, _stream(stream)), "qmoe_experts")
    return y


def qmoe_experts_batch(gate_all: QMat, up_all: QMat, down_all: QMat, n_experts: int, shared3,
                       router_logits, top_k: int, x, norm_w=None, eps: float = 1e-5, y=None,
                       sel_ids=None, sel_w=None, ws=None, stream=None):
    """qmoe_experts for M tokens: x [M, H], router_logits [M, n_experts], y [M, H],
    sel_ids / sel_w [M, top_k] or None."""
    import torch
    F = gate_all.N // n_experts
    H = gate_all.K
    M = x.shape[0]
    _need(x, M * H, "x", _f32())
    if y is None:
        y = torch.empty_like(x)
    _need(y, M * H, "y", _f32())
    _need(router_logits, M * n_experts, "router_logits", _f32())
    _need(norm_w, H, "norm_w", _f16())
    _need(sel_ids, M * top_k, "sel_ids", _i32())
    _need(sel_w, M * top_k, "sel_w", _f32())
    sh = None
    if shared3 is not None:
        arr = (qg_qmat * 3)(shared3[0].c, shared3[1].c, shared3[2].c)
        sh = ctypes.cast(arr, ctypes.POINTER(qg_qmat))
    wp, wn = _ws_args(ws)
    _check(lib().qmoe_experts_batch(ctypes.byref(gate_all.c), ctypes.byref(up_all.c),
                                    ctypes.byref(down_all.c), n_experts, F, H, M, gate_all.group,
                                    gate_all.bits, gate_all.fmt, sh, _ptr(router_logits), top_k,
                                    _ptr(norm_w), float(eps), _ptr(x), _ptr(y), _ptr(sel_ids),
                                    _ptr(sel_w), wp, wn, _stream(stream)), "qmoe_experts_batch")
    return y


def qlogits_topk(W: QMat, x, k: int, norm_w=None, eps: float = 1e-5, logits=None, idx=None,
                 vals=None, ws=None, stream=None):
    """(logits, idx, vals): logits = W x' and its k largest entries."""
    import torch
    dev = x.device
    if logits is None:
        logits = torch.empty(W.N, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
    _need(x, W.K, "x", (torch.float16, torch.float32))
    _need(norm_w, W.K, "norm_w", _f16())
    _need(logits, W.N, "logits", _f32())
    _need(idx, k, "idx", _i32())
    _need(vals, k, "vals", _f32())
    wp, wn = _ws_args(ws)
    _check(lib().qlogits_topk(ctypes.byref(W.c), W.N, W.K, W.group, W.bits, W.fmt, _ptr(x),
                              _xdtype(x), _ptr(norm_w), float(eps), _ptr(logits), k, _ptr(idx),
                              _ptr(vals), wp, wn, _stream(stream)), "qlogits_topk")
    return logits, idx, vals


def qlogits_topk_noalloc(W: QMat, x, k: int, norm_w=None, eps: float = 1e-5, logits=None,
                         idx=None, vals=None, stream=None):
    """qlogits_topk on the library's own scratch memory (no workspace)."""
    import torch
    dev = x.device
    if logits is None:
        logits = torch.empty(W.N, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
    _need(x, W.K, "x", (torch.float16, torch.float32))
    _need(norm_w, W.K, "norm_w", _f16())
    _need(logits, W.N, "logits", _f32())
    _need(idx, k, "idx", _i32())
    _need(vals, k, "vals", _f32())
    _check(lib().qlogits_topk_noalloc(ctypes.byref(W.c), W.N, W.K, W.group, W.bits, W.fmt, _ptr(x),
                                      _xdtype(x), _ptr(norm_w), float(eps), _ptr(logits), k,
                                      _ptr(idx), _ptr(vals), _stream(stream)),
           "qlogits_topk_noalloc")
    return logits, idx, vals


def qlogits_sample(W: QMat, x, k: int, temperature: float, top_p: float, seed: int,
                   counter=None, norm_w=None, eps: float = 1e-5, logits=None, idx=None,
                   vals=None, token=None, ws=None, stream=None):
    """(logits, idx, vals, token): qlogits_topk, then one token drawn from the
    k candidates (token: int32[1] on the device; counter: int64[1] on the
    device, read and advanced by one, or None for draw number 0)."""
    import torch
    dev = x.device
    if logits is None:
        logits = torch.empty(W.N, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty(k, dtype=torch.float32, device=dev)
    _need(x, W.K, "x", (torch.float16, torch.float32))
    _need(norm_w, W.K, "norm_w", _f16())
    _need(logits, W.N, "logits", _f32())
    _need(idx, k, "idx", _i32())
    _need(vals, k, "vals", _f32())
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=dev)
    _need(token, 1, "token", _i32())
    _need(counter, 1, "counter", (torch.int64,))
    wp, wn = _ws_args(ws)
    _check(lib().qlogits_sample(ctypes.byref(W.c), W.N, W.K, W.group, W.bits, W.fmt, _ptr(x),
                                _xdtype(x), _ptr(norm_w), float(eps), _ptr(logits), k, _ptr(idx),
                                _ptr(vals), float(temperature), float(top_p),
                                seed & (2**64 - 1), _ptr(counter), _ptr(token), wp, wn,
                                _stream(stream)), "qlogits_sample")
    return logits, idx, vals, token


def qattn_decode(q, k_cache, v_cache, pos: int, scale: float, k_new=None, v_new=None, out=None,
                 ws=None, stream=None):
    """out [H][d] fp32: one decode step of attention. q [H][d] fp32; caches
    [Hkv][T_max][d] fp16 (k_new/v_new [Hkv][d] fp32 are written at pos first
    when given); positions 0..pos are attended."""
    import torch
    H, d = q.shape
    Hkv, T_max, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != (Hkv, T_max, d):
        raise ValueError("k_cache / v_cache must both be [Hkv][T_max][d] with q's d")
    _need(q, H * d, "q", _f32())
    _need(k_cache, Hkv * T_max * d, "k_cache", _f16())
    _need(v_cache, Hkv * T_max * d, "v_cache", _f16())
    _need(k_new, Hkv * d, "k_new", _f32())
    _need(v_new, Hkv * d, "v_new", _f32())
    if out is None:
        out = torch.empty(H, d, dtype=torch.float32, device=q.device)
    _need(out, H * d, "out", _f32())
    wp, wn = _ws_args(ws)
    _check(lib().qattn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              H, Hkv, d, T_max, int(pos), float(scale), _ptr(out), wp, wn,
                              _stream(stream)), "qattn_decode")
    return out


def qg_sample_topk(idx, vals, temperature: float, top_p: float, seed: int, counter=None,
                   token=None, stream=None):
    """token (int32[1] on the device) drawn from a top-k list (idx, vals)."""
    import torch
    if token is None:
        token = torch.empty(1, dtype=torch.int32, device=idx.device)
    _need(idx, 1, "idx", _i32())
    _need(vals, idx.numel(), "vals", _f32())
    _need(token, 1, "token", _i32())
    _need(counter, 1, "counter", (torch.int64,))
    _check(lib().qg_sample_topk(_ptr(idx), _ptr(vals), int(idx.numel()), float(temperature),
                                float(top_p), seed & (2**64 - 1), _ptr(counter), _ptr(token),
                                _stream(stream)), "qg_sample_topk")
    return token
