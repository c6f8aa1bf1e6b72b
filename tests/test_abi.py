"""Host-side checks of the C ABI: the library loads, exports every entry
point that include/qgemv.h declares, and rejects invalid arguments with the
documented status before touching the GPU. No kernel runs here."""

import ctypes
import os
import re

import pytest

import dequant_gemv_qgemv_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qg.LIB_PATH):
        from dequant_gemv_qgemv_amd import build
        build.build()
    return qg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qg\w+|qgemv\w*|qswiglu|qmoe_experts\w*|qlogits_\w+|qattn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qgemv", "qgemv_rmsnorm", "qswiglu", "qmoe_experts", "qmoe_experts_batch", "qlogits_topk",
              "qlogits_sample", "qg_sample_topk", "qattn_decode",
              "qg_workspace_bytes", "qg_workspace_init", "qg_status_str", "qg_tune"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) <= set(qg.EXPORTED)


def test_status_strings(L):
    for s in (qg.QG_OK, qg.QG_EINVAL, qg.QG_EUNSUPPORTED, qg.QG_EWORKSPACE, qg.QG_ELAUNCH,
              qg.QG_EDEVICE, 12345):
        assert isinstance(qg.qg_status_str(s), str) and qg.qg_status_str(s)


def _mat(q=0x1000, s=0x2000, b=0x3000, lut=None):
    return qg.qg_qmat(q, s, b, lut)


X = ctypes.c_void_p(0x10000)
Y = ctypes.c_void_p(0x80000000)


def call_gemv(L, W=None, N=64, K=128, M=1, group=64, bits=4, fmt=0, x=X, xdt=1, res=None, y=Y):
    W = _mat() if W is None else W
    return L.qgemv(ctypes.byref(W) if W is not False else None, N, K, M, group, bits, fmt, x, xdt,
                   res, y, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=False), qg.QG_EINVAL),                 # NULL descriptor
    (dict(W=_mat(q=0)), qg.QG_EINVAL),            # NULL codes
    (dict(W=_mat(q=0x1008)), qg.QG_EINVAL),       # codes not 16-byte aligned
    (dict(W=_mat(s=0)), qg.QG_EINVAL),            # affine without scales
    (dict(K=100), qg.QG_EINVAL),                  # K not a multiple of 64
    (dict(K=0), qg.QG_EINVAL),
    (dict(N=-1), qg.QG_EINVAL),
    (dict(M=0), qg.QG_EINVAL),
    (dict(group=32), qg.QG_EUNSUPPORTED),
    (dict(bits=3), qg.QG_EUNSUPPORTED),
    (dict(bits=16), qg.QG_EUNSUPPORTED),          # affine codes are 2, 4 or 8 bits
    (dict(bits=1), qg.QG_EUNSUPPORTED),
    (dict(fmt=1, W=_mat(s=0, b=0, lut=0x4000), bits=8), qg.QG_EUNSUPPORTED),  # LUT needs 4 bits
    (dict(fmt=2, W=_mat(s=0, b=0), bits=4), qg.QG_EUNSUPPORTED),  # dense fields are 16 bits
    (dict(fmt=2, W=_mat(q=0, s=0, b=0), bits=16), qg.QG_EINVAL),  # dense without weights
    (dict(M=2, K=576, bits=4), qg.QG_EUNSUPPORTED),              # matrix cores: K % 512
    (dict(fmt=1, W=_mat(s=0, b=0, lut=0x4000), bits=2), qg.QG_EUNSUPPORTED),  # LUT needs 4 bits
    (dict(fmt=1, W=_mat()), qg.QG_EINVAL),        # LUT without a table
    (dict(fmt=7), qg.QG_EINVAL),
    (dict(M=9), qg.QG_EUNSUPPORTED),
    (dict(K=65536 + 64), qg.QG_EUNSUPPORTED),
    (dict(xdt=5), qg.QG_EINVAL),
    (dict(x=None), qg.QG_EINVAL),
    (dict(y=None), qg.QG_EINVAL),
    (dict(x=ctypes.c_void_p(0x10004)), qg.QG_EINVAL),           # x not 16-byte aligned
    (dict(y=ctypes.c_void_p(0x10000 + 64)), qg.QG_EINVAL),      # y overlaps x
    (dict(res=ctypes.c_void_p(0x80000000 + 4)), qg.QG_EINVAL),  # residual partly overlaps y
    (dict(N=1 << 20, K=8192), qg.QG_EUNSUPPORTED),              # matrix over 2^31 bytes
    (dict(M=2, K=576), qg.QG_EUNSUPPORTED),                     # M > 1 needs K % 512 == 0
    (dict(M=2, K=512, W=_mat(s=0x2002)), qg.QG_EUNSUPPORTED),   # ... and 16-byte aligned scales
    (dict(M=2, K=512, W=_mat(b=0x3008)), qg.QG_EUNSUPPORTED),   # ... and biases
    (dict(M=2, K=512, fmt=1, W=_mat(s=0, b=0, lut=0x4008)), qg.QG_EUNSUPPORTED),  # ... and lut
])
def test_qgemv_rejects_before_launch(L, kw, status):
    assert call_gemv(L, **kw) == status


def test_other_entry_points_reject(L):
    W = _mat()
    # rmsnorm without norm weights
    assert L.qgemv_rmsnorm(ctypes.byref(W), 64, 128, 1, 64, 4, 0, X, 1, None, 1e-5, None, Y,
                           None, 0, None) == qg.QG_EINVAL
    # negative eps
    assert L.qgemv_rmsnorm(ctypes.byref(W), 64, 128, 1, 64, 4, 0, X, 1, ctypes.c_void_p(0x20000),
                           -1.0, None, Y, None, 0, None) == qg.QG_EINVAL
    # swiglu without the up matrix
    assert L.qswiglu(ctypes.byref(W), None, 64, 128, 1, 64, 4, 0, X, 1, None, 0.0, Y, None, 0,
                     None) == qg.QG_EINVAL
    # top-k: k out of range, then missing workspace
    logits, idx, vals = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000))
    assert L.qlogits_topk(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 0, idx,
                          vals, None, 0, None) == qg.QG_EINVAL
    assert L.qlogits_topk(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 65, idx,
                          vals, None, 0, None) == qg.QG_EINVAL
    assert L.qlogits_topk(ctypes.byref(W), 2048, 128, 64, 4, 0, X, 1, None, 0.0, logits, 1025,
                          idx, vals, None, 0, None) == qg.QG_EUNSUPPORTED
    assert L.qlogits_topk(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 8, idx,
                          vals, None, 0, None) == qg.QG_EWORKSPACE
    # sampling: temperature, top_p, k, token and counter alignment are checked
    # before anything else; qlogits_sample then checks like qlogits_topk
    tok, ctr = ctypes.c_void_p(0x500000), ctypes.c_void_p(0x600000)
    S = L.qg_sample_topk
    for T, tp, k, t, c in ((-1.0, 1.0, 8, tok, ctr), (float("nan"), 1.0, 8, tok, ctr),
                           (float("inf"), 1.0, 8, tok, ctr), (1.0, 0.0, 8, tok, ctr),
                           (1.0, 1.5, 8, tok, ctr), (1.0, float("nan"), 8, tok, ctr),
                           (1.0, 1.0, 0, tok, ctr), (1.0, 1.0, 8, None, ctr),
                           (1.0, 1.0, 8, ctypes.c_void_p(0x500002), ctr),
                           (1.0, 1.0, 8, tok, ctypes.c_void_p(0x600004))):
        assert S(idx, vals, k, T, tp, 1, c, t, None) == qg.QG_EINVAL, (T, tp, k)
    assert S(idx, vals, 1025, 1.0, 1.0, 1, ctr, tok, None) == qg.QG_EUNSUPPORTED
    assert S(None, vals, 8, 1.0, 1.0, 1, ctr, tok, None) == qg.QG_EINVAL
    QS = L.qlogits_sample
    assert QS(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 8, idx, vals, -1.0,
              1.0, 1, ctr, tok, None, 0, None) == qg.QG_EINVAL
    assert QS(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 65, idx, vals, 1.0,
              1.0, 1, ctr, tok, None, 0, None) == qg.QG_EINVAL
    assert QS(ctypes.byref(W), 64, 128, 64, 4, 0, X, 1, None, 0.0, logits, 8, idx, vals, 1.0,
              1.0, 1, ctr, tok, None, 0, None) == qg.QG_EWORKSPACE
    # attention: shapes, head grouping, position range, alignment, workspace
    A = L.qattn_decode
    qp, kcp, vcp, op = (ctypes.c_void_p(a) for a in (0x700000, 0x800000, 0x900000, 0xA00000))
    ok = dict(q=qp, kn=None, vn=None, kc=kcp, vc=vcp, H=32, Hkv=8, d=128, T=4096, pos=10, sc=0.1, o=op)
    def attn(**kw):
        a = dict(ok, **kw)
        return A(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["H"], a["Hkv"], a["d"], a["T"],
                 a["pos"], a["sc"], a["o"], None, 0, None)
    assert attn(H=30) == qg.QG_EINVAL
    assert attn(pos=4096) == qg.QG_EINVAL and attn(pos=-1) == qg.QG_EINVAL
    assert attn(d=96) == qg.QG_EUNSUPPORTED and attn(H=48, Hkv=3) == qg.QG_EUNSUPPORTED
    assert attn(q=ctypes.c_void_p(0x700004)) == qg.QG_EINVAL
    assert attn(kn=ctypes.c_void_p(0xB00000)) == qg.QG_EINVAL  # k without v
    assert attn(sc=float("nan")) == qg.QG_EINVAL
    assert attn() == qg.QG_EWORKSPACE
    n = ctypes.c_size_t()
    assert L.qg_workspace_bytes(5, 32, 4096, 8, 4, 0, 128, ctypes.byref(n)) == qg.QG_OK and n.value > 0
    assert L.qg_workspace_bytes(5, 32, 4096, 8, 4, 0, 96, ctypes.byref(n)) == qg.QG_EUNSUPPORTED
    # MoE: top_k above the limit, then more than the experts
    lg = ctypes.c_void_p(0x400000)
    assert L.qmoe_experts(ctypes.byref(W), ctypes.byref(W), ctypes.byref(W), 16, 128, 256, 64, 4,
                          0, None, lg, 9, None, 0.0, X, X, None, None, None, 0,
                          None) == qg.QG_EUNSUPPORTED
    assert L.qmoe_experts(ctypes.byref(W), ctypes.byref(W), ctypes.byref(W), 2, 128, 256, 64, 4,
                          0, None, lg, 3, None, 0.0, X, X, None, None, None, 0,
                          None) == qg.QG_EUNSUPPORTED
    # MoE without a workspace
    assert L.qmoe_experts(ctypes.byref(W), ctypes.byref(W), ctypes.byref(W), 16, 128, 256, 64, 4,
                          0, None, lg, 3, None, 0.0, X, X, None, None, None, 0,
                          None) == qg.QG_EWORKSPACE

    # batched MoE: no tokens, too many tokens, output overlapping the input,
    # then a workspace sized for fewer tokens
    def moe_batch(M, y=X, ws=None, nb=0):
        return L.qmoe_experts_batch(ctypes.byref(W), ctypes.byref(W), ctypes.byref(W), 16, 128, 256,
                                    M, 64, 4, 0, None, lg, 3, None, 0.0, X, y, None, None, ws, nb,
                                    None)
    assert moe_batch(0) == qg.QG_EINVAL
    assert moe_batch(9) == qg.QG_EUNSUPPORTED
    assert moe_batch(4, y=ctypes.c_void_p(0x10000 + 256 * 4)) == qg.QG_EINVAL  # token 1 of x
    one, four = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.qg_workspace_bytes(3, 256, 128, 1, 4, 0, 3, ctypes.byref(one)) == qg.QG_OK
    assert L.qg_workspace_bytes(3, 256, 128, 4, 4, 0, 3, ctypes.byref(four)) == qg.QG_OK
    assert four.value > one.value
    assert L.qg_workspace_bytes(3, 256, 128, 9, 4, 0, 3, ctypes.byref(four)) == qg.QG_EUNSUPPORTED
    assert moe_batch(4, ws=ctypes.c_void_p(0x20000000), nb=one.value) == qg.QG_EWORKSPACE


def test_workspace_queries(L):
    for op in (qg.QG_OP_GEMV, qg.QG_OP_GEMV_RMSNORM, qg.QG_OP_SWIGLU):
        assert qg.qg_workspace_bytes(op, 4096, 4096) > 0
    assert qg.qg_workspace_bytes(qg.QG_OP_MOE, 4096, 1024, 1, 4, 0, 3) > 0
    assert qg.qg_workspace_bytes(qg.QG_OP_LOGITS_TOPK, 151936, 1024, 1, 4, 0, 40) > 0
    with pytest.raises(qg.QgError):
        qg.qg_workspace_bytes(qg.QG_OP_LOGITS_TOPK, 100, 64, 1, 4, 0, 2000)
    with pytest.raises(qg.QgError):
        qg.qg_workspace_bytes(99, 1, 1)
    assert L.qg_workspace_init(None, 256, None) == qg.QG_EINVAL
    assert L.qg_workspace_init(ctypes.c_void_p(0x1000), 6, None) == qg.QG_EINVAL


def test_tune_rejects_bad_values(L):
    assert L.qg_tune(9, 1) == qg.QG_EINVAL
    assert L.qg_tune(1, 3) == qg.QG_EINVAL
    assert L.qg_tune(2, 48) == qg.QG_EINVAL
    assert L.qg_tune(0, 17) == qg.QG_EINVAL
    assert L.qg_tune(4, 3) == qg.QG_EINVAL
    assert L.qg_tune(5, 2) == qg.QG_EINVAL
    assert L.qg_tune(6, 2) == qg.QG_EINVAL
    assert L.qg_tune(7, 0) == qg.QG_EINVAL
    for k in range(7):
        assert L.qg_tune(k, 0) == qg.QG_OK


def test_logits_workspace_holds_both_topk_forms(L):
    """The logits workspace: a 1 KiB ticket region, then room for the larger
    of the one-launch top-k's lists (up to 512 workgroup lists and 32 group
    lists of 64 eight-byte keys) and the two-launch top-k's lists (k keys per
    4096-entry slice, rounded up to 256 bytes), then the matvec's region."""
    one = (512 + 32) * 64 * 8
    for V, k in ((151936, 40), (1000, 1), (9000, 1024), (1 << 20, 1024)):
        slices = -(-V // 4096)
        two = -(-slices * k * 8 // 256) * 256
        mv = qg.qg_workspace_bytes(qg.QG_OP_GEMV, V, 1024)
        got = qg.qg_workspace_bytes(qg.QG_OP_LOGITS_TOPK, V, 1024, 1, 4, 0, k)
        assert got == 1024 + max(one, two) + mv, (V, k)


def test_launch_query_checks_arguments(L):
    n = ctypes.c_int(0)
    assert L.qg_logits_topk_launches(None, 1000, 1024, 64, 4, 0, 40, None) == qg.QG_EINVAL
    assert L.qg_logits_topk_launches(None, 1000, 1024, 64, 4, 0, 1001, ctypes.byref(n)) == qg.QG_EINVAL
    assert L.qg_logits_topk_launches(None, 1000, 1024, 64, 4, 0, 0, ctypes.byref(n)) == qg.QG_EINVAL
    assert L.qg_logits_topk_launches(None, 5000, 1024, 64, 4, 0, 1025, ctypes.byref(n)) == qg.QG_EUNSUPPORTED
    assert L.qg_logits_topk_launches(None, 1000, 1000, 64, 4, 0, 4, ctypes.byref(n)) == qg.QG_EINVAL
    assert L.qg_logits_topk_launches(None, 1000, 1024, 32, 4, 0, 4, ctypes.byref(n)) == qg.QG_EUNSUPPORTED


def test_phase_probe_checks_arguments(L):
    p = ctypes.c_void_p(0x10000)
    assert L.qg_probe_phases(None, 256, p, 1, 0, None, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 250, p, 1, 0, None, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 0, 0, None, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, 3, None, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, -1, None, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, 0, None, p, None, 0, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, 0, None, p, None, 4, 0, None) == qg.QG_EINVAL
    # the barrier needs its flags and error counter
    assert L.qg_probe_phases(p, 256, p, 1, 1, None, p, p, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, 1, p, p, None, 4, 16, None) == qg.QG_EINVAL
    assert L.qg_probe_phases(p, 256, p, 1, 2, None, p, p, 4, 16, None) == qg.QG_EINVAL


def test_empty_rows_is_a_no_op(L):
    # N = 0 is valid and enqueues nothing (it returns before any HIP call)
    assert call_gemv(L, N=0) == qg.QG_OK


def test_noalloc_logits_checks_before_any_launch(L):
    """qlogits_topk_noalloc validates its arguments and the size of its
    library-held scratch on the host: these refusals never touch a device."""
    W = _mat()
    LG, IDX, VALS = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)

    def call(V=1000, K=128, k=40, logits=LG, idx=IDX, vals=VALS, x=X):
        return L.qlogits_topk_noalloc(ctypes.byref(W), V, K, 64, 4, 0, x, 1, None, 0.0, logits, k,
                                      idx, vals, None)

    assert call(logits=None) == qg.QG_EINVAL
    assert call(idx=None) == qg.QG_EINVAL
    assert call(k=0) == qg.QG_EINVAL
    assert call(k=1001) == qg.QG_EINVAL
    assert call(k=2000, V=5000) == qg.QG_EUNSUPPORTED  # k beyond QG_MAX_TOPK
    assert call(K=100) == qg.QG_EINVAL  # K not a multiple of the group
    # a vocabulary whose workspace need exceeds the 24 MiB scratch array
    assert call(V=600000, K=64) == qg.QG_EUNSUPPORTED
