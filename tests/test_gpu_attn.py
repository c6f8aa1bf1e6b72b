"""GPU parity of the decode attention step (page "Booster la vitesse
d'inference sur Apple Silicon", section 2 "KV cache": fp16 cache laid out
along time per head, one query, split along the cache, GQA) against the
oracle's plain softmax attention on the same cache contents. The new k/v
row written at `pos` must be the nearest fp16 of the given values, bit for
bit; the output follows the floating-point bar of the matvecs (max error at
most 2e-3 of the largest reference value per call); repeated calls are
bitwise identical."""

import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-3


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


def setup(seed, H, Hkv, d, T_max, qscale=1.0):
    rng = np.random.default_rng(seed)
    kc = rng.normal(size=(Hkv, T_max, d)).astype(np.float16)
    vc = rng.normal(size=(Hkv, T_max, d)).astype(np.float16)
    q = (rng.normal(size=(H, d)) * qscale).astype(np.float32)
    kn = rng.normal(size=(Hkv, d)).astype(np.float32)
    vn = rng.normal(size=(Hkv, d)).astype(np.float32)
    return kc, vc, q, kn, vn


def check(out, ref, what):
    out = np.asarray(out, np.float64)
    assert np.all(np.isfinite(out)), what
    err = np.max(np.abs(out - ref))
    bound = TOL * np.max(np.abs(ref))
    assert err <= bound, f"{what}: max err {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("H,Hkv,d,T_max,pos", [
    (32, 8, 128, 4096, 0), (32, 8, 128, 4096, 1), (32, 8, 128, 4096, 63), (32, 8, 128, 4096, 64),
    (32, 8, 128, 4096, 1000), (32, 8, 128, 4096, 4095),   # Llama-3-8B heads
    (16, 8, 128, 2048, 777),                                # Qwen3-0.6B heads
    (8, 8, 64, 3000, 2999), (8, 1, 64, 5000, 4321), (4, 2, 128, 130, 129), (8, 4, 64, 1, 0)])
def test_attention_with_new_row(qg, H, Hkv, d, T_max, pos):
    say(f"qattn_decode H={H} Hkv={Hkv} d={d} T_max={T_max} pos={pos}")
    kc, vc, q, kn, vn = setup(H * 1000 + pos, H, Hkv, d, T_max)
    scale = 1.0 / np.sqrt(d)
    dk, dv = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    dq, dkn, dvn = (torch.from_numpy(a).to(DEV) for a in (q, kn, vn))
    ws = qg.workspace(qg.QG_OP_ATTN, H, T_max, Hkv, k=d, device=DEV)
    out = qg.qattn_decode(dq, dk, dv, pos, scale, dkn, dvn, ws=ws)
    torch.cuda.synchronize()
    kc2, vc2 = dk.cpu().numpy(), dv.cpu().numpy()
    assert np.array_equal(kc2[:, pos], kn.astype(np.float16))
    assert np.array_equal(vc2[:, pos], vn.astype(np.float16))
    others = np.ones(T_max, bool)
    others[pos] = False
    assert np.array_equal(kc2[:, others], kc[:, others]) and np.array_equal(vc2[:, others], vc[:, others])
    ref = oracle.attention(q.astype(np.float64), kc2, vc2, pos + 1, scale)
    check(out.cpu().numpy(), ref, "attention")
    out2 = qg.qattn_decode(dq, dk, dv, pos, scale, dkn, dvn, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("pos,qscale", [(32767, 1.0), (20000, 8.0)])
def test_attention_long_context_existing_cache(qg, pos, qscale):
    say(f"qattn_decode long context pos={pos} qscale={qscale}")
    H, Hkv, d, T_max = 32, 8, 128, 32768
    kc, vc, q, _, _ = setup(pos, H, Hkv, d, T_max, qscale)
    scale = 1.0 / np.sqrt(d)
    dk, dv, dq = (torch.from_numpy(a).to(DEV) for a in (kc, vc, q))
    ws = qg.workspace(qg.QG_OP_ATTN, H, T_max, Hkv, k=d, device=DEV)
    out = qg.qattn_decode(dq, dk, dv, pos, scale, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(dk.cpu(), torch.from_numpy(kc))  # no row given: cache untouched
    ref = oracle.attention(q.astype(np.float64), kc, vc, pos + 1, scale)
    check(out.cpu().numpy(), ref, "long-context attention")


def test_attention_steps_reuse_the_workspace(qg):
    say("qattn_decode successive steps")
    H, Hkv, d, T_max = 16, 8, 128, 600
    kc, vc, _, _, _ = setup(9, H, Hkv, d, T_max)
    dk, dv = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    ws = qg.workspace(qg.QG_OP_ATTN, H, T_max, Hkv, k=d, device=DEV)
    rng = np.random.default_rng(10)
    host_k, host_v = kc.copy(), vc.copy()
    for pos in (100, 101, 102, 300, 599):
        q = rng.normal(size=(H, d)).astype(np.float32)
        kn = rng.normal(size=(Hkv, d)).astype(np.float32)
        vn = rng.normal(size=(Hkv, d)).astype(np.float32)
        out = qg.qattn_decode(torch.from_numpy(q).to(DEV), dk, dv, pos, 0.1,
                              torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV), ws=ws)
        host_k[:, pos] = kn.astype(np.float16)
        host_v[:, pos] = vn.astype(np.float16)
        torch.cuda.synchronize()
        ref = oracle.attention(q.astype(np.float64), host_k, host_v, pos + 1, 0.1)
        check(out.cpu().numpy(), ref, f"step pos={pos}")
