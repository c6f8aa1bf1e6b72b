"""Host-only checks of the Python binding: tensors handed to the library by
pointer are refused when undersized, non-contiguous or of the wrong dtype,
before any library call (the C-ABI cannot see a buffer's size)."""
import pytest

torch = pytest.importorskip("torch")
import dequant_gemv_qgemv_amd as qg  # noqa: E402


def qmat(N=32, K=128, bits=4, fmt=qg.QG_AFFINE, **over):
    t = dict(q=torch.zeros(N, K * bits // 32, dtype=torch.int32),
             scales=torch.zeros(N, K // 64, dtype=torch.float16),
             biases=torch.zeros(N, K // 64, dtype=torch.float16),
             lut=torch.zeros(N, 16, dtype=torch.float16) if fmt == qg.QG_LUT else None)
    if fmt == qg.QG_LUT:
        t["scales"] = t["biases"] = None
    t.update(over)
    return qg.QMat(t["q"], t["scales"], t["biases"], t["lut"], N=N, K=K, bits=bits, fmt=fmt)


def test_qmat_sizes():
    qmat()
    qmat(fmt=qg.QG_LUT)
    with pytest.raises(ValueError):
        qmat(q=torch.zeros(32, 15, dtype=torch.int32))
    with pytest.raises(ValueError):
        qmat(scales=torch.zeros(31, 2, dtype=torch.float16))
    with pytest.raises(TypeError):
        qmat(biases=torch.zeros(32, 2, dtype=torch.float32))
    with pytest.raises(ValueError):
        qmat(fmt=qg.QG_LUT, lut=torch.zeros(32, 8, dtype=torch.float16))


def test_matvec_buffers():
    W = qmat()
    x = torch.zeros(128)
    with pytest.raises(ValueError):
        qg.qgemv(W, torch.zeros(127))  # x shorter than K
    with pytest.raises(ValueError):
        qg.qgemv(W, torch.zeros(2, 100))  # rows of the wrong length
    with pytest.raises(ValueError):
        qg.qgemv(W, x, y=torch.zeros(31))
    with pytest.raises(ValueError):
        qg.qgemv(W, torch.zeros(2, 128), y=torch.zeros(32))  # [M, N] output needs M * N
    with pytest.raises(ValueError):
        qg.qgemv(W, x, residual=torch.zeros(16))
    with pytest.raises(TypeError):
        qg.qgemv(W, x, y=torch.zeros(32, dtype=torch.float16))
    with pytest.raises(ValueError):
        qg.qgemv(W, torch.zeros(256)[::2])  # not contiguous
    with pytest.raises(ValueError):
        qg.qgemv_rmsnorm(W, x, torch.zeros(64, dtype=torch.float16))
    with pytest.raises(ValueError):
        qg.qswiglu(W, W, x, u=torch.zeros(8))


def test_logits_and_sampling_buffers():
    W = qmat(N=100)
    x = torch.zeros(128)
    with pytest.raises(ValueError):
        qg.qlogits_topk(W, x, 8, logits=torch.zeros(99))
    with pytest.raises(ValueError):
        qg.qlogits_topk(W, x, 8, idx=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(TypeError):
        qg.qlogits_topk(W, x, 8, idx=torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError):
        qg.qlogits_topk_noalloc(W, x, 8, vals=torch.zeros(7))
    with pytest.raises(TypeError):
        qg.qlogits_sample(W, x, 8, 1.0, 0.9, 1, counter=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        qg.qg_sample_topk(torch.zeros(8, dtype=torch.int32), torch.zeros(4), 1.0, 0.9, 1)


def test_moe_and_attention_buffers():
    gate = qmat(N=4 * 16, K=128)
    down = qmat(N=4 * 128, K=64)
    x = torch.zeros(128)
    with pytest.raises(ValueError):
        qg.qmoe_experts(gate, gate, down, 4, None, torch.zeros(3), 2, x)
    with pytest.raises(ValueError):
        qg.qmoe_experts(gate, gate, down, 4, None, torch.zeros(4), 2, x,
                        sel_ids=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        qg.qmoe_experts_batch(gate, gate, down, 4, None, torch.zeros(4), 2, torch.zeros(2, 128))
    q = torch.zeros(8, 64)
    kc = torch.zeros(2, 16, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        qg.qattn_decode(q, kc, torch.zeros(2, 8, 64, dtype=torch.float16), 3, 0.125)
    with pytest.raises(ValueError):
        qg.qattn_decode(q, kc, kc.clone(), 3, 0.125, k_new=torch.zeros(64))
    with pytest.raises(ValueError):
        qg.qattn_decode(q, kc, kc.clone(), 3, 0.125, out=torch.zeros(8, 32))
