"""GPU parity of the draw after top-k (page "Booster la vitesse d'inference
sur Apple Silicon", section 1: logits matvec + top-k sampling on the GPU,
only the token comes back): every token the device draws equals the oracle's
token for the same candidates, temperature, top-p and draw number, and the
device counter advances by one per call (also inside a replayed graph).

The device forms the weights with its own double-precision exp; a token can
only differ from the oracle's when the uniform number lands within a few ulps
of a cumulative boundary (probability about 1e-14 per draw), so exact token
equality is the bar."""

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

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
    qg.qg_tune(5, 0)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f32(v):
    """The value the device sees for a float argument."""
    return float(np.float32(v))


def candidates(rng, k, scale):
    vals = np.sort(rng.normal(scale=scale, size=k).astype(np.float32))[::-1].copy()
    idx = rng.choice(151936, size=k, replace=False).astype(np.int32)
    return vals, idx


def oracle_tokens(vals, idx, T, top_p, seed, counters):
    v = vals.astype(np.float64)
    return [oracle.sample(v, idx, f32(T), f32(top_p), oracle.uniform(seed, c)) if T != 0 else
            int(idx[0]) for c in counters]


@pytest.mark.parametrize("k,T,top_p,scale", [(40, 1.0, 1.0, 1.0), (40, 0.7, 0.9, 2.0),
                                              (40, 1.5, 0.5, 0.5), (1, 0.8, 1.0, 1.0),
                                              (2, 1.0, 1.0, 0.3), (1024, 1.0, 0.95, 3.0),
                                              (300, 0.05, 1.0, 1.0), (40, 0.0, 1.0, 1.0)])
def test_sample_topk_matches_oracle(qg, k, T, top_p, scale):
    say(f"qg_sample_topk k={k} T={T} top_p={top_p}")
    rng = np.random.default_rng(k * 7 + int(T * 10))
    vals, idx = candidates(rng, k, scale)
    seed = 0x5EED0000 + k
    n = 200
    start = 17
    counter = torch.tensor([start], dtype=torch.int64, device=DEV)
    tokens = torch.empty(n, dtype=torch.int32, device=DEV)
    dv, di = torch.from_numpy(vals).to(DEV), torch.from_numpy(idx).to(DEV)
    for i in range(n):
        qg.qg_sample_topk(di, dv, T, top_p, seed, counter, token=tokens[i:i + 1])
    torch.cuda.synchronize()
    assert int(counter.item()) == start + n
    got = tokens.cpu().numpy().tolist()
    assert got == oracle_tokens(vals, idx, T, top_p, seed, range(start, start + n))
    if T != 0 and k > 1 and top_p == 1.0 and scale <= 1.0:
        assert len(set(got)) > 1  # a real draw, not a constant


def test_sample_without_counter_uses_draw_zero(qg):
    rng = np.random.default_rng(3)
    vals, idx = candidates(rng, 40, 1.0)
    dv, di = torch.from_numpy(vals).to(DEV), torch.from_numpy(idx).to(DEV)
    toks = [int(qg.qg_sample_topk(di, dv, 1.0, 1.0, 42).item()) for _ in range(3)]
    assert toks == oracle_tokens(vals, idx, 1.0, 1.0, 42, [0, 0, 0])


@pytest.mark.parametrize("path", ["one_launch", "two_launch"])
@pytest.mark.parametrize("V,K,k,T,top_p", [(151936, 1024, 40, 0.8, 0.95), (5000, 256, 1, 1.0, 1.0),
                                            (9000, 64, 1024, 1.0, 1.0), (777, 128, 40, 0.0, 1.0),
                                            (32000, 4096, 64, 1.3, 0.7)])
def test_qlogits_sample_matches_topk_and_oracle(qg, V, K, k, T, top_p, path):
    """The draw in the launch that finishes the top-k: the matvec's own (one
    launch, k <= 64) or the separate top-k kernel (knob 5, and k > 64); the
    tokens are the oracle's draws from the GPU's top-k, draw by draw."""
    say(f"qlogits_sample V={V} K={K} k={k} T={T} top_p={top_p} {path}")
    qg.qg_tune(5, 1 if path == "two_launch" else 0)
    W = qg.QMat.from_host(synth.qmat(21, ("lm", V, K), V, K, 4), DEV)
    g = torch.from_numpy(synth.norm_weight(21, "gf", K)).to(DEV)
    x = torch.from_numpy(synth.activations(21, "x", K, np.float32) * 5.0).to(DEV)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k, DEV)
    z_ref, idx_ref, vals_ref = qg.qlogits_topk(W, x, k, g, 1e-5, ws=ws)
    torch.cuda.synchronize()
    z_ref, idx_ref, vals_ref = z_ref.clone(), idx_ref.clone(), vals_ref.clone()
    seed, start, n = 99, 5, 12
    counter = torch.tensor([start], dtype=torch.int64, device=DEV)
    toks = []
    for _ in range(n):
        z, idx, vals, tok = qg.qlogits_sample(W, x, k, T, top_p, seed, counter, g, 1e-5, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(z, z_ref) and torch.equal(idx, idx_ref) and torch.equal(vals, vals_ref)
        toks.append(int(tok.item()))
    qg.qg_tune(5, 0)
    assert int(counter.item()) == start + n
    assert toks == oracle_tokens(vals_ref.cpu().numpy(), idx_ref.cpu().numpy(), T, top_p, seed,
                                 range(start, start + n))


def test_sample_in_a_replayed_graph_draws_successive_numbers(qg):
    say("qlogits_sample graph replay")
    V, K, k = 20000, 512, 40
    W = qg.QMat.from_host(synth.qmat(22, ("lm", V, K), V, K, 4), DEV)
    x = torch.from_numpy(synth.activations(22, "x", K, np.float32)).to(DEV)
    ws = qg.workspace(qg.QG_OP_LOGITS_TOPK, V, K, 1, 4, 0, k, DEV)
    logits = torch.empty(V, dtype=torch.float32, device=DEV)
    idx = torch.empty(k, dtype=torch.int32, device=DEV)
    vals = torch.empty(k, dtype=torch.float32, device=DEV)
    tok = torch.empty(1, dtype=torch.int32, device=DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        qg.qlogits_sample(W, x, k, 1.0, 1.0, 7, counter, logits=logits, idx=idx, vals=vals,
                          token=tok, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qg.qlogits_sample(W, x, k, 1.0, 1.0, 7, counter, logits=logits, idx=idx, vals=vals,
                          token=tok, ws=ws)
    counter.fill_(100)
    torch.cuda.synchronize()
    got = []
    for r in range(5):
        graph.replay()
        torch.cuda.synchronize()
        got.append(int(tok.item()))
        x.mul_(1.0)  # eager work between replays
    assert int(counter.item()) == 105
    assert got == oracle_tokens(vals.cpu().numpy(), idx.cpu().numpy(), 1.0, 1.0, 7, range(100, 105))
