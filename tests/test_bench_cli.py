"""bench.py's argument checks, which run before anything touches a GPU. CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,needle", [
    (["--gpus", "2"], "one GPU"),
    (["--bits", "16"], "--bits 16 --fmt 2"),
    (["--fmt", "2"], "--bits 16 --fmt 2"),
    (["--fmt", "1", "--bits", "2"], "4-bit codes"),
    (["--m", "9"], "--m must be 1..8"),
    (["--tune", "6"], "KNOB=VALUE"),
    (["--tune", "a=1"], "KNOB=VALUE"),
    (["--config", "nope"], "invalid choice"),
    (["--tp", "3"], "invalid choice"),
    (["--tp", "8", "--m", "2"], "--tp is for --config stack with --m 1"),
    (["--tp", "2", "--config", "qwen"], "--tp is for --config stack with --m 1"),
])
def test_rejected_before_any_gpu_work(args, needle):
    r = run(*args)
    assert r.returncode == 2
    assert needle in r.stderr


def test_several_ranks_are_refused(monkeypatch):
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_tp_shard_shapes():
    """The shard of one GPU under tensor parallelism: qkv / gate.up rows and
    the o / down inputs divided, everything else as the whole model."""
    sys.path.insert(0, ROOT)
    import synth
    m = synth.tp_shard(synth.LLAMA3_8B, 8)
    assert (m["qkv"], m["q_dim"], m["o_in"], m["ffn"]) == (768, 512, 512, 1792)
    assert m["hidden"] == 4096 and m["layers"] == 32 and m["name"] != synth.LLAMA3_8B["name"]
    assert synth.tp_shard(synth.LLAMA3_8B, 1) == synth.LLAMA3_8B
    with pytest.raises(ValueError):
        synth.tp_shard(synth.QWEN3_06B, 64)  # 2048 / 64 columns are not whole groups of 64
