"""Builds libqgemv.so (the gfx950 HIP kernels + C ABI) in this directory.

hipcc cross-compiles for gfx950 without a GPU. Packed-fp32 instructions are
disabled for all device code (-packed-fp32-ops); the host pass warns that it
does not know that feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemv.so")
SOURCES = ["qg_api.hip", "qg_mv.hip", "qg_mm.hip", "qg_topk.hip", "qg_moe.hip", "qg_attn.hip", "qg_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library (always rebuilds)."""
    objs = []
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(" ".join(cmd) + "\n" + out)
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(failed))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
