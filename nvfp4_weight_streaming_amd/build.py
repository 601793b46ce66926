"""Build libnvfp4.so (all HIP sources, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # No packed fp32 (v_pk_*_f32) generation.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs (no accumulation-register round trips).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


# The prefill kernel keeps its 256 accumulators per lane in the accumulation
# registers, so it is built without the VGPR form.
AGPR_SOURCES = ("prefill.hip",)


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def flags_for(src):
    fl = [f for f in FLAGS if f != "-shared"]
    if os.path.basename(src) in AGPR_SOURCES:
        i = fl.index("-amdgpu-mfma-vgpr-form")
        del fl[i - 1:i + 1]
    return fl


def build(verbose: bool = False) -> str:
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    procs = []
    for src in sources():
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        cmd = [HIPCC] + flags_for(src) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for src, text in failed:
            sys.stderr.write("hipcc failed on %s:\n%s\n" % (src, text))
        raise RuntimeError("HIP build failed")
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
