"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m lossless_speculative_kv_amd.build

produces lossless_speculative_kv_amd/libvc.so (the C-ABI hot path) and
synth/libvcsynth.so (the device copy of the seeded input generator). Every
call recompiles; objects go to _build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "lossless_speculative_kv_amd")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("VC_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled: the compiler otherwise forms them
# from ordinary float code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]

LIBS = {
    os.path.join(PKG, "libvc.so"): [
        os.path.join(PKG, "csrc", f) for f in
        ("draft_attn.hip", "verify_attn.hip", "vocab.hip", "round_ops.hip", "api.cpp")],
    os.path.join(ROOT, "synth", "libvcsynth.so"): [os.path.join(ROOT, "synth", "synth_dev.hip")],
}


# Per-source extra flags. The draft attention kernels keep their MFMA
# accumulators in VGPRs: the online-softmax rescale touches them with VALU
# instructions, and in AGPRs every touch is a copy out and back.
EXTRA = {
    "draft_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for lst in LIBS.values() for s in lst]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    out = []
    for lib, lst in LIBS.items():
        tmp = lib + ".tmp"
        cmd = [HIPCC, *COMMON, "-shared", "-o", tmp, *[objs[s] for s in lst]]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {lib}:\n{r.stderr}")
        os.replace(tmp, lib)
        out.append(lib)
        if verbose:
            print(f"built {os.path.relpath(lib, ROOT)}")
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
