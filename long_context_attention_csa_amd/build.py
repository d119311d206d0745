"""Build libcsa_hip.so (gfx950 only) in the package directory with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel, then
linked into one shared library. Run as ``python -m long_context_attention_csa_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa_hip.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Werror",
    # the host pass warns that it does not know the device-only feature below
    "-Wno-unused-command-line-argument",
    # packed fp32 vector instructions stay off (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source extra flags. The indexer's and the attention's MFMA results feed
# VALU math at once (weighted ReLU, softmax, rescaling): the VGPR form of the
# MFMA saves an accumulator-register copy per element.
EXTRA = {
    "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"   # host pass does not know the device feature: harmless
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_native_demo(verbose)
    return LIB


# A plain C program that drives the library through its C ABI alone (no
# Python), used by the tests: tests/native/layer_demo.c -> tests/native/layer_demo.
DEMO_SRC = os.path.join(os.path.dirname(HERE), "tests", "native", "layer_demo.c")
DEMO = os.path.join(os.path.dirname(HERE), "tests", "native", "layer_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_native_demo(verbose: bool = True) -> str | None:
    if not os.path.exists(DEMO_SRC):
        return None
    cc = os.environ.get("CC", "gcc")
    inc = os.path.join(os.path.dirname(HERE), "include")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{inc}",
           f"-I{ROCM}/include", DEMO_SRC, f"-L{HERE}", "-lcsa_hip", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../long_context_attention_csa_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", DEMO + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {DEMO_SRC} failed:\n{r.stdout}{r.stderr}")
    os.replace(DEMO + ".tmp", DEMO)
    if verbose:
        print(f"built {DEMO}")
    return DEMO


if __name__ == "__main__":
    build()
