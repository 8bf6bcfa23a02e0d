"""Build libsparselora.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled with:
  --offload-arch=gfx950 -O3
  -ffp-contract=off                     (no implicit fused multiply-add: the
                                          channel scores are defined op by op)
  -fno-gpu-flush-denormals-to-zero      (IEEE binary32 denormals)
  -fhip-fp32-correctly-rounded-divide-sqrt
  -Xclang -target-feature -Xclang -packed-fp32-ops   (no packed fp32 VALU ops)
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparselora.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sl_api.cpp", "k_select.hip", "k_gemm.hip", "k_lora.hip", "k_layer.hip", "k_train.hip", "k_factor.hip", "k_attn.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I" + os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # a kernel whose host-side stub was not emitted links fine and fails at load
    nm = subprocess.run(["nm", "-u", tmp], capture_output=True, text=True)
    missing = [l for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the library:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
