"""Build libmoe355.so in-tree with hipcc for gfx950.

    python -m fp8_block_scaled_grouped_amd.build [--save-temps DIR]

Every source under csrc/ is compiled on each call (no staleness check), so
the library always matches the tree.
"""
import argparse
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe355.so")
SOURCES = ["gemm.hip", "topk.hip", "sort.hip", "quant.hip", "shuffle.hip", "status.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# per-source extra flags: MFMA results in VGPRs so the fp32 fold reads them directly
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain scalar fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _compile(src, save_temps, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(CSRC, "_obj", src + ".o")
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    cmd = [HIPCC] + HIP_FLAGS + EXTRA.get(src, []) + ["-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    if save_temps and src.endswith(".hip"):
        os.makedirs(save_temps, exist_ok=True)
        cmd += ["-save-temps=obj"]
        cmd[cmd.index("-o") + 1] = os.path.join(save_temps, src + ".o")
        obj = cmd[cmd.index("-o") + 1]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on " + src)
    return obj


def build(save_temps=None, verbose=False):
    # the sources compile independently (gemm.hip, the longest, first)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda src: _compile(src, save_temps, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmoe355.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.save_temps, a.verbose))
