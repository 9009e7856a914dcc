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
TRACE_LIB = os.path.join(PKG, "libmoe355_trace.so")
# standalone probe programs (tuning/<name>.hip -> <package>/<name>)
PROBES = ["lds_fill_probe", "kstep_probe", "e4m3_cvt_check"]
SOURCES = ["gemm.hip", "gemm_big.hip", "dense_small.hip", "topk.hip", "sort.hip", "quant.hip", "shuffle.hip", "status.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# per-source extra flags: MFMA results in VGPRs so the fp32 fold reads them directly
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "gemm_big.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain scalar fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _compile(src, save_temps, verbose, trace=False):
    path = os.path.join(CSRC, src)
    obj = os.path.join(CSRC, "_obj", src + (".trace.o" if trace else ".o"))
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    cmd = [HIPCC] + HIP_FLAGS + EXTRA.get(src, []) + (["-DMOE355_PHASE_TRACE"] if trace else []) + ["-c", path, "-o", obj]
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


def _trace_obj(obj, trace_obj):
    """The object of the diagnostic library: the traced gemm.hip in place of the plain one."""
    return trace_obj if obj.endswith(os.sep + "gemm.hip.o") else obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of %s failed" % os.path.basename(lib))
    os.replace(tmp, lib)


def _probe(name, verbose):
    """One standalone probe program: tuning/<name>.hip built to <package>/<name>."""
    out = os.path.join(PKG, name)
    tmp = out + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + ["-mllvm", "-amdgpu-mfma-vgpr-form", os.path.join(PKG, "tuning", name + ".hip"),
                                 "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s.hip" % name)
    os.replace(tmp, out)
    return out


def build(save_temps=None, verbose=False, trace=True):
    """Builds libmoe355.so, (trace) libmoe355_trace.so, the diagnostic variant whose
    gate/up kernel records per-step phase clocks (bench.py --phases), and the probe
    programs lds_fill_probe (LDS fill and operand traffic) and kstep_probe (the engine's
    K step alone)."""
    # the sources compile independently (gemm.hip, the longest, first)
    jobs = [(src, False) for src in SOURCES] + ([("gemm.hip", True)] if trace else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=5) as ex:
        probes = [ex.submit(_probe, name, verbose) for name in PROBES]
        objs = list(ex.map(lambda j: _compile(j[0], save_temps, verbose, j[1]), jobs))
        for pr in probes:
            pr.result()
    _link(objs[:len(SOURCES)], LIB)
    if trace:
        _link([_trace_obj(o, objs[-1]) for o in objs[:len(SOURCES)]], TRACE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.save_temps, a.verbose))
