"""Builds libmoe4.so (all HIP sources under csrc/) in-tree for gfx950.

    python -m precision_moe_numerics_quant_amd.build

Flags: -ffp-contract=off keeps every float operation a separate IEEE
operation (the quantisers must match their specification bit for bit);
packed-fp32 instruction selection is disabled; the default correctly rounded
float32 division is kept.

The SiLU / SiLU' tables are constant data of the library: gen_act_tab.cpp,
compiled and run on the host first, writes them as the initialiser that
capi.hip includes (act_tab.inc, in the build directory).
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe4.so")
SOURCES = ["capi.hip", "nvfp4_quant.hip", "mxfp8.hip", "route.hip", "gemm_fwd.hip", "gemm_bwd.hip", "combine_q.hip", "router.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def build(verbose=False, jobs=8):
    tmp = tempfile.mkdtemp(prefix="moe4_build_")
    try:
        gen = os.path.join(tmp, "gen_act_tab")
        r = subprocess.run([CXX, "-O2", "-std=c++17", "-o", gen, os.path.join(CSRC, "gen_act_tab.cpp")],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("activation table generator failed to compile:\n" + r.stdout)
        with open(os.path.join(tmp, "act_tab.inc"), "w") as f:
            subprocess.run([gen], stdout=f, check=True)
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [HIPCC] + FLAGS + ["-I", tmp, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs)
                procs = []
        _wait(procs)
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


def _wait(procs):
    errs = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            errs.append(f"{src}:\n{text}")
        elif "error" in text:
            errs.append(f"{src}:\n{text}")
    if errs:
        raise RuntimeError("HIP compile failed:\n" + "\n".join(errs))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
