"""Build the HIP libraries in-tree for gfx950: ``libmoe.so`` (the layer) and ``synth/libmoe_synth.so``
(the device fill of synthetic inputs). Always recompiles. Usage: ``python fine_grained_mixture_gemm_amd/build.py``
(runs without importing the package, which needs the built library)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["capi.hip", "router.hip", "dispatch.hip", "quant.hip", "gemm_mfma.hip", "gemm_decode.hip", "gemm_simt.hip", "combine.hip", "balance.hip", "backward.hip"]
LIB = os.path.join(PKG, "libmoe.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "csrc", "synth_dev.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libmoe_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are kept out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include")] + DEVICE_FLAGS


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = [[HIPCC] + FLAGS + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs.append([HIPCC] + FLAGS + ["-shared", SYNTH_SRC, "-o", SYNTH_LIB + ".tmp"])
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", LIB + ".tmp"])
    os.replace(LIB + ".tmp", LIB)
    os.replace(SYNTH_LIB + ".tmp", SYNTH_LIB)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB, SYNTH_LIB)
