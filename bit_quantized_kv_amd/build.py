"""Build the HIP library ``libtq.so`` in-tree for gfx950.

Usage: ``python bit_quantized_kv_amd/build.py`` (or ``__graft_entry__.build()``).
Every source is compiled on each call; objects go to ``_build/`` at the
repository root and the shared library next to this file.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtq.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["tq_host.cpp", "tq_tables.cpp", "tq4_quantize.hip", "tq4_decode.hip", "mxfp4.hip", "calibrate.hip", "tq4_multitoken.hip", "debug_dequant.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep every fp32 rounding where the source writes it (no fma contraction)
    "-ffp-contract=off",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    warn = [ln for ln in p.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return obj, warn


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, w in results:
            for ln in w:
                print(ln, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fno-gpu-rdc", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    shutil.move(tmp, OUT)
    build_probe()
    return OUT


PROBE_SRC = os.path.join(HERE, "probe", "ceiling.hip")
PROBE_OUT = os.path.join(HERE, "libtqprobe.so")


def build_probe():
    """The bench's bandwidth probes (stream read, record gather), a library of
    their own: no entry point of libtq.so uses them."""
    tmp = PROBE_OUT + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", "-x", "hip", PROBE_SRC, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    shutil.move(tmp, PROBE_OUT)
    return PROBE_OUT


if __name__ == "__main__":
    print(build(verbose=True))
