"""Build libdsa.so (the C-ABI library of the DSA hot path) for gfx950 with hipcc.

Usage: python -m sparse_attention_long_06_amd.build [-v]

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into sparse_attention_long_06_amd/libdsa.so next to this file.  The
attainable-peak probes under probes/ (include/dsa_probes.h; used by bench.py
only) are linked into libdsa_probes.so the same way.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
PROBES = os.path.join(HERE, "probes")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
PROBES_LIB = os.path.join(HERE, "libdsa_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# Per-file extra flags.  The indexer keeps its MFMA accumulators in ordinary
# VGPRs (its register budget allows it), so the epilogue reads them without
# accumulator-register moves.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources(folder: str = CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile and link libdsa.so and libdsa_probes.so; returns the path of libdsa.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    lib_srcs, probe_srcs = sources(CSRC), sources(PROBES)
    with ThreadPoolExecutor(max_workers=min(8, len(lib_srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, verbose), lib_srcs + probe_srcs))
    _link(objs[: len(lib_srcs)], LIB)
    _link(objs[len(lib_srcs):], PROBES_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
