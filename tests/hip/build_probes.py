"""Build the test-only HIP probes under tests/hip/ (gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PROBES = {"mfma_precision.hip": "libmfma_precision.so"}


def build():
    for src, lib in PROBES.items():
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", os.path.join(HERE, src), "-o", os.path.join(HERE, lib)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")


if __name__ == "__main__":
    build()
