"""Build the bandwidth probe (probe/librmsn_probe.so) that bench.py times beside
the normalisation kernels. It is not part of the normalisation library: it
streams bytes with the kernels' access pattern and no arithmetic, to show the
practical HBM ceiling of the device the bench runs on."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rmsn_stream_probe.hip")
LIB = os.path.join(HERE, "librmsn_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRC}:\n{err}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
