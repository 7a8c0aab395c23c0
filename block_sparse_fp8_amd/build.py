"""Build libbsa_fp8.so in-tree with hipcc for gfx950.

    python -m block_sparse_fp8_amd.build
"""
import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
SOURCES = [os.path.join(_HERE, "csrc", "bsa_fp8_prefill.hip"),
           os.path.join(_HERE, "csrc", "bsa_fp8_schedule.hip"),
           os.path.join(_HERE, "csrc", "bsa_fp8_quantize.hip"),
           os.path.join(_HERE, "csrc", "bsa_fp8_decode.hip"),
           os.path.join(_HERE, "csrc", "bsa_fp8_status.cpp")]
OUTPUT = os.path.join(_HERE, "libbsa_fp8.so")

# Packed fp32 VALU forms are switched off for all device code.  Device code
# does not rely on NaN propagation (it never sees NaN from valid inputs), so
# NaN-quieting canonicalisations before max operations are not needed.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_device", "-fno-honor-nans",
    "-I" + os.path.join(_ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False):
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + OUTPUT)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
