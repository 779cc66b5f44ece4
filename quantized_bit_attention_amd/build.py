"""Build libsage.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsage.so")
SOURCES = ["sage_api.cpp", "sage_quant.hip", "sage_attn.hip", "sage_bwd.hip"]
HEADERS = ["sage_device.h", "sage_internal.h", "sage_tiles.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(out: str = LIB, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "hip", *sources(), "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building libsage.so")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
