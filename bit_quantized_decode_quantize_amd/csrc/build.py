"""Build libbqd.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m bit_quantized_decode_quantize_amd.csrc.build

The library links libamdhip64 by soname, so inside a process that imported
torch first it binds to torch's HIP runtime (one runtime per process).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
SRC = os.path.join(HERE, "bqd_kernels.hip")
OUT = os.path.join(PKG, "libbqd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-mcode-object-version=5",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra=(), out=OUT, verbose=False):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
