"""Build the HIP library libfa4.so in-tree with hipcc for gfx950.

Usage: python fp8_quantized_attention_amd/build.py   (or __graft_entry__.build()); run it as a script so
that the package (which loads the library) is not imported first.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa4.so")
SOURCES = ["fa4_abi.hip", "quantize.hip", "select.hip", "attn_fwd.hip", "decode.hip", "decode_mla.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # hand-written kernels only; no packed fp32 instructions (see the notes on the target)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around the decode kernel's MFMAs)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # IEEE float division (the quantizers' rounding depends on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
]


def build(verbose=False, extra_flags=()):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(HERE, "..", "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
