"""Build the HIP library libfa4.so in-tree with hipcc for gfx950.

Usage: python fp8_quantized_attention_amd/build.py [--sanitize]   (or __graft_entry__.build()); run it as
a script so that the package (which loads the library) is not imported first. --sanitize builds the
host-sanitized copy under _build/sanitize/ instead.
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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # hand-written kernels only; no packed fp32 instructions (see the notes on the target)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around the decode kernel's MFMAs)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # IEEE float division (the quantizers' rounding depends on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
]
# Per-source additions. The attention kernels take maxima of MFMA results, which the compiler would
# otherwise first quiet for signalling NaNs (one extra instruction per operand); no NaN reaches them
# (masked scores are -inf, every row has an unmasked key), so they are compiled without NaN semantics.
SOURCE_FLAGS = {"attn_fwd.hip": ["-fno-honor-nans"]}


# The host code (argument validation, dispatch) with AddressSanitizer and UndefinedBehaviorSanitizer, for
# tests of the C ABI on the CPU: the sanitizers apply to host code only, device code is built at -O1.
SAN_LIB = os.path.join(HERE, "_build", "sanitize", "libfa4.so")
SAN_FLAGS = [
    "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
    # each sanitizer flag right after -Xarch_host: host code only
    "-Xarch_host", "-fsanitize=" + "address", "-Xarch_host", "-fsanitize=" + "undefined",
    "-Xarch_device", "-O1",
]


def sanitizer_runtime():
    """The clang AddressSanitizer runtime that a process loading SAN_LIB must preload."""
    import glob
    libs = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*", "lib",
                                         "linux", "libclang_rt.asan-x86_64.so")))
    return libs[-1] if libs else None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)


def build(verbose=False, extra_flags=(), sanitize=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    dst = SAN_LIB if sanitize else LIB
    os.makedirs(os.path.dirname(dst), exist_ok=True)
    tmp = dst + ".tmp"
    inc = ["-I", os.path.join(HERE, "..", "include")]
    if sanitize:
        _run([HIPCC, *SAN_FLAGS, *extra_flags, *inc, "-o", tmp, *srcs], verbose)
    else:
        # one object per source (in parallel), each with its own additions, then one shared library
        objdir = os.path.join(HERE, "_build", "obj")
        os.makedirs(objdir, exist_ok=True)
        jobs, objs = [], []
        for name, src in zip(SOURCES, srcs):
            obj = os.path.join(objdir, name + ".o")
            cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(name, []), *extra_flags, *inc, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), name))
            objs.append(obj)
        errors = []
        for proc, name in jobs:
            out = "\n".join(l for l in proc.communicate()[0].splitlines() if "packed-fp32-ops" not in l)
            if proc.returncode != 0:
                errors.append(f"{name}:\n{out}")
            elif verbose and out.strip():
                print(out)
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
