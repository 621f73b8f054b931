"""Build libsf.so in-tree with hipcc for gfx950.

    python -m speculative_decoding_verification_decode_amd.build
    python -m speculative_decoding_verification_decode_amd.build --asan OUT_DIR   (host ASan build)
    python -m speculative_decoding_verification_decode_amd.build --checks         (device-checking build)
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsf.so")
SOURCES = ["kernels.hip", "runtime.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # Packed fp32 vector ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected.
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libsf.so")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


# Host code under AddressSanitizer: the same sources with the device code built as usual and
# only the host pass instrumented.  Loaded through SF_LIB with the ASan runtime preloaded.
ASAN_HOST_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_asan(out_dir):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    out = os.path.join(out_dir, "libsf_asan.so")
    flags = [f for f in FLAGS if f != "-O3"] + ASAN_HOST_FLAGS
    cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building the AddressSanitizer library")
    return out


# Checking build: the same sources with SF_CHECKS=1, so kernels record violated invariants
# (token ids, draft counts, positions and commits against the capacity, NaN logits) in a
# device word that sf_debug_checks reads.  A library of its own, loaded through SF_LIB.
CHECKS_LIB = os.path.join(PKG, "libsf_checks.so")


def build_checks(out=CHECKS_LIB):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-DSF_CHECKS=1", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building the checking library")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if sys.argv[1:2] == ["--asan"]:
        print(build_asan(sys.argv[2] if len(sys.argv) > 2 else os.getcwd()))
    elif sys.argv[1:2] == ["--checks"]:
        print(build_checks())
    else:
        print(build(verbose=True))
