"""The library's host code under AddressSanitizer, on the CPU (no GPU).

A second build of the same sources instruments only the host pass (argument checks, the
n-gram proposer, model-description checks, error strings, fault injection); it is loaded
through SF_LIB with the ASan runtime preloaded, and the host-side ABI tests run against it
in a child process.  Any ASan report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import os, sys
import pytest
import speculative_decoding_verification_decode_amd as sfb
assert sfb.LIB_PATH == os.environ["SF_LIB"], sfb.LIB_PATH
sfb.lib()
maps = open("/proc/self/maps").read()
assert "libsf_asan.so" in maps and "libclang_rt.asan" in maps
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", os.path.join(sys.argv[1], "tests", "test_abi_cpu.py")]))
"""


def test_host_abi_paths_are_clean_under_asan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime in this image")
    from speculative_decoding_verification_decode_amd import build
    lib = build.build_asan(str(tmp_path))
    env = dict(os.environ, SF_LIB=lib, LD_PRELOAD=rt[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True, text=True,
                       timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
