"""The host side of the library and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU).

Builds (gcc/g++, -fsanitize=address,undefined, every finding fatal):
  * the host part of the C ABI -- abi.cpp's argument checks, threaded blob
    packer and unpacker, workspace sizing -- with the kernel launches replaced
    by stubs (tests/sanitize/launch_stubs.cpp);
  * oracle.c, with OpenMP.
Then runs the host ABI tests (among them pack/unpack round trips of every
format at the largest widths the ABI takes) and the oracle pins against those
builds in a child process with the ASan runtime preloaded.  A report from either
sanitizer ends the child with a non-zero status and fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]


def _build():
    os.makedirs(OUT, exist_ok=True)
    moe = os.path.join(OUT, "libmoe_host_san.so")
    orc = os.path.join(OUT, "liborc_san.so")
    subprocess.check_call(
        ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         os.path.join(ROOT, "expert_grouped_quantized_amd", "csrc", "abi.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", moe, "-lpthread"])
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
                           "-o", orc, "-lm"])
    return moe, orc


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs the HIP headers")
def test_host_side_and_oracle_under_asan_ubsan():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc has no libasan")
    moe, orc = _build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (asan, os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["MOE_LIB_OVERRIDE"] = moe
    env["ORC_LIB_OVERRIDE"] = orc
    env["OMP_NUM_THREADS"] = "4"
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_abi_host.py", "test_oracle_pins.py", "test_oracle_mx.py")]
    # -s: a sanitizer report goes to the child's stderr and the child exits at
    # once; with pytest's own capture the report would be lost with it
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m",
                        "not gpu and not slow", "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=1800)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    print(tail.splitlines()[-1])
