"""CPU-only sanitizer builds of the host gzip stage (gsa_prepare and the persistent pool).

The stress driver (tests/native/prep_stress.cpp) is compiled with g++ together with the
host-stage sources under ThreadSanitizer, and again under AddressSanitizer with
UndefinedBehaviorSanitizer; it runs gsa_prepare at several thread counts, the pool with
back-to-back submits and changing block sizes, destroy during a batch, and the zlib
error path through a test-only allocator hook (GSA_TEST_HOOKS, never defined in the
library build), which makes deflate's allocations fail so that gsa_prepare and the pool
return GSA_ERR_ZLIB.  The sizes are checked against the one-thread gsa_prepare inside the
driver.  No GPU code is built or run here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "content_adaptive_block_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SANITIZERS = {
    "thread": ["-fsanitize=thread"],
    "address-undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
}


@pytest.mark.parametrize("kind", list(SANITIZERS))
def test_host_stage_under_sanitizer(kind, tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / f"prep_stress_{kind}"
    cmd = [gxx, "-O1", "-g", "-std=c++17", *SANITIZERS[kind], "-DGSA_TEST_HOOKS", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{ROCM}/include",
           os.path.join(ROOT, "tests", "native", "prep_stress.cpp"), os.path.join(CSRC, "gsa_prepare.cpp"),
           os.path.join(CSRC, "gsa_error.cpp"), "-lz", "-lpthread", "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66",
               ASAN_OPTIONS="detect_leaks=1 halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout[-4000:]
    assert "WARNING: ThreadSanitizer" not in r.stdout and "ERROR: AddressSanitizer" not in r.stdout
