"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

xattn_api.cpp and profile.cpp are compiled with -fsanitize=address,undefined on the host side
(device code is not instrumented) and linked with the library's other objects into
tests/sanitize/boundary_driver.cpp, a C++ caller of every entry point with invalid arguments
and size queries.  No call reaches a kernel launch.  The run must report no sanitizer error and
every documented status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_gqa_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIP_OBJECTS = ["attn.o", "attn_bf16.o", "prologue.o", "decode.o", "proj.o", "gemm.o",
               "noalloc.o"]
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def test_c_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    objs = [os.path.join(BUILD, o) for o in HIP_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        from causal_gqa_attention_amd import build
        build.build()
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-fno-sanitize-recover=undefined"]
    sources = [(os.path.join(CSRC, "xattn_api.cpp"), "api.o"),
               (os.path.join(CSRC, "profile.cpp"), "profile.o"),
               (os.path.join(ROOT, "tests", "sanitize", "boundary_driver.cpp"), "driver.o")]
    for src, obj in sources:
        rc, out = _run([hipcc, *flags, *SANITIZE, "-c", src, "-o", str(tmp_path / obj)])
        assert rc == 0, out
    exe = str(tmp_path / "boundary_driver")
    rc, out = _run([hipcc, "--offload-arch=gfx950", "-o", exe,
                    *[str(tmp_path / o) for _, o in sources], *objs, *SANITIZE])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, out = _run([exe], env=env, timeout=120)
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert "LeakSanitizer" not in out, out
    assert rc == 0 and "0 failures" in out, out
