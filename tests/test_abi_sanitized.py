"""The C ABI's argument checks under the host address and undefined-behaviour sanitizers.

`tests/abi_check.cpp` (with `tests/abi_check_c.c` for the one call only C can make) calls every entry point with arguments it must reject (null or
misaligned pointers, bad shapes and dtypes, missing or short workspace) and with the
documented no-ops (M = 0), plus the size, name and status-string functions. It is linked
against the library's objects with the API translation unit rebuilt under
-fsanitize=address,undefined (host code only: each flag directly after -Xarch_host), so any
out-of-bounds read, use of freed memory or undefined behaviour on those paths aborts the run.
No GPU is needed: every call returns before anything is enqueued.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(900)
def test_abi_argument_checks_under_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from weight_only_int4_w4a16_amd import build as b

    objs = {src: os.path.join(b.BUILD, os.path.splitext(src)[0] + ".o") for src in b.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        b.build(verbose=False, incremental=True)
    out = os.path.join(b.BUILD, "sanitized")
    os.makedirs(out, exist_ok=True)
    api_obj = os.path.join(out, "w4a16_api.o")
    exe = os.path.join(out, "abi_check")
    r = subprocess.run([hipcc, *b.common_flags(), "-O1", "-g", *SAN, "-c",
                        os.path.join(b.CSRC, "w4a16_api.hip"), "-o", api_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    check_obj = os.path.join(out, "abi_check.o")
    r = subprocess.run([hipcc, "-std=c++17", "-O1", "-g", *SAN, f"-I{os.path.join(ROOT, 'include')}",
                        "-c", os.path.join(ROOT, "tests", "abi_check.cpp"), "-o", check_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    c_obj = os.path.join(out, "abi_check_c.o")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    r = subprocess.run([cc, "-std=c11", "-O1", "-g", f"-I{os.path.join(ROOT, 'include')}", "-c",
                        os.path.join(ROOT, "tests", "abi_check_c.c"), "-o", c_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    others = [o for src, o in objs.items() if src != "w4a16_api.hip"]
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", *SAN, check_obj, c_obj, api_obj, *others, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all expectations held" in r.stdout
