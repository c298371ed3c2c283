"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no GPU).

Builds csrc/moe_ep.hip with the sanitizers on the host side only (each -fsanitize= follows
-Xarch_host, so the device code is the ordinary build's) and tests/abi_host_checks.c with ROCm's
clang and the same sanitizers, then runs the client: every argument check of every entry point,
the size helpers on extreme shapes and the calls with nothing to launch must finish without a
sanitizer report.  Nothing here launches a kernel.
"""
import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_moe_ep_build_san", os.path.join(ROOT, "combine_get_dispatch_07_amd",
                                                                                     "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


@pytest.fixture(scope="module")
def sanitized_client(tmp_path_factory):
    b = _build_module()
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not available")
    d = str(tmp_path_factory.mktemp("asan"))
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = os.path.join(d, "libmoe_ep.so")
    cmd = [hipcc, *b.HIPCC_FLAGS, "-O1", "-g", *host_san, f"-I{b.INCLUDE}", b.SRC, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    client = os.path.join(d, "abi_host_checks")
    cmd = [clang, "-std=c11", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           f"-I{b.INCLUDE}", f"-I{rocm}/include", os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", client,
           f"-L{d}", "-lmoe_ep", f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{d}", f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return client


def test_host_checks_under_sanitizers(sanitized_client):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sanitized_client], capture_output=True, text=True, timeout=300, env=env)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert "host checks: all passed" in r.stdout
