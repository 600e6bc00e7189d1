"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

capi.cpp -- argument validation, workspace carving, KV-region checks, the pinned stage's host side,
the several-sequence staging tables -- is compiled with the sanitizers on its host code (each
-fsanitize after -Xarch_host: the GPU code is built as usual), linked with the other objects into
a test copy of the library, and the host-side C-ABI tests run against that copy in a child process
with the sanitizer runtime preloaded.  Any out-of-bounds access, use after free or undefined
behaviour on those paths aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from quantized_transformer_prefill_amd import build as B  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    r = subprocess.run([B.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_checks_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    objs = []
    for src in B.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        cmd = [B.HIPCC, *B.FLAGS]
        if src.endswith(".cpp"):  # the host code under test: sanitized
            cmd += [*SAN, "-x", "hip"]
        else:
            prebuilt = os.path.join(B.BUILD_DIR, os.path.splitext(src)[0] + ".o")
            if os.path.exists(prebuilt) and os.path.getmtime(prebuilt) >= os.path.getmtime(os.path.join(B.CSRC, src)):
                objs.append(prebuilt)
                continue
        r = subprocess.run(cmd + ["-c", os.path.join(B.CSRC, src), "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(tmp_path / "libmi_prefill_sanitized.so")
    r = subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *SAN, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, "the test library is not instrumented"
    env = dict(os.environ, MI_PREFILL_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_capi_host.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    print(p.stdout[-2000:])
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr[-3000:]
