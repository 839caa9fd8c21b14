"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds made here in a temporary directory:
  - the library's host side (csrc/flint_moe.cpp: argument checks, workspace
    carving, path choice) with ASan + UBSan, linked with the already compiled
    kernel objects; the CPU tests of the C ABI run against it;
  - the C oracle with ASan + UBSan (gcc); the oracle pins run against it.
Each runs in a child process that preloads the matching sanitizer runtime;
any report (or a UBSan abort) fails the test.  The kernels themselves are
device code and are not instrumented.
"""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_moe_transformer_gemv_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# host-only sanitizer flags (each applies to the host pass only)
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-shared-libasan"]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run_child(script, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, "-c", script], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    text = p.stdout + p.stderr
    assert p.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    return text


def test_c_abi_host_code_under_asan_ubsan():
    rt = _clang_asan_runtime()
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.hip.o")))
    if rt is None or not objs or not os.path.exists(HIPCC):
        pytest.skip("needs hipcc, the clang ASan runtime and the built kernel objects")
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "flint_moe_san.o")
        so = os.path.join(tmp, "libflint_moe_san.so")
        subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", *SAN_HOST,
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                        "-c", os.path.join(PKG, "csrc", "flint_moe.cpp"), "-o", obj], check=True,
                       capture_output=True)
        subprocess.run([HIPCC, "-shared", "-fPIC", *SAN_HOST, "-o", so, obj, *objs], check=True,
                       capture_output=True)
        script = (
            "import sys; sys.path[:0] = [%r, %r]\n"
            "from sparse_moe_transformer_gemv_amd import flint_moe as b\n"
            "b.load_library(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
        ) % (ROOT, os.path.join(ROOT, "tests"), so, os.path.join(ROOT, "tests", "test_abi_cpu.py"))
        text = _run_child(script, rt)
        assert " passed" in text


def test_oracle_pins_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's ASan runtime is not installed")
    src = os.path.join(ROOT, "oracle", "moe_oracle.c")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", "-o", so, src, "-lm"], check=True, capture_output=True)
        script = (
            "import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle\n"
            "oracle._lib = oracle.load_library(%r)\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
        ) % (ROOT, os.path.join(ROOT, "tests"), so, os.path.join(ROOT, "tests", "test_oracle_pins.py"))
        text = _run_child(script, asan)
        assert " passed" in text
