"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The C oracle, rebuilt with gcc's ASan + UBSan (every UB check fatal), runs
  the oracle's pin tests in a child process that preloads gcc's runtime.
* The C ABI's host code (argument checks, overlap and alignment logic, error
  strings), rebuilt with clang's ASan + UBSan for the host pass only and
  linked with the library's other objects, runs the ABI's CPU tests in a
  child process that preloads clang's runtime (no kernel is launched there).

Both children must exit cleanly; a sanitizer report ends them with a
non-zero status.  Built objects go to the package's _build/ directory."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_attention_recurrence_09_amd")
BUILD = os.path.join(PKG, "_build", "sanitize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")
CLANG_RT = "/opt/rocm/llvm/lib/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT)
    return r.returncode, r.stdout + r.stderr


def _clang_asan_runtime():
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_oracle_pins_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    lib = os.path.join(BUILD, "liboracle_san.so")
    rc, out = _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", ORACLE_SRC, "-o", lib, "-lm"])
    assert rc == 0, out
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True).stdout.strip()
    code = ("import sys, pytest; sys.path.insert(0, %r); import oracle.build as b; "
            "b.ensure_built = lambda: %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            "'tests/test_oracle_recurrence.py', 'tests/test_oracle_conv_norm.py', "
            "'tests/test_oracle_layer.py', 'tests/test_oracle_mutations.py']))" % (ROOT, lib))
    rc, out = _run([sys.executable, "-c", code], env=dict(ENV, LD_PRELOAD=rt))
    assert rc == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_abi_host_checks_under_asan_ubsan():
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    from linear_attention_recurrence_09_amd import build as kb
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in kb.SOURCES:
        obj = os.path.join(kb.OBJ_DIR, os.path.splitext(src)[0] + ".o")
        if src == "kda_api.cpp" or not os.path.exists(obj):
            if src == "kda_api.cpp":
                obj = os.path.join(BUILD, "kda_api_san.o")
                flags = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                         "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                         "-Xarch_host", "-fno-omit-frame-pointer"]
            else:
                flags = ["-O3"]
            rc, out = _run([kb.HIPCC, f"--offload-arch={kb.ARCH}", "-fPIC", "-std=c++17",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            f"-I{kb.INCLUDE}", f"-I{kb.CSRC}", *flags, "-x", "hip", "-c",
                            os.path.join(kb.CSRC, src), "-o", obj])
            assert rc == 0, out
        objs.append(obj)
    lib = os.path.join(BUILD, "libkda_san.so")
    rc, out = _run([kb.HIPCC, f"--offload-arch={kb.ARCH}", "-shared", "-fPIC", *objs, "-o", lib])
    assert rc == 0, out
    code = ("import sys, pytest; sys.path.insert(0, %r); "
            "import linear_attention_recurrence_09_amd as k; k.LIB_PATH = %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            "'tests/test_abi_cpu.py']))" % (ROOT, lib))
    rc, out = _run([sys.executable, "-c", code], env=dict(ENV, LD_PRELOAD=rt))
    assert rc == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "passed" in out, out[-2000:]
