"""The CPU tier under AddressSanitizer and UndefinedBehaviorSanitizer.

Two host builds, each in a temporary directory, each exercised in a child
interpreter with its sanitizer runtime preloaded (Python itself is not
instrumented):

  * the fp64 oracle (oracle/gdn_oracle.c) built with gcc, running the oracle
    pins and the solve study;
  * libgdn.so built with hipcc, sanitizers on the host pass only (the device
    code is built as usual and never runs here), running the C-ABI argument
    checks of test_abi_cpu.py (every call there is refused on the host).

A sanitizer report or a failing test fails the run.  No GPU is used.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
ORACLE = os.path.join(ROOT, "oracle")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(compiler, name):
    if not shutil.which(compiler) and not os.path.exists(compiler):
        return None
    r = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(code, preload, lib):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "ERROR: AddressSanitizer" not in out
    assert "runtime error:" not in out
    assert r.returncode == 0
    assert f"mapped {lib}" in out


MAPPED = ("import os\n"
          "maps = open('/proc/self/maps').read()\n"
          "assert LIB in maps, 'the instrumented library is not loaded'\n"
          "print('mapped', LIB)\n")


def test_oracle_under_asan_ubsan(tmp_path):
    asan = _runtime("gcc", "libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", ORACLE,
                    os.path.join(ORACLE, "gdn_oracle.c"), "-o", lib, "-lm"], check=True)
    code = (f"import sys, ctypes\nsys.path[:0] = [{ROOT!r}, {TESTS!r}]\nLIB = {lib!r}\n"
            "import oracle\n"
            "oracle._lib = oracle._declare(ctypes.CDLL(LIB))\n"
            "oracle._lib_path = LIB\n"
            + MAPPED +
            "import pytest\n"
            f"rc = pytest.main([{os.path.join(TESTS, 'test_oracle_pins.py')!r}, "
            f"{os.path.join(TESTS, 'test_solve_study.py')!r}, '-q', '-x', '-p', 'no:cacheprovider'])\n"
            "assert oracle._lib._name == LIB\n"
            "sys.exit(int(rc))\n")
    _run_child(code, asan, lib)


def test_library_host_checks_under_asan_ubsan(tmp_path):
    asan = _runtime(CLANG, "libclang_rt.asan-x86_64.so")
    if asan is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from linear_attention_recurrence_04_amd import build as gbuild
    lib = str(tmp_path / "libgdn_san.so")
    flags = [f for f in gbuild.FLAGS if f != "-O3"]
    san = ["-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = ([HIPCC, "-O1", "-g"] + flags + san
           + ["-I", gbuild.INCLUDE, "-I", gbuild.CSRC] + gbuild.sources() + ["-o", lib])
    subprocess.run(cmd, check=True, capture_output=True)
    code = (f"import sys, ctypes\nsys.path[:0] = [{ROOT!r}, {TESTS!r}]\nLIB = {lib!r}\n"
            "from linear_attention_recurrence_04_amd import binding as B\n"
            "B.LIBRARY = LIB\n"
            "B._lib = B._declare(ctypes.CDLL(LIB))\n"
            + MAPPED +
            "import pytest\n"
            f"rc = pytest.main([{os.path.join(TESTS, 'test_abi_cpu.py')!r}, '-q', '-x', "
            "'-p', 'no:cacheprovider', '-k', 'not python_binding'])\n"
            "sys.exit(int(rc))\n")
    _run_child(code, asan, lib)
