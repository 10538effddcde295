"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
liboracle is rebuilt from the same source with both sanitizers (aborting on
the first report), and the oracle's own CPU test files run against that
build in a child process.  Any out-of-bounds access, use after free, signed
overflow or misaligned access in the oracle fails the run (leak checking is
left off: the interpreter's own libraries hold blocks until exit)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bkv_oracle.c")
ORACLE_TESTS = ["test_oracle_fps.py", "test_oracle_fps_full.py", "test_oracle_rope_bf16.py",
                "test_oracle_score_select.py", "test_oracle_fill.py", "test_oracle_policies.py",
                "test_oracle_decode.py", "test_golden_pages.py", "test_checkpoint_resume.py"]


def runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_oracle_suite_clean_under_asan_and_ubsan(tmp_path):
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(lib), SRC, "-lm"])
    env = dict(os.environ)
    # leak checking is off: the interpreter and its libraries keep blocks until exit
    env.update(BKV_ORACLE_LIB=str(lib), LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    args = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    args += [os.path.join(ROOT, "tests", t) for t in ORACLE_TESTS]
    r = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=550)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    print(r.stdout.strip().splitlines()[-1])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_the_sanitized_build_catches_an_out_of_bounds_read(tmp_path):
    """Control: the same flags and preload catch a planted heap overflow, so
    a clean run above means something."""
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = tmp_path / "oob.c"
    src.write_text("#include <stdlib.h>\n"
                   "double oob(int n) { double *a = malloc(sizeof(double) * n); double s = 0;\n"
                   "  for (int i = 0; i <= n; ++i) s += a[i]; free(a); return s; }\n")
    lib = tmp_path / "liboob.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(lib), str(src)])
    code = "import ctypes; l = ctypes.CDLL(%r); l.oob.restype = ctypes.c_double; l.oob(8)" % str(lib)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
