"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, gcc): oracle/sanitize_check.c links oracle/la_oracle.c and runs a
prefill against step-by-step decode (bitwise), lambda = 0 and lambda = 1
heads, an empty sequence and rejected arguments; any out-of-bounds access,
leak or undefined operation aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "sanitize_check")
    flags = ["-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    r = subprocess.run([gcc, *flags, "-o", exe, os.path.join(ORACLE, "la_oracle.c"),
                        os.path.join(ORACLE, "sanitize_check.c"), "-lm"],
                       capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr):
        pytest.skip("this gcc has no sanitizer runtime: " + r.stderr.strip()[:200])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout


def test_the_sanitizer_flags_catch_a_planted_overflow(tmp_path):
    # the same flags on a program with a one-past-the-end heap write must abort:
    # the check above is not vacuous
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile int *p = malloc(4 * sizeof(int));"
                   " p[4] = 1; free((void *)p); return 0; }\n")
    exe = str(tmp_path / "overflow")
    r = subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-o", exe, str(src)], capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr):
        pytest.skip("this gcc has no sanitizer runtime")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:verify_asan_link_order=0")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode != 0 and "heap-buffer-overflow" in run.stderr
