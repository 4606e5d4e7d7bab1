"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code,
gcc): a driver (tests/oracle_sanitize_main.c) runs prefill over ragged
sequences with a partial column block, decode into a slot cache, and the
argument checks, on heap buffers of exactly the documented sizes. A copy of the
oracle with an off-by-one output write shows that the run would catch one."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_C = os.path.join(HERE, "..", "oracle", "kda_oracle.c")
DRIVER_C = os.path.join(HERE, "oracle_sanitize_main.c")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
         "-fopenmp", "-std=c99"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _build_and_run(tmp_path, oracle_src):
    exe = str(tmp_path / "kda_oracle_sanitized")
    subprocess.check_call(["gcc", *FLAGS, "-o", exe, oracle_src, DRIVER_C, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    r = _build_and_run(tmp_path, ORACLE_C)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checksum" in r.stdout and "Sanitizer" not in r.stderr


def test_the_sanitized_run_catches_an_out_of_bounds_write(tmp_path):
    src = open(ORACLE_C).read()
    old = "o[bv + j0 + j] = scale * acc;"
    assert src.count(old) == 1
    bad = tmp_path / "kda_oracle_off_by_one.c"
    bad.write_text(src.replace(old, "o[bv + j0 + j + (t == t1 - 1 && h == H - 1 && j0 + j == V - 1)] = scale * acc;"))
    r = _build_and_run(tmp_path, str(bad))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
