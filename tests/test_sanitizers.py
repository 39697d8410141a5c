"""The generator and the oracle under host sanitizers (CPU only).

tests/sanitize_driver.c calls every exported function of gen/maxsim_gen.c and
oracle/maxsim_oracle.c on small inputs with their edge cases (empty and one-token
documents, masks, ragged CSR, several threads, optional outputs). It is built twice
with gcc -- AddressSanitizer + UndefinedBehaviorSanitizer (with leak checks), then
ThreadSanitizer for the threads that split the documents -- and run as a child
process; any report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "sanitize_driver.c"),
           os.path.join(ROOT, "gen", "maxsim_gen.c"),
           os.path.join(ROOT, "oracle", "maxsim_oracle.c")]
BASE = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall"]

SANITIZERS = {
    "address,undefined": {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=23",
                          "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"},
    "thread": {"TSAN_OPTIONS": "halt_on_error=1:exitcode=24"},
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("san", sorted(SANITIZERS))
def test_generator_and_oracle_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / ("driver_" + san.replace(",", "_")))
    build = subprocess.run(["gcc", *BASE, f"-fsanitize={san}", "-fno-sanitize-recover=all",
                            "-o", exe, *SOURCES, "-lm", "-lpthread"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in build.stderr and "not supported" in build.stderr:
        pytest.skip(f"gcc cannot build -fsanitize={san} here")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, **SANITIZERS[san])
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if run.returncode != 0 and "does not work under ptrace" in run.stderr:
        pytest.skip("the sanitizer runtime cannot run under this process tracer")
    assert run.returncode == 0 and "sanitize driver: ok" in run.stdout, run.stdout + run.stderr
