"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

gdn_oracle.c is rebuilt with gcc -fsanitize=address,undefined into a
temporary directory, and the oracle's pin, brute-force, error-path and
golden suites run against that build in a child process with the ASan
runtime preloaded (CPython itself is not instrumented; leak checking is off
because the interpreter keeps its own allocations to exit).  Any heap or
stack overflow, use after free, signed overflow, bad shift or misaligned
access in the oracle stops the child with the sanitizer's report, and the
test fails with it.  The malformed trees, paths and slots of the error-path
suite are the inputs most likely to reach an out-of-range index."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
SUITES = ["test_oracle_pins.py", "test_oracle_bruteforce.py", "test_oracle_errors.py",
          "test_oracle_golden.py"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_suites_clean_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libgdn_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-DORA_MUTATION=0", SRC, "-o", lib, "-lm"], check=True)
    plugin = tmp_path / "sanitized_oracle.py"
    plugin.write_text("import os\nimport oracle\n"
                      "oracle._lib = oracle.load(os.environ['GDN_ORACLE_SANITIZED_LIB'])\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (asan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["GDN_ORACLE_SANITIZED_LIB"] = lib
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), os.path.join(ROOT, "tests"), ROOT])
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "--noconftest", "-p", "no:cacheprovider",
           "-p", "sanitized_oracle"] + [os.path.join(ROOT, "tests", s) for s in SUITES]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=str(tmp_path))
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in log, log[-4000:]
