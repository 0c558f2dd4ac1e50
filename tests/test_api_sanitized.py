"""The library's host code (argument validation, launch set-up) under
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no device work).

Every HIP source is rebuilt with the sanitizers on the host pass only (each
-fsanitize= after -Xarch_host; the gfx950 code is built as usual but never
launched here) into a temporary directory, and the C-ABI suite (exports and
every argument check, which return before any launch) runs against that
build in a child process with clang's ASan runtime preloaded.  A sanitizer
report from the host code fails the test."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_speculative_verification_gdn_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_abi_suite_clean_under_host_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = str(tmp_path / (f[:-4] + ".o"))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c", os.path.join(CSRC, f),
                        "-o", obj], check=True, capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libgdntree_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *HOST_SAN[:4],
                    *objs, "-o", lib], check=True, capture_output=True)
    (tmp_path / "sanitized_library.py").write_text(
        "import os\nimport tree_speculative_verification_gdn_amd as g\n"
        "g.library_path = lambda: os.environ['GDN_LIB_SANITIZED']\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (asan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["GDN_LIB_SANITIZED"] = lib
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), ROOT])
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "--noconftest", "-p", "no:cacheprovider",
           "-p", "sanitized_library", os.path.join(ROOT, "tests", "test_abi.py")]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600, cwd=str(tmp_path))
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in log and " skipped" not in log, log[-4000:]
