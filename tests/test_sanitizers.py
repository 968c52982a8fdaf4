"""CPU sanitizer job: the oracle and the library's host code (argument
validation, workspace sizing, status strings, the check switch) built with
AddressSanitizer + UndefinedBehaviorSanitizer, and the CPU tests that drive
them run against those builds in child processes (each with its compiler's
sanitizer runtime preloaded).  Any sanitizer report fails the test.  The
device code is built as usual; nothing here needs a GPU."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(tests, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    bad = [l for l in out.splitlines()
           if "runtime error" in l or "AddressSanitizer" in l or "SUMMARY:" in l]
    assert r.returncode == 0 and not bad, "\n".join(bad) or out[-3000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    rt = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    _run(["tests/test_oracle_pins.py", "tests/test_numerics_probe.py"],
         {"PSAMP_ORACLE_LIB": lib, "LD_PRELOAD": rt})


def test_host_code_under_asan_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    from proportional_sampling_amd import build as B
    lib = B.build(verbose=False, sanitize_host=True, out=str(tmp_path / "libpsamp_san.so"))
    _run(["tests/test_abi.py"], {"PSAMP_LIB": lib, "LD_PRELOAD": rts[-1]})
