"""Host code under address and undefined-behaviour sanitizers (CPU only).

The C ABI's host side (argument checks, workspace carving, the device
scratch lookup's error paths) is rebuilt with ASan and UBSan on its host pass
and the ABI checks of test_abi_cpu.py run against it; the C oracle is rebuilt
under gcc's ASan and UBSan and its pins (forward and reverse mode) run against
it. Each suite runs in a child process with the sanitizer runtime preloaded;
any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehaviorSanitizer")


def _run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *args], cwd=ROOT, env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=900)
    found = [r for r in REPORTS if r in res.stdout]
    assert res.returncode == 0 and not found, res.stdout[-4000:]
    return res.stdout


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from bilinear_rnn_amd import build
    rt = build.sanitizer_runtime()
    if not rt:
        pytest.skip("no ASan runtime for the HIP compiler")
    lib = build.build_sanitized(str(tmp_path))
    out = _run({"LD_PRELOAD": rt, "COMBA_LIBRARY": lib}, ["tests/test_abi_cpu.py"])
    assert " passed" in out


def test_c_oracle_under_asan_and_ubsan(tmp_path):
    import oracle
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], stdout=subprocess.PIPE, text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.isabs(ubsan)):
        pytest.skip("no gcc sanitizer runtimes")
    lib = oracle.build_c_sanitized(str(tmp_path / "liboracle_san.so"))
    out = _run({"LD_PRELOAD": f"{asan} {ubsan}", "COMBA_ORACLE_LIBRARY": lib},
               ["tests/test_oracle_pins.py", "-k", "c] or c_backward or c_and_numpy or parity_measures"])
    assert " passed" in out
