"""CPU sanitizer runs: the oracle (plain C) built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc) and the library's host code (argument checks,
workspace sizing, plan building, tiling metadata, the C ABI) built with the
same sanitizers (clang, host side only), each run under the CPU tests that
exercise it.  Any sanitizer report, or a test failure under the sanitizers,
fails this test.  No GPU is used: the library's calls in these tests return
before anything is enqueued.  The exhaustive 2^32 cast sweep is left out (85 s
under ASan); the rest of the oracle's pins run in full."""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TESTS = ["tests/test_oracle_cast.py", "tests/test_oracle_patch.py", "tests/test_oracle_lz4.py",
                "tests/test_oracle_fp8.py", "tests/test_oracle_next.py", "tests/test_fullsize_checker.py"]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior")


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(env_extra, tests, deselect=()):
    env = dict(os.environ)
    env.update(env_extra)
    env.update({"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    for d in deselect:
        cmd += ["--deselect", d]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    build = _load("_oracle_build_san", os.path.join(ROOT, "oracle", "_build.py"))
    lib = build.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    out = _run({"LD_PRELOAD": libasan, "SDC_ORACLE_LIB": lib}, ORACLE_TESTS,
               deselect=["tests/test_oracle_cast.py::test_full_sweep_matches_torch"])
    assert " passed" in out


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    build = _load("_pulse_build_san", os.path.join(ROOT, "sparse_delta_codec_amd", "_build.py"))
    lib = build.build_host_sanitized(str(tmp_path / "pulse"))
    out = _run({"LD_PRELOAD": rts[-1], "SDC_PULSE_LIB": lib}, ["tests/test_abi.py"])
    assert " passed" in out
