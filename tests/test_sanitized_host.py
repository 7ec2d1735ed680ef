"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (host code instrumented, device code as usual):
the CPU tests of the C ABI (argument checks, list validation, the mask bank
writer and reader including crafted files, the calibration driver's rules,
the property tests) run in a child process against libcalibatt_asan.so with
the sanitizer runtime preloaded, and the plain C consumer is linked against
it. Any report fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_bank_host.py", "tests/test_calibrate_host.py",
              "tests/test_properties.py"]


@pytest.fixture(scope="module")
def asan_build():
    from calibrated_block_sparse_amd import build as b
    try:
        rt = b.asan_runtime()
        lib = b.build(sanitize=True)
    except RuntimeError as e:  # pragma: no cover - toolchain without the runtime
        pytest.skip(f"sanitized build unavailable: {e}")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, CALIBATT_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    return lib, env


def _no_reports(text: str):
    assert "ERROR: AddressSanitizer" not in text, text[-4000:]
    assert "runtime error:" not in text, text[-4000:]


def test_host_tests_under_sanitizers(asan_build):
    lib, env = asan_build
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *HOST_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    _no_reports(out)
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout


def test_sanitized_library_is_the_one_loaded(asan_build):
    lib, env = asan_build
    code = ("import calibrated_block_sparse_amd as c; l = c.load_library(); "
            "print(l._name)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == lib


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_consumer_under_sanitizers(asan_build, tmp_path):
    lib, env = asan_build
    exe = str(tmp_path / "consumer")
    link_dir = str(tmp_path)
    os.symlink(lib, os.path.join(link_dir, "libcalibatt.so"))
    rt_dir = os.path.dirname(env["LD_PRELOAD"])
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_consumer", "consumer.c"), "-o", exe,
           "-L", link_dir, "-lcalibatt", f"-Wl,-rpath,{link_dir}",
           "-L", rt_dir, "-l:libclang_rt.asan-x86_64.so", f"-Wl,-rpath,{rt_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, str(tmp_path / "bank.cbsm")], env=env, capture_output=True, text=True,
                       timeout=300)
    _no_reports(r.stdout + r.stderr)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip() == "ok"
