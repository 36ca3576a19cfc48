"""Host-side sanitizer runs (CPU only): the oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer running every pin, and the C ABI's argument validation (the host
code of the library, built with the same sanitizers) running every validation test.  The
bitone README's "Security" list asks for null, bounds and size checks on every input of the
native bridge; these runs show the checks themselves read nothing out of bounds and do no
undefined arithmetic (size products, shifts, signed overflow) on hostile sizes.

Each run is a subprocess with the sanitizer runtime preloaded (ASan must come first);
leak checking is off (the interpreter and the HIP runtime keep allocations to the end)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(script, preload, timeout):
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allow_user_segv_handler=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONPATH=f"{ROOT}:{TESTS}")
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    assert r.returncode == 0, (r.returncode, r.stdout[-3000:], r.stderr[-6000:])
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(output=str(tmp_path / "liboracle_san.so"), extra_flags=SAN)
    out = _run(f"""
import oracle, pins
orc = oracle.Oracle({lib!r})
for pin in pins.PINS:
    pin(orc)
print("pins", len(pins.PINS))
""", asan, 900)
    assert "pins" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    from bit_gemm_02_amd import build as hip_build
    asan = _runtime([hip_build.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"])
    if asan is None or not os.path.exists(hip_build.HIPCC):
        pytest.skip("hipcc's AddressSanitizer runtime is not installed")
    host = [f for flag in SAN for f in ("-Xarch_host", flag)]
    lib = hip_build.build(output=str(tmp_path / "libbitlinear_san.so"), extra_flags=host,
                          extra_link_flags=host)
    out = _run(f"""
import sys, pytest
import bit_gemm_02_amd as bl
bl.LIBRARY = {lib!r}
rc = pytest.main(["-q", "-p", "no:cacheprovider", {os.path.join(TESTS, "test_abi.py")!r}])
print("pytest exit", int(rc))
sys.exit(int(rc))
""", asan, 900)
    assert "pytest exit 0" in out
