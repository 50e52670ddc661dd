"""Host-side sanitizer runs (CPU only; no GPU code is instrumented).

* The oracle built with AddressSanitizer + UndefinedBehaviorSanitizer (gcc)
  runs every oracle pin; a planted mistake (an output buffer one row short)
  must be reported, so the instrumentation is known to be active.
* libw8a8.so built with the host half of every translation unit under
  AddressSanitizer + UndefinedBehaviorSanitizer (clang, -Xarch_host: the
  gfx950 code objects are built as usual) runs the C ABI's CPU tests, which
  drive every argument check and error code.

Each run is a child process with the sanitizer runtime preloaded.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")


def _runtime(cmd):
    try:
        path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _child(code, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1",
               **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


@pytest.fixture(scope="module")
def gcc_san():
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    ubsan = _runtime(["gcc", "-print-file-name=libubsan.so"])
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    import oracle
    os.makedirs(SAN_DIR, exist_ok=True)
    lib = oracle.oracle.build_oracle_sanitized(os.path.join(SAN_DIR, "liboracle_san.so"))
    return {"LD_PRELOAD": f"{asan}:{ubsan}", "W8A8_ORACLE_LIB": lib}


def test_oracle_pins_under_asan_ubsan(gcc_san):
    code = ("import sys, pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_pins.py']))")
    r = _child(code, gcc_san)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


def test_sanitized_oracle_catches_a_planted_overrun(gcc_san):
    """The int GEMM writes into an output buffer one row short: AddressSanitizer must stop
    the process with a heap-buffer-overflow report."""
    code = (
        "import ctypes, numpy as np, oracle\n"
        "lib = oracle.load_oracle()\n"
        "assert 'liboracle_san' in open('/proc/self/maps').read()\n"
        "M, N, K = 8, 16, 32\n"
        "x = np.ones((M, K), np.int8); w = np.ones((N, K), np.int8)\n"
        "out = np.zeros(((M - 1) * N,), np.int32)\n"
        "lib.oracle_gemm_i32(x.ctypes.data, w.ctypes.data, M, N, K, out.ctypes.data)\n"
        "print('no report')\n")
    r = _child(code, gcc_san)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]


@pytest.fixture(scope="module")
def clang_san_lib():
    from quantized_gemm_quantize_amd import build
    rt = _runtime([build.HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"])
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not installed")
    return rt, build.build_host_sanitized(os.path.join(SAN_DIR, "libw8a8_san.so"))


def test_abi_checks_under_asan_ubsan(clang_san_lib):
    rt, lib = clang_san_lib
    code = ("import sys, pytest\n"
            "from quantized_gemm_quantize_amd import binding\n"
            f"binding.LIB_PATH = {lib!r}\n"
            "binding.load()\n"
            "assert 'libw8a8_san' in open('/proc/self/maps').read()\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))\n")
    r = _child(code, {"LD_PRELOAD": rt})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
