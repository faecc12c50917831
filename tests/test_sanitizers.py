"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's validation, planning and pool code (swr_api.cpp and the host
side of the .hip files; device code is not instrumented) and the oracle are
rebuilt with both sanitizers, and the CPU tests that exercise them run again
in a child Python with the sanitizer runtime preloaded: test_abi.py and
test_pool.py against libswr_san.so, the oracle's pins against
liboracle_san.so.  Any report aborts the child and fails the test.  A
planted heap overflow in a copy of the oracle shows that the setup catches
what it should.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

ASAN_OPTIONS = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:abort_on_error=0"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"


def _env(preload, **extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=preload, ASAN_OPTIONS=ASAN_OPTIONS, UBSAN_OPTIONS=UBSAN_OPTIONS, OMP_NUM_THREADS="4",
               **extra)
    return env


def _pytest(files, env, timeout=600):
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *files]
    return subprocess.run(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                          timeout=timeout)


def test_library_host_code_under_asan_ubsan():
    if not shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc is not available")
    from sliding_window_ring_amd import build as swr_build

    lib = swr_build.build_sanitized()
    r = _pytest(["tests/test_abi.py", "tests/test_pool.py"],
                _env(swr_build.sanitizer_runtime(), SWR_SANITIZED_LIB=lib))
    assert r.returncode == 0, r.stdout[-6000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout


def test_oracle_pins_under_asan_ubsan():
    lib = oracle.build_sanitized()
    r = _pytest(["tests/test_oracle_formats.py", "tests/test_oracle_ring.py", "tests/test_oracle_attention.py",
                 "tests/test_golden.py"],
                _env(oracle.sanitizer_runtime(), ORACLE_SANITIZED_LIB=lib))
    assert r.returncode == 0, r.stdout[-6000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout


def test_sanitizers_catch_a_planted_overflow(tmp_path):
    # a copy of the oracle whose bf16 widening reads one element past its input
    src = open(os.path.join(ROOT, "oracle", "swr_oracle.c")).read()
    anchor = "void orc_bf16_value_n("
    assert anchor in src
    head, tail = src.split(anchor, 1)
    body_start = tail.index("{")
    planted = anchor + tail[:body_start + 1] + "\n  volatile uint16_t past = x[n]; (void)past;" + tail[body_start + 1:]
    variant = tmp_path / "swr_oracle.c"
    variant.write_text(head + planted)
    so = tmp_path / "liboracle_planted.so"
    subprocess.check_call(["gcc", *oracle._CFLAGS, *oracle._SAN_FLAGS, str(variant),
                           os.path.join(ROOT, "oracle", "swr_layout.c"), "-o", str(so), "-lm"])
    script = textwrap.dedent(f"""
        import ctypes, numpy as np
        lib = ctypes.CDLL({str(so)!r})
        x = np.zeros(4096, np.uint16)  # 8 KB: a malloc of its own, with a redzone right after it
        y = np.zeros(4096, np.float64)
        lib.orc_bf16_value_n(x.ctypes.data_as(ctypes.c_void_p), ctypes.c_int64(4096),
                             y.ctypes.data_as(ctypes.c_void_p))
        print("no report")
    """)
    r = subprocess.run([sys.executable, "-c", script], env=_env(oracle.sanitizer_runtime()), stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode != 0 and "AddressSanitizer" in r.stdout, r.stdout[-3000:]
