"""The host code under AddressSanitizer (CPU).

libmt_asan.so is the library with every source's host code instrumented
(device code as usual).  Each check runs in a child process with clang's
sanitizer runtime preloaded and the package pointed at that build:

* a canary: the host Adam handed a moment buffer shorter than `n` must be
  reported by the sanitizer, from inside the library (the build is
  instrumented and the runtime active);
* the host-code tests: store layout, configuration checks, the schedule and
  its hazard proof, the host Adam, the API's error paths; every one must
  pass with no sanitizer report.
"""
import os
import subprocess
import sys

import pytest

from host_memory_layer_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_env():
    if not os.path.exists(B.ASAN_LIB):
        B.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), MT_LIBRARY=B.ASAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    return env


CANARY = r"""
import ctypes, numpy as np
import host_memory_layer_amd as mt
assert mt.LIB_PATH.endswith("libmt_asan.so"), mt.LIB_PATH
n = 4096
w, g, v = (np.ones(n, np.float32) for _ in range(3))
m = np.zeros(n - 16, np.float32)  # 16 elements short
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
print("calling", flush=True)
mt.lib().mt_host_adam(mt.MT_F32, p(w), p(g), p(m), p(v), n, 1, 1e-3, 0.9, 0.95, 1e-8, 1)
print("returned", flush=True)
"""


def test_sanitizer_catches_an_overrun_inside_the_library(asan_env):
    r = subprocess.run([sys.executable, "-c", CANARY], cwd=ROOT, env=asan_env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode != 0, r.stdout[-2000:]
    assert "calling" in r.stdout and "returned" not in r.stdout
    assert "AddressSanitizer: heap-buffer-overflow" in r.stdout, r.stdout[-2000:]
    assert "libmt_asan.so" in r.stdout


def test_host_code_tests_pass_under_the_sanitizer(asan_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_library.py", "tests/test_schedule.py"],
                       cwd=ROOT, env=asan_env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=900)
    print(r.stdout[-1500:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "AddressSanitizer" not in r.stdout
    assert " passed" in r.stdout
