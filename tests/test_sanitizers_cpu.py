"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/oracle.cpp) and the library's host layer (csrc/abi.cpp:
validation and dispatch) are rebuilt with -fsanitize=address,undefined
(tests/sanitize_build.py) and the CPU suites that drive them (every ABI status
path, every oracle pin) run again in a child process with the sanitizer
runtimes preloaded; any report fails the run. The device code is not
instrumented (GPU sanitizers are not used here).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi_cpu.py", "tests/test_oracle_pins.py", "tests/test_oracle_pins_masks.py",
          "tests/test_oracle_pins_fp8.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout
    return p.strip()


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    if not os.path.exists(os.path.join(ROOT, "_build", "bwd.hip.o")):
        pytest.skip("the regular build has not been run (no device objects in _build/)")
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import sanitize_build
    libs = sanitize_build.build(str(tmp_path_factory.mktemp("san")))
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               SDPA07_LIBRARY=libs["lib"], ORACLE_LIBRARY=libs["oracle"], PYTHONPATH=ROOT)
    return env


def test_sanitized_builds_are_the_ones_loaded(san_env):
    code = ("import oracle, scaled_dot_product_07_amd as s; oracle._load(); s._load(); "
            "print(open('/proc/self/maps').read())")
    r = subprocess.run([sys.executable, "-c", code], env=san_env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    for name in ("liboracle_san.so", "libsdpa07_san.so", "libasan.so", "libubsan.so"):
        assert name in r.stdout, f"{name} not mapped"


def test_cpu_suites_clean_under_sanitizers(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *SUITES], env=san_env, cwd=ROOT, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer"):
        assert marker not in out, out[-4000:]
