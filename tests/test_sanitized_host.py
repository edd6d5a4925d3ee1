"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU):
the packer, the C ABI's argument validation and the oracle, built with both
sanitizers (w2_a8_matmul_amd/sanitize_build.py), run the packer, ABI and
oracle-pin test files in a child process that halts on the first report.  A
second child writes past a deliberately short host buffer through the ABI and
must be stopped by ASan, so a silently uninstrumented build cannot pass."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


@pytest.fixture(scope="module")
def san():
    from w2_a8_matmul_amd import sanitize_build as sb
    try:
        sb.asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    sb.build_sanitized()
    return sb


def test_host_tests_pass_under_sanitizers(san):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_packer.py", "tests/test_abi.py", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=san.sanitizer_env(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


CANARY = r"""
import sys, numpy as np
sys.path.insert(0, {root!r})
import oracle
from w2_a8_matmul_amd import _lib
oracle.quant_act(np.ones((1, 16), np.float32))
_lib.lib()
maps = open('/proc/self/maps').read()
assert {lib!r} in maps and {olib!r} in maps, 'sanitized libraries not loaded'
print('LOADED', flush=True)
W = np.ones((6, 16), np.float32)
C = np.ones((32, 3), np.uint8)
scales = np.empty((6,), np.uint16)
packed = np.empty((1, 16), np.uint8)   # two triples need two rows
_lib.call('s3d8_encode', W.ctypes.data, 6, 16, C.ctypes.data, 1, scales.ctypes.data, packed.ctypes.data)
print('NOT CAUGHT', flush=True)
"""


def test_sanitizer_catches_a_host_overflow(san):
    code = CANARY.format(root=ROOT, lib=san.SAN_LIB, olib=san.SAN_ORACLE)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san.sanitizer_env(), capture_output=True,
                       text=True, timeout=300)
    assert "LOADED" in r.stdout, r.stderr[-2000:]
    assert "NOT CAUGHT" not in r.stdout
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
