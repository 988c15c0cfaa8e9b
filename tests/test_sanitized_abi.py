"""The CPU tests of the C ABI (tests/test_abi.py) run again against a build of
libpyr whose host code is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer: argument validation, geometry helpers and
workspace planning must make no out-of-bounds access, use no freed memory and
hit no undefined behaviour (signed overflow, bad shifts, misaligned loads) on
any of the valid and invalid problems those tests pass.  No device work is
enqueued: every call there validates or plans only."""

import os
import shutil
import subprocess
import sys

import pytest

from hierarchical_block_sparse_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def san_env():
    B.build_sanitized()
    return B.sanitizer_env()


def _run(args, env):
    return subprocess.run([sys.executable, *args], env=env, cwd=ROOT, capture_output=True,
                          text=True, timeout=900)


def test_sanitized_library_is_the_one_loaded(san_env):
    probe = ("import hierarchical_block_sparse_amd as H; H.lib();"
             "maps = open('/proc/self/maps').read();"
             "assert 'libclang_rt.asan' in maps, 'ASan runtime not loaded';"
             "assert '_build/san/libpyr.so' in maps, 'sanitized libpyr not loaded';"
             "print('ok')")
    r = _run(["-c", probe], san_env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_abi_tests_clean_under_asan_and_ubsan(san_env):
    r = _run(["-m", "pytest", "tests/test_abi.py", "-q", "-m", "not gpu",
              "-p", "no:cacheprovider"], san_env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout and " skipped" not in r.stdout.splitlines()[-1], r.stdout[-2000:]
