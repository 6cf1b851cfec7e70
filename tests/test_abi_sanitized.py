"""The CPU-only ABI tests again, against a build whose host code (argument validation, launch
planning, workspace sizing) runs under AddressSanitizer and UndefinedBehaviorSanitizer.  The
sanitized library is built into _build/sanitized/ and loaded in a child process with the
sanitizer runtime preloaded; any report fails the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc is needed to build the sanitized library")

_CHECK_LOADED = (
    "import decodability_aware_token_amd.binding as F; F.lib(); "
    "maps = open('/proc/self/maps').read(); "
    "assert F.LIB_PATH in maps, 'sanitized library not loaded'; "
    "assert 'libclang_rt.asan' in maps, 'sanitizer runtime not loaded'; "
    "print('loaded', F.LIB_PATH)"
)


def test_abi_under_address_and_undefined_sanitizers():
    from decodability_aware_token_amd import build as B
    lib = B.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": B.sanitizer_runtime(),
        "FOCUS_LIBRARY": lib,
        # Python itself keeps allocations alive at exit; leaks are not what this checks
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87",
    })
    for cmd in ([sys.executable, "-c", _CHECK_LOADED],
                [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                 os.path.join(ROOT, "tests", "test_abi.py")]):
        res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                             timeout=600)
        out = res.stdout + res.stderr
        assert res.returncode == 0, out[-4000:]
        assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
