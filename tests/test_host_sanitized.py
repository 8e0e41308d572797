"""The host tests under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/test_host_lib.py (layout analysis, rotation tables, block maps, schedules, workspace sizes
and every argument check that must refuse a call before any launch) runs in a child process
against libqi_san.so, the library built with both sanitizers on its host code
(image_generation_qi_amd/build_sanitized.py), with the sanitizer runtime preloaded and the first
report fatal.  The library is rebuilt when a source is newer than it.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from image_generation_qi_amd import build as B  # noqa: E402


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(ROOT, "include", "qi.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


def test_host_tests_clean_under_sanitizers():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    from image_generation_qi_amd import build_sanitized as S
    if _stale(S.LIB_SAN):
        S.build_sanitized(jobs=min(8, os.cpu_count() or 4))
    env = S.sanitizer_env()
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_host_lib.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-p", "no:faulthandler"],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=900)
    reports = [l for l in r.stderr.splitlines() if "runtime error" in l or "AddressSanitizer" in l or "SUMMARY" in l]
    assert r.returncode == 0 and not reports, (r.returncode, r.stdout[-2000:], "\n".join(reports[:20]))
    assert " passed" in r.stdout
