"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the real
sources, built with the sanitizers on the host side only (the gfx950 device code is built as
usual), linked into a driver that exercises argument validation, launch planning over random
ragged, paged and extreme-length batches, the plan query with several CU counts, the
page-table check and the page pool. No GPU is used."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the library sources")
def test_host_code_is_clean_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        b = subprocess.run(["bash", os.path.join(HERE, "host_sanitize", "build.sh"), d], capture_output=True,
                           text=True, timeout=600)
        assert b.returncode == 0, b.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
                   HIP_VISIBLE_DEVICES="")
        r = subprocess.run([os.path.join(d, "drive")], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host sanitizer driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
