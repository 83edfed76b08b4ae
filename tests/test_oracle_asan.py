"""The oracle's pins and its composition pin, run once more against a copy of
oracle.c built with the host compiler's AddressSanitizer (in a child process
that preloads libasan).  Any out-of-bounds access, use after free or double
free in the oracle ends that process with an ASan report and fails this test.
Host code only: nothing here touches a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_pins_run_clean_under_address_sanitizer(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not available")
    env = dict(os.environ, ORACLE_LIB_DIR=str(tmp_path), ORACLE_SANITIZE="address", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1", OMP_NUM_THREADS="4")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_torch_ref.py"),
           "-k", "not spread_between_oracle_precisions"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert os.path.exists(tmp_path / "liboracle32.so") and os.path.exists(tmp_path / "liboracle64.so"), tail
    assert "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert r.returncode == 0, tail
