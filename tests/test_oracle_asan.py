"""The oracle's CPU pin tests again, with the oracle built under AddressSanitizer, so that any
out-of-bounds access in the oracle fails loudly instead of corrupting the host heap (CPU only)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_libasan() is None, reason="gcc has no AddressSanitizer runtime here")
def test_oracle_suite_under_asan(tmp_path):
    import oracle

    lib = tmp_path / "libpkv_oracle_asan.so"
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fsanitize=address",
                                                        "-fno-omit-frame-pointer"]
    subprocess.run(["gcc", *flags, oracle._SRC, "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ)
    env["PKV_ORACLE_LIB"] = str(lib)
    env["LD_PRELOAD"] = _libasan()
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    tests = ["tests/test_oracle_store.py", "tests/test_oracle_dequant.py", "tests/test_oracle_decode.py",
             "tests/test_oracle_mla.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
