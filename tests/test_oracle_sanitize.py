"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every routine of
nm_oracle.c runs over small ragged shapes with buffers of exactly the size its caller
contract gives (oracle/sanitize_check.c), plus the pack/unpack, slide/fold and bitmap
round trips.  CPU only."""
import subprocess

import oracle as O


def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = O.build_sanitize_check(tmp_path / "sanitize_check")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitize check ok" in r.stdout
