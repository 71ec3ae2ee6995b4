"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/native/oracle_sanitized.c calls every oracle entry point on small inputs held in
buffers of their exact extent (odd widths, strides above the row length, empty, single and
long bags, negative and oversize indices under hashing) and takes each error path once;
built with gcc's sanitizers, any out-of-bounds access, leak or undefined operation in the
oracle ends the program with a report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_runs_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    src = os.path.join(HERE, "native", "oracle_sanitized.c")
    subprocess.run(["gcc", "-O1", "-g", "-std=gnu11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-o", exe, src, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
