"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's sources are compiled with hipcc, the sanitizers applied to their host code
only, and linked with tests/native/abi_sanitized.cpp, which calls every entry point with
arguments the checks must refuse and the pure size queries over ordinary and extreme sizes.
No GPU is touched: every call stops at its checks.  (This test found an out-of-range enum
value reaching the library's C++ when a caller passed an unknown dtype code, and signed
overflows in the workspace-size queries near 2^31.)"""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_checks_run_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "embedding_lookup_feature_amd", "csrc")]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN + inc
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(ROOT, "embedding_lookup_feature_amd", "csrc", "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *common, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    drv = str(tmp_path / "drv.o")
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17"] + SAN + inc +
                   ["-c", os.path.join(HERE, "native", "abi_sanitized.cpp"), "-o", drv], check=True)
    exe = str(tmp_path / "abi_sanitized")
    subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + [*objs, drv, "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime's own allocations
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-3000:]
