"""The host-side C ABI code (abi.hip) built with AddressSanitizer and run
against stub kernel launchers (tests/asan/abi_host_asan.cpp): argument
validation before any launch, exactly one launch for valid arguments, and no
out-of-bounds host access on valid, invalid or corrupted layouts.  Host code
only: no GPU, no device code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return h if os.path.exists(h) else None


def test_abi_host_code_under_address_sanitizer(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_host_asan")
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "--cuda-host-only", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           f"-I{ROOT}/include", f"-I{ROOT}/tile_sparse_attention_head_amd/csrc",
           "-x", "hip", f"{ROOT}/tile_sparse_attention_head_amd/csrc/abi.hip",
           f"{ROOT}/tests/asan/abi_host_asan.cpp", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    env.pop("VEDA_DEBUG_SYNC", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ALL OK" in r.stdout
    assert "AddressSanitizer" not in r.stderr
