"""The host block manager under AddressSanitizer and UndefinedBehaviorSanitizer:
random add (with repeated prompts for prefix hits) / append (with copy-on-write
after fork) / fork / free sequences on pools of 8-127 blocks of 16-256 tokens,
checking after every operation that table entries, slots, reference counts and
the free count agree. Builds block_manager.cpp with the host compiler."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_fuzz_sanitized(tmp_path):
    exe = tmp_path / "bm_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-D__HIP_PLATFORM_AMD__", os.path.join(HERE, "block_manager_fuzz.cpp"),
           os.path.join(ROOT, "paged_kv_cache_store_amd", "csrc", "block_manager.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the sanitizer runtime need not be first among the loaded libraries
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-2000:]
