"""The host C++ of libpa (allocator, prefix cache, block tables) under
AddressSanitizer and UndefinedBehaviorSanitizer (no GPU; g++ only, no HIP).

tests/native/allocator_stress.cpp runs random operation sequences and
checks the exported state after each one; this test builds it with the
sanitizers against the plain C++ source and runs it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = shutil.which("g++")


@pytest.mark.skipif(GXX is None, reason="needs g++")
def test_allocator_and_prefix_cache_under_sanitizers(tmp_path):
    exe = tmp_path / "allocator_stress"
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{ROOT}/include", f"-I{ROOT}/paged_attention_kv_block_amd/csrc",
           os.path.join(ROOT, "tests", "native", "allocator_stress.cpp"),
           os.path.join(ROOT, "paged_attention_kv_block_amd", "csrc", "pa_host.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower():
        pytest.skip("sanitizer runtime unavailable: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-2000:]
    # the sanitizer runtime is linked into the program; a library preloaded
    # into every process may come before it, which is harmless here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.returncode, run.stdout[-1000:], run.stderr[-3000:])
    assert run.stdout.strip().endswith("ok")
