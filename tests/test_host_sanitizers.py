"""The host packers under sanitizers (CPU only).

tests/native/pack_sanitize.cpp drives w4a16_pack, w4a16_codec_pack (every
codec), w4a16_kv_pack (both widths) and w4a16_blob_check at ragged and large
shapes, with every buffer allocated at exactly its documented size. It is
built together with the library's packer source by g++ under
AddressSanitizer + UndefinedBehaviorSanitizer (out-of-bounds reads and writes,
undefined arithmetic) and under ThreadSanitizer (the packers split large
inputs over threads), and must finish clean with its own checks passing.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "bit_weight_quantized_w4a16_amd", "csrc", "w4a16_pack.cpp"),
           os.path.join(ROOT, "tests", "native", "pack_sanitize.cpp")]
INCLUDES = ["-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
            "-I" + os.path.join(ROOT, "bit_weight_quantized_w4a16_amd", "csrc")]

FLAVOURS = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}


@pytest.mark.parametrize("flavour", sorted(FLAVOURS))
def test_packers_clean_under_sanitizer(tmp_path, flavour):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / f"pack_{flavour}")
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-pthread", "-D__HIP_PLATFORM_AMD__"] + FLAVOURS[flavour]
           + INCLUDES + SOURCES + ["-o", exe])
    built = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert built.returncode == 0, built.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = (run.stdout + run.stderr)[-6000:]
    assert run.returncode == 0, report
    assert run.stdout.strip().startswith("ok "), report
    assert "Sanitizer" not in run.stderr and "runtime error" not in run.stderr, report
