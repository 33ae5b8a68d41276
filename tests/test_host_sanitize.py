"""The C ABI's host code under AddressSanitizer and UBSan (CPU only).

tests/host_sanitize/abi_drive.cpp calls every validator, size query and
entry point with valid arguments and with about 60 000 seeded random field
mutations; the host part of api.hip is built with both sanitizers and
linked against launchers that launch nothing (stub_launch.cpp), so no GPU
is touched and device pointers are never dereferenced.  Any sanitizer
report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "masked_bidirectional_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


LLVM_CXX = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _host_san(flags):
    """Each sanitizer flag applies to the host pass of a hipcc line only."""
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(LLVM_CXX)), reason="ROCm compilers not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    # api.hip is compiled as the library compiles it (its device array needs
    # the device pass); the sanitizers instrument its host pass only.
    for src, host_only in ((os.path.join(CSRC, "api.hip"), False), (os.path.join(HERE, "stub_launch.cpp"), True)):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "-c", "-x", "hip", "-O1", "-g", "-std=c++17", *_host_san(SAN), *inc, src, "-o", obj]
        cmd.insert(1, "--offload-host-only" if host_only else "--offload-arch=gfx950")
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_drive")
    cmd = [LLVM_CXX, "-O1", "-g", "-std=c++17", *SAN, *inc, *objs,
           os.path.join(HERE, "stub_runtime.cpp"), os.path.join(HERE, "abi_drive.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "calls checked" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
