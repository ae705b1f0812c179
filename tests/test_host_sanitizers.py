"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every library source is compiled with the sanitizers on its host side only (`-Xarch_host`;
device code is untouched) and linked with `tests/host/abi_host_check.cpp`, which calls every
entry point with arguments the host rejects before any HIP call, and the size queries over a
grid of sizes. No GPU is needed or used: nothing is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_sampling_verification_head_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_abi_validation_under_sanitizers(tmp_path):
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    procs = []
    for f in sources:
        obj = tmp_path / (f[:-4] + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN,
               f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(CSRC, f), "-o", str(obj)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for cmd, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{' '.join(cmd)}\n{out}\n{err}"
    drv_o = tmp_path / "abi_host_check.o"
    _run([CLANG, "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          f"-I{os.path.join(ROOT, 'include')}", "-c",
          os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"), "-o", str(drv_o)])
    exe = tmp_path / "abi_host_check"
    objs = [str(tmp_path / (f[:-4] + ".o")) for f in sources] + [str(drv_o)]
    _run([HIPCC, "--offload-arch=gfx950", *SAN[:2], *objs, "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0 and "ok (0 failures)" in res.stdout, res.stdout + res.stderr
