"""The C ABI's host-side validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer: the library's sources are compiled with the host
part instrumented (device code is not: GPU sanitizers are not used here), a C
driver (tests/sanitize/abi_validation.c) makes every validation-failing call,
the size queries and, without a GPU, the calls that must stop at the device
check; any sanitizer report or failed check fails the test."""
import os
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mlp_prefill_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc and clang")
def test_host_validation_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libnvfp4_san.so"
    srcs = [os.path.join(CSRC, f) for f in ("nvfp4_abi.hip", "quant.hip", "gemm.hip", "moe.hip")]
    build = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fvisibility=hidden",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", str(lib)]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_validation"
    r = subprocess.run([CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_validation.c"),
                        "-L", str(tmp_path), "-lnvfp4_san", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    args = [str(exe)] + (["nodevice"] if torch.cuda.device_count() == 0 else [])
    r = subprocess.run(args, capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
