"""The library from C++ through include/seg_attn.h alone: tests/native/abi_gpu_check.cpp is
compiled with the host compiler against the HIP runtime and the built libsegattn.so (host code
only, no device code) and run on the GPU; it checks exact one-key rows, decode against
prefill, the allocation-free decode against decode, and the argument errors."""
import os
import shutil
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@needs_gpu
def test_native_caller(tmp_path):
    import attention_segmented_kv_amd as sa
    lib = sa.library_path("release")
    if not os.path.exists(lib):
        pytest.skip("libsegattn.so not built")
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "abi_gpu_check"
    libdir = os.path.dirname(lib)
    cmd = [cxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "native", "abi_gpu_check.cpp"),
           "-o", str(exe), "-L" + libdir, "-l:" + os.path.basename(lib), "-Wl,-rpath," + libdir,
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print("[case] native C++ caller of the C ABI", flush=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
