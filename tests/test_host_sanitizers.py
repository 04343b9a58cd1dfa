"""The C-ABI host layer under the host sanitizers (CPU only): emb_api.cpp and
emb_plan.cpp are compiled with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only; the device side is replaced by stubs that abort, so no
GPU and no HIP runtime is involved), linked with a C harness that drives every
entry point through its argument checks, and run. Any sanitizer report, leak,
or a check reaching the device fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dlrm_sparse_embedding_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None or
                    not os.path.isdir(HIP_INCLUDE), reason="needs gcc/g++ and the HIP headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HIP_INCLUDE, "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, lang in ((os.path.join(CSRC, "emb_api.cpp"), "c++"), (os.path.join(CSRC, "emb_plan.cpp"), "c++"),
                      (os.path.join(HERE, "device_stubs.cpp"), "c++"), (os.path.join(HERE, "abi_harness.c"), "c")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cc = ["g++", "-std=c++17"] if lang == "c++" else ["gcc", "-std=c11"]
        r = subprocess.run(cc + san + inc + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_harness")
    r = subprocess.run(["g++"] + san + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the environment is passed on unchanged; ASan is told not to insist on
    # being the first library loaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"harness failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    assert "abi harness ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
