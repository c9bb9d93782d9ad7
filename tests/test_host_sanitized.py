"""Host-only AddressSanitizer + UndefinedBehaviorSanitizer build of libfa's C
ABI argument validation (fa_api.cpp, with stub launchers that report no
device) and of the fp64 oracle, built with the host compilers (gcc/g++) and
run on the CPU: every error code is forced, calls that pass validation stop
at FA_ERR_DEVICE, the size helpers take extreme arguments, and the oracle
runs on tiny inputs (tests/sanitize/driver.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None
                    or not os.path.isdir(ROCM_INC), reason="needs gcc, g++ and the HIP headers")
def test_abi_validation_and_oracle_under_asan_ubsan(tmp_path):
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
    inc = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", f"-I{ROOT}/include",
           f"-I{ROOT}/exact_io_aware_08_amd/csrc"]
    objs = []

    def cc(cmd, src, obj):
        subprocess.run(cmd + san + ["-c", src, "-o", str(tmp_path / obj)], check=True,
                       timeout=600)
        objs.append(str(tmp_path / obj))

    cc(["gcc", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off"], f"{ROOT}/oracle/oracle.c",
       "oracle.o")
    cc(["g++", "-std=c++17"] + inc, f"{ROOT}/exact_io_aware_08_amd/csrc/fa_api.cpp", "fa_api.o")
    cc(["g++", "-std=c++17"] + inc, f"{ROOT}/tests/sanitize/launch_stubs.cpp", "stubs.o")
    cc(["g++", "-std=c++17", f"-I{ROOT}/include"], f"{ROOT}/tests/sanitize/driver.cpp", "driver.o")
    exe = str(tmp_path / "driver")
    subprocess.run(["g++"] + san + objs + ["-o", exe, "-lpthread", "-lm"], check=True, timeout=600)
    # verify_asan_link_order=0: the run must not depend on what the
    # environment preloads
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
