"""AddressSanitizer + UndefinedBehaviorSanitizer run of the host C++: the
library's validation and planning (plan.cpp) and the fp64 oracle (oracle.c),
compiled with g++/gcc into the standalone driver tests/host_sanitize/driver.cpp
(no HIP, no Python in the process), which walks the error grid and the oracle's
edge cases (empty, negative and shorter-than-t_q sequences).  Host code only:
nothing here is built for or run on a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")
PLAN = os.path.join(ROOT, "gqa_split_kv_amd", "csrc", "plan.cpp")
ORACLE = os.path.join(ROOT, "oracle", "oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gqa_split_kv_amd", "csrc")]
    objs = []
    for src, cc, extra in [(PLAN, "g++", ["-std=c++17"]), (DRIVER, "g++", ["-std=c++17"]),
                           (ORACLE, "gcc", ["-std=c11", "-fopenmp", "-ffp-contract=off"])]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([cc, *SAN, *extra, *inc, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "host_sanitize")
    subprocess.run(["g++", *SAN, "-fopenmp", "-o", exe, *objs, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "0 failed" in r.stdout, r.stdout
