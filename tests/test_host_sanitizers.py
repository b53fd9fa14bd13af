"""The library's host code (config validation, KV / workspace / backward
layouts, the KV slot and offset arithmetic, every argument error of the C
ABI) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host_check/dory_host_check.cpp: seeded random configurations whose every
KV element is checked to lie inside the buffer and to belong to exactly one
cache position, configurations with one field pushed to an extreme, and the
context calls' argument errors. api.cpp and plan.cpp are compiled here with
g++ and the sanitizers; the kernels' host stubs come from the in-tree build
(looped_ngpt_amd/_build), and no call on these paths reaches HIP."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "looped_ngpt_amd", "csrc")
BUILD = os.path.join(ROOT, "looped_ngpt_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]


def _kernel_objects():
    return sorted(glob.glob(os.path.join(BUILD, "k_*.hip.o")))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    objs = _kernel_objects()
    if not objs:
        pytest.skip("no in-tree kernel objects: build the library first (python -m looped_ngpt_amd.build)")
    d = tmp_path_factory.mktemp("host_asan")
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
            os.path.join(ROOT, "tests", "host_check", "dory_host_check.cpp")]
    procs, outs = [], []
    for s in srcs:
        o = str(d / (os.path.basename(s) + ".o"))
        procs.append(subprocess.Popen(["g++", *FLAGS, "-c", s, "-o", o], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
        outs.append(o)
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out
    exe = str(d / "dory_host_check")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", *outs, *objs, f"-L{ROCM}/lib", "-lamdhip64",
                        f"-Wl,-rpath,{ROCM}/lib", "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_host_code_under_asan_ubsan(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([checker, "300"], capture_output=True, text=True, timeout=600, env=env)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert " 0 failed" in r.stdout
