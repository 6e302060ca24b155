"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library's host source (csrc/api.cpp, with the layout rule of
csrc/layout_rule.h) together with tests/host/schedule_check.cpp and stand-ins
for the device entry points (tests/host/kernel_stubs.cpp) with g++ and
``-fsanitize=address,undefined``, then runs the checker: random layouts of
every host-built kind, batch sizes, head widths and device sizes, each
schedule checked for complete, in-order, in-limit unit and tile lists.  Any
sanitizer report aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
ROCM = "/opt/rocm"

FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
         f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def _build():
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(HOST, "kernel_stubs.cpp"),
                os.path.join(HOST, "schedule_check.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run(["g++", *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"g++ failed for {src}:\n{r.stderr[-4000:]}"
        objs.append(obj)
    exe = os.path.join(OUT, "schedule_check")
    r = subprocess.run(["g++", *FLAGS, *objs, "-o", exe, f"-L{ROCM}/lib", "-lamdhip64", "-lrocblas", "-lhipblaslt",
                        f"-Wl,-rpath,{ROCM}/lib"], capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"
    return exe


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(f"{ROCM}/include/hip"),
                    reason="needs g++ and the HIP headers")
def test_schedule_packing_under_sanitizers():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for seed in (1, 2):
        r = subprocess.run([exe, "150", str(seed)], capture_output=True, text=True, env=env, timeout=600)
        assert r.returncode == 0, f"seed {seed}: exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
        assert r.stdout.startswith("OK "), r.stdout
        assert int(r.stdout.split()[1]) >= 100, r.stdout   # most random shapes are packable
