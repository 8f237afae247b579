"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU call): ssm_abi.cpp is compiled
again with g++ -fsanitize=address,undefined, linked with the library's other
objects from the last build into a library of its own, and
tests/test_abi_host.py runs against that library in a child process with the
sanitizer runtime preloaded. Any report fails the run."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_state_space_16_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    objs = sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o"))
                  if os.path.basename(o) not in ("ssm_abi.cpp.o", "ssm_calib.hip.o"))
    if not objs or not shutil.which("g++"):
        pytest.skip("the library's objects are not built (run __graft_entry__.build()) or g++ is missing")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("libasan is not installed")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "ssm_abi_san.o")
    lib = str(tmp_path / "libssm_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", *san,
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(PKG, "csrc", "ssm_abi.cpp"), "-o", obj], check=True)
    subprocess.run(["g++", "-shared", *san, "-o", lib, obj, *objs, "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    env = dict(os.environ, SSM_LIBRARY=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the binding-with-torch case is left out: torch is not built with the sanitizer
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "not binding_refuses_cpu_tensors", os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in r.stdout, out
