"""Host AddressSanitizer / UndefinedBehaviorSanitizer over the C ABI's argument
validation (CPU only).  obl_api.hip is rebuilt with host-side sanitizers
(device code is not instrumented: every -fsanitize is given to the host pass
only) and linked with the regular kernel objects of the last build; a C
driver then runs every rejection path.  No GPU is touched: each call returns
before its first HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "bit_weight_linear_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang not available")
    from bit_weight_linear_amd import build as b
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "obl_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run the build first)")
    return hipcc, objs, b


def test_abi_validation_under_host_sanitizers(tmp_path):
    hipcc, objs, b = _tools()
    api_o = str(tmp_path / "obl_api_san.o")
    lib = str(tmp_path / "libobl_san.so")
    drv = str(tmp_path / "abi_reject")
    common = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}", "-I", os.path.join(ROOT, "include")]
    r = subprocess.run([hipcc, *common, *b.DEVICE_FLAGS, *HOST_SAN, "-c", os.path.join(CSRC, "obl_api.hip"),
                        "-o", api_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={b.ARCH}", api_o, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_reject.c"),
                        lib, f"-Wl,-rpath,{tmp_path}", "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "all ABI rejection checks passed" in out
