"""The C-ABI tests again, against a build of libfgq whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged).

The host code is the argument validation, the workspace planning and the
launch set-up that every C call runs before any kernel; the tests in
test_abi.py drive its error paths without a GPU.  The sanitized library is
built once per source state under _build/host_sanitized/ and loaded in a
child process with the clang ASan runtime preloaded (the Python interpreter
itself is not instrumented).  CPU only.
"""
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_fp8_quant_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "host_sanitized")

# host-side sanitizers only; the device code is built as usual
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
SAN_STRICT = "-Xarch_host -fno-sanitize-recover=undefined".split()
COMMON = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]
SOURCES = {"fgq_api.cpp": [], "quant.hip": ["-ffp-contract=off"], "dispatch.hip": ["-ffp-contract=off"],
           "gemm.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _source_key():
    h = hashlib.sha256(" ".join(COMMON + SAN + SAN_STRICT).encode())
    for f in sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _build_sanitized(cc):
    key = _source_key()
    lib = os.path.join(OUT, f"libfgq_host_sanitized_{key}.so")
    if os.path.exists(lib):
        return lib
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(OUT, src.replace(".", "_") + ".o")
        subprocess.run([cc, *COMMON, *extra, *SAN, *SAN_STRICT, "-c", os.path.join(CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, *objs, "-o", lib], check=True,
                   capture_output=True)
    return lib


@pytest.mark.skipif(_hipcc() is None or _asan_runtime() is None, reason="needs hipcc and the clang ASan runtime")
def test_abi_tests_pass_under_host_sanitizers():
    lib = _build_sanitized(_hipcc())
    # the host code is instrumented: it calls the sanitizers' report hooks
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True, check=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update(FGQ_LIB=lib, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
