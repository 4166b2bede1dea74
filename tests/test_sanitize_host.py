"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer:

  * the oracle's C, driven over small and edge shapes (tests/native/oracle_sanitize.c);
  * the library's host code (argument validation, workspace and launch
    planning), its compute entry points called with arguments that validation
    rejects before any HIP call and its planners swept over shapes up to and
    beyond the limits (tests/native/host_sanitize.c).  Only the host half of
    adamas.hip is instrumented; the decode launcher objects of the normal
    build are linked as they are.

Each build runs without a GPU and must finish with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "compressed_key_sparse_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
LLVM = "/opt/rocm/llvm/bin"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "OMP_NUM_THREADS": "4"}


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout,
                       env=dict(os.environ, **(env or {})))
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fopenmp", "-o", exe, os.path.join(ROOT, "oracle", "adamas_oracle.c"),
                    os.path.join(NATIVE, "oracle_sanitize.c"), "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], SAN_ENV)
    print(out)
    assert rc == 0, out
    assert "0 out-of-range" in out and "runtime error" not in out


def test_library_host_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    if not (os.path.exists(hipcc) and os.path.exists(os.path.join(LLVM, "clang++"))):
        pytest.skip("ROCm toolchain not available")
    from compressed_key_sparse_amd import _build
    _build.build(force=False)       # the normal objects supply the decode launchers
    objs = sorted(os.path.join(_build.OBJDIR, n + ".o") for n, _, _ in _build.UNITS
                  if n != "adamas")
    obj, lib, exe = (str(tmp_path / n) for n in ("adamas_san.o", "libadamas_san.so", "host_san"))
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"):
        san += ["-Xarch_host", f]      # host code only; device code is built as usual
    rc, out = _run([hipcc] + [f for f in _build.HIP_FLAGS if f != "-O3"] + ["-O1"] + san +
                   ["-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, "adamas.hip")])
    assert rc == 0, out
    rc, out = _run([os.path.join(LLVM, "clang++"), "-shared", "-fsanitize=address,undefined",
                    "-shared-libsan", "-o", lib, obj] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, out
    rc, out = _run([os.path.join(LLVM, "clang"), "-std=c11", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-shared-libsan", "-D__HIP_PLATFORM_AMD__",
                    "-I", INCLUDE, "-I", "/opt/rocm/include", "-o", exe,
                    os.path.join(NATIVE, "host_sanitize.c"), lib, f"-Wl,-rpath,{tmp_path}",
                    "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, out
    rc, rt = _run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"])
    env = dict(SAN_ENV, LD_LIBRARY_PATH=os.path.dirname(rt.strip()))
    rc, out = _run([exe], env)
    print(out)
    assert rc == 0, out
    assert "0 failures" in out and "runtime error" not in out
