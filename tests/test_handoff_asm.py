"""The cross-workgroup hand-offs wait for their stores before counting.

A workgroup that hands data to another workgroup of the same launch writes it
with device-coherent stores and then increments an arrival counter; the
reader trusts the data once the count is complete.  On gfx950 a
workgroup-scope release fence and the workgroup barrier do not wait for
outstanding vector stores, so every wavefront must wait for vmcnt(0) itself
before the barrier that precedes the arrival atomic; otherwise the count can
become visible before the data it announces.

This test compiles the kernels that hand data over (to gfx950 assembly, on
the CPU) and checks, for every device-scope atomic add, that between the
last vector store before it and the barrier before it there is an
`s_waitcnt` with vmcnt(0)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_key_sparse_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

# one launch of every kernel that counts arrivals (host stubs instantiate them)
TU = r'''
#include "kernels.hpp"
using namespace adm;
void instantiate() {
  hipLaunchKernelGGL((k_decode<128, 1, true, 0, false>), dim3(1), dim3(1024), 0, 0, nullptr,
      nullptr, nullptr, nullptr, 0, 0, (int64_t)0, (int64_t)0, 0, 0, 0, 0, 0, 0, 0.f, nullptr,
      nullptr, nullptr, nullptr, 0, 0, EncodeRule{}, RaggedArgs{}, nullptr, 0, nullptr);
  hipLaunchKernelGGL((k_decode<128, 3, true, 1, false>), dim3(1), dim3(1024), 0, 0, nullptr,
      nullptr, nullptr, nullptr, 0, 0, (int64_t)0, (int64_t)0, 0, 0, 0, 0, 0, 0, 0.f, nullptr,
      nullptr, nullptr, nullptr, 0, 0, EncodeRule{}, RaggedArgs{}, nullptr, 0, nullptr);
  hipLaunchKernelGGL((k_decode<128, 3, true, 0, false, true>), dim3(1), dim3(1024), 0, 0,
      nullptr, nullptr, nullptr, nullptr, 0, 0, (int64_t)0, (int64_t)0, 0, 0, 0, 0, 0, 0, 0.f,
      nullptr, nullptr, nullptr, nullptr, 0, 0, EncodeRule{}, RaggedArgs{}, nullptr, 0, nullptr);
  hipLaunchKernelGGL((k_decode<128, 2, true, 0, false, false, true>), dim3(1), dim3(1024), 0, 0,
      nullptr, nullptr, nullptr, nullptr, 0, 0, (int64_t)0, (int64_t)0, 0, 0, 0, 0, 0, 0, 0.f,
      nullptr, nullptr, nullptr, nullptr, 0, 0, EncodeRule{}, RaggedArgs{}, nullptr, 0, nullptr);
  hipLaunchKernelGGL((k_decode_gs<128, 1, true>), dim3(1), dim3(1024), 0, 0, nullptr, nullptr,
      nullptr, nullptr, 0, 0, (int64_t)0, (int64_t)0, 0, 0, 0, 0, 0.f, nullptr, nullptr, nullptr,
      nullptr, nullptr, 0u, nullptr, nullptr, 0, 0, EncodeRule{}, nullptr);
  hipLaunchKernelGGL((k_attend<128, true, false>), dim3(1), dim3(1024), 0, 0, nullptr, nullptr,
      nullptr, nullptr, 0, 0, (int64_t)0, 0, 0.f, nullptr, nullptr, nullptr, PageArgs{});
  hipLaunchKernelGGL((k_select<128>), dim3(1), dim3(1024), 0, 0, nullptr, 0, (int64_t)0, 0, 0,
      0, 0, 0, nullptr, nullptr, nullptr, 0, 0);
  hipLaunchKernelGGL((k_split_select<128, true>), dim3(1), dim3(1024), 0, 0, nullptr, nullptr,
      0, 0, 0, 0, 0, 0, 0, 0, nullptr, SplitAttend{});
}
'''

STORE = re.compile(r"^\s*(buffer_store|global_store|flat_store)")
ATOMIC = re.compile(r"^\s*(global_atomic_add|flat_atomic_add|buffer_atomic_add)")
BARRIER = re.compile(r"^\s*s_barrier\b")
WAIT0 = re.compile(r"^\s*s_waitcnt\b.*\bvmcnt\(0\)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("handoff")
    src, out = d / "handoff.hip", d / "handoff.s"
    src.write_text(TU)
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC,
           "-o", str(out), str(src)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out.read_text().splitlines()


def kernels(lines):
    """(name, body lines) of every kernel in the assembly."""
    out, name, body = [], None, []
    for ln in lines:
        m = re.match(r"^(_Z\w+):\s*(;.*)?$", ln)
        if m and name is None:
            name, body = m.group(1), []
            continue
        if name is not None:
            if ln.startswith(".Lfunc_end"):
                out.append((name, body))
                name = None
            else:
                body.append(ln)
    return out


def test_every_arrival_waits_for_its_stores(asm):
    ks = kernels(asm)
    names = " ".join(n for n, _ in ks)
    for k in ("k_decode", "k_decode_gs", "k_attend", "k_select", "k_split_select"):
        assert k in names, f"{k} missing from the assembly"
    checked = 0
    for name, body in ks:
        for i, ln in enumerate(body):
            if not ATOMIC.match(ln):
                continue
            # the barrier before the atomic, and the last store before that barrier
            bar = next((j for j in range(i - 1, -1, -1) if BARRIER.match(body[j])), None)
            assert bar is not None, f"{name}: arrival atomic without a preceding barrier"
            st = next((j for j in range(bar - 1, -1, -1) if STORE.match(body[j])), None)
            if st is None:
                continue
            assert any(WAIT0.match(body[j]) for j in range(st + 1, bar)), (
                f"{name}: no s_waitcnt vmcnt(0) between the store at asm line {st} and the "
                f"barrier before the arrival atomic:\n" + "\n".join(body[st:i + 1]))
            checked += 1
    assert checked >= 6, f"only {checked} arrival atomics found"
