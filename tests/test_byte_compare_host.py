"""Exhaustive host check of the bytewise key comparison the one-byte-key
selections use (bytes_below_u, byte_flags_nibble in device_common.hpp).

The GPU kernels count, four keys per 32-bit word, how many one-byte keys lie
below a threshold byte u; this compiles those helpers into a host program
(hipcc, CPU only) and compares them with a per-byte comparison for every key
byte value at every byte position, every u in both forms' ranges, and the
other three bytes of the word drawn from a fixed mix of values (so a borrow
or carry leaking between bytes would show)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_key_sparse_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

PROG = r'''
#include <cstdio>
#include "device_common.hpp"
using namespace adm;
static unsigned ref_below(unsigned x, unsigned u) {
  unsigned r = 0;
  for (int b = 0; b < 4; ++b)
    if (((x >> (8 * b)) & 0xFFu) < u) r |= 0x80u << (8 * b);
  return r;
}
int main() {
  const unsigned others[] = {0x00u, 0x01u, 0x7Fu, 0x80u, 0x81u, 0xFEu, 0xFFu, 0x3Cu, 0xC3u};
  long checked = 0;
  for (unsigned u = 0; u <= 255; ++u) {
    for (unsigned pos = 0; pos < 4; ++pos)
      for (unsigned v = 0; v <= 255; ++v)
        for (unsigned o : others)
          for (unsigned o2 : others) {
            unsigned x = 0;
            for (unsigned b = 0; b < 4; ++b)
              x |= (b == pos ? v : (b & 1 ? o : o2)) << (8 * b);
            const unsigned want = ref_below(x, u), xm = x | 0x80808080u;
            if (u <= 128) {
              const unsigned got = bytes_below_u<false>(x, xm, u * 0x01010101u);
              if (got != want) { printf("LO u=%u x=%08x got %08x want %08x\n", u, x, got, want); return 1; }
              ++checked;
            }
            if (u >= 128) {
              const unsigned got = bytes_below_u<true>(x, xm, (u - 128u) * 0x01010101u);
              if (got != want) { printf("HI u=%u x=%08x got %08x want %08x\n", u, x, got, want); return 1; }
              ++checked;
            }
          }
  }
  for (unsigned f = 0; f < 16; ++f) {
    unsigned m = 0;
    for (int k = 0; k < 4; ++k) if (f >> k & 1) m |= 0x80u << (8 * k);
    if (byte_flags_nibble(m) != f) { printf("nibble %x -> %x\n", f, byte_flags_nibble(m)); return 1; }
  }
  printf("ok %ld\n", checked);
  return 0;
}
'''


def test_bytes_below_exhaustive(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "bytes_below.hip"
    src.write_text(PROG)
    exe = tmp_path / "bytes_below"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
                    "-o", str(exe), str(src)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
