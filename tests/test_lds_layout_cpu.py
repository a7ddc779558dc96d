"""CPU checks of the swizzled LDS tile layout (csrc/lds_layout.h).

The header's own functions are compiled for the host with g++ (the device
qualifiers defined away) and checked on every row and slot of a 64-row tile:

* lds_slot_source, which the loaders use, is the exact inverse of lds_phys;
* under the gfx950 LDS model of 64 four-byte banks (a 16-byte read serves 16
  lanes per cycle, an 8-byte transposing read 32), the three access shapes
  the header documents touch each bank once per cycle: 16-byte reads of one
  column in 16 consecutive rows, 8-byte reads of 4 consecutive rows x 64
  bytes, and 8-byte reads of two 4-row groups 8 rows apart x 32 bytes.

The bank model is the one that reproduces the hardware counter
SQ_LDS_BANK_CONFLICT on the kernels (zero on every pattern of these shapes,
and 32 cycles per wave and pass for the two-group reads under a swizzle that
moved super-row bit 2 to slot bit 0 only).
"""

import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "scheduling_persistent_attn_amd", "csrc")

PROGRAM = r"""
#define __device__
#define __forceinline__ inline
#include <cstdio>
#include <set>
#include <vector>
#include "lds_layout.h"
using namespace dash;

// byte address of byte `b` of row `row` in a tile with RB-byte rows
template <int RB> static int addr(int row, int b) { return lds_phys<RB>(row, b >> 4) + (b & 15); }

// the dwords one cycle touches, as (bank, dword) pairs; true if no bank holds two dwords
static bool one_per_bank(const std::vector<int>& byte_addrs, int width) {
  std::vector<std::set<int>> bank(64);
  for (int a : byte_addrs)
    for (int d = 0; d < width / 4; ++d) bank[(a / 4 + d) % 64].insert(a / 4 + d);
  for (auto& s : bank)
    if (s.size() > 1) return false;
  return true;
}

template <int RB> static int check() {
  int bad = 0;
  const int chunks = RB / 16, rows = 64;
  for (int R = 0; R < rows * RB / 256; ++R)
    for (int slot = 0; slot < 16; ++slot) {
      int row, chunk;
      lds_slot_source<RB>(R, slot, &row, &chunk);
      if (lds_phys<RB>(row, chunk) != R * 256 + slot * 16) {
        printf("inverse RB=%d R=%d slot=%d\n", RB, R, slot);
        ++bad;
      }
    }
  // 16-byte reads of one column in 16 consecutive rows
  for (int r0 = 0; r0 + 16 <= rows; r0 += 16)
    for (int c = 0; c < chunks; ++c) {
      std::vector<int> a;
      for (int i = 0; i < 16; ++i) a.push_back(lds_phys<RB>(r0 + i, c));
      if (!one_per_bank(a, 16)) { printf("col16 RB=%d r0=%d c=%d\n", RB, r0, c); ++bad; }
    }
  // 8-byte reads of 4 consecutive rows x 64 bytes
  for (int r0 = 0; r0 + 4 <= rows; r0 += 4)
    for (int m = 0; m < RB / 64; ++m) {
      std::vector<int> a;
      for (int i = 0; i < 4; ++i)
        for (int e = 0; e < 8; ++e) a.push_back(addr<RB>(r0 + i, 64 * m + 8 * e));
      if (!one_per_bank(a, 8)) { printf("rows4 RB=%d r0=%d m=%d\n", RB, r0, m); ++bad; }
    }
  // 8-byte reads of two 4-row groups 8 rows apart x 32 bytes
  for (int r0 = 0; r0 + 12 <= rows; r0 += 4) {
    if (r0 % 16 >= 8) continue;  // groups start at rows 16k and 16k + 4
    for (int m = 0; m < RB / 32; ++m) {
      std::vector<int> a;
      for (int g = 0; g < 2; ++g)
        for (int i = 0; i < 4; ++i)
          for (int e = 0; e < 4; ++e) a.push_back(addr<RB>(r0 + 8 * g + i, 32 * m + 8 * e));
      if (!one_per_bank(a, 8)) { printf("rows4x2 RB=%d r0=%d m=%d\n", RB, r0, m); ++bad; }
    }
  }
  return bad;
}

int main() {
  const int bad = check<128>() + check<256>();
  printf(bad ? "FAILED %d\n" : "OK\n", bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_lds_layout_inverse_and_conflict_free(tmp_path):
    src = tmp_path / "lds_layout_check.cpp"
    exe = tmp_path / "lds_layout_check"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout
