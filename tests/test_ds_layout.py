"""Host check of the stored-dS tile order (attn_tiles.h, ds_chunk_offset).

The dK/dV kernel writes its dS chunks with it, and the dQ kernel loads the
32-key groups as stored and gathers its operand with it.  This test compiles
the header with the host compiler and checks three things over every lane and
step:
* the stores of one tile cover its 32 KiB exactly once;
* each store instruction writes one aligned 1 KiB run, i.e. whole cache lines;
* the dQ kernel's reads of key row r and query chunk c find the chunk that the
  dK/dV wave of that key stored for those queries.
It also checks that the reads are conflict-free on 64 four-byte banks per
32 lanes.  The lane roles follow the kernels: a dK/dV lane (key l32, half hh)
stores chunk 4 qb + 2 h + hh, and the transposed reads use the lane split
(h, mh, e, s) of BTile::tr_frag, with the K tile holding key pi32(x) in LDS
row x.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_softmax_attention_amd", "csrc")

CHECK = r"""
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <utility>
#include "attn_tiles.h"
using namespace attn;
static int pi32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
#define REQUIRE(c) do { if (!(c)) { std::printf("FAIL %s line %d\n", #c, __LINE__); return 1; } } while (0)
int main() {
  // dK/dV stores: wave w (keys 32w..), lane (l32, hh), query block qb, half h
  std::map<int, std::pair<int, int>> content;   // byte -> (key, query chunk)
  for (int w = 0; w < 4; ++w)
    for (int qb = 0; qb < 4; ++qb)
      for (int h = 0; h < 2; ++h) {
        std::set<int> inst;
        for (int lane = 0; lane < 64; ++lane) {
          const int l32 = lane & 31, hh = lane >> 5;
          const int byte = w * 8192 + ds_chunk_offset(l32, 4 * qb + 2 * h + hh);
          REQUIRE(byte % 16 == 0 && byte >= 0 && byte < DS_ELEMS * 2);
          REQUIRE(content.count(byte) == 0);
          content[byte] = std::make_pair(32 * w + l32, 4 * qb + 2 * h + hh);
          inst.insert(byte);
        }
        REQUIRE(*inst.begin() % 1024 == 0 && *inst.rbegin() == *inst.begin() + 1008);
        REQUIRE((int)inst.size() == 64);
      }
  REQUIRE((int)content.size() == DS_ELEMS * 2 / 16);
  // dQ kernel: steps of BN keys (BN / 32 contiguous groups), 1 KiB loads, then
  // transposed reads of key pi32(r) for LDS row r of the K tile
  for (int BN = 32; BN <= 64; BN += 32)
    for (int part = 0; part < DS_T / BN; ++part)
      for (int w = 0; w < 4; ++w)
        for (int t = 0; t < BN / 16; ++t)
          for (int second = 0; second < 2; ++second) {
            std::map<int, std::set<int>> banks[2];
            for (int lane = 0; lane < 64; ++lane) {
              const int h = lane >> 5, mh = (lane >> 4) & 1, e = (lane & 15) >> 2, s = lane & 3;
              const int c = 4 * w + 2 * mh + (s >> 1);
              const int r = 16 * t + 4 * h + e + 8 * second;
              const int k = (r & ~31) | pi32(r & 31);
              const int off = (k >> 5) * 8192 + ds_chunk_offset(k & 31, c) + ((s & 1) << 3);
              REQUIRE(off >= 0 && off + 8 <= BN * DS_T * 2);
              const int gbyte = part * BN * DS_T * 2 + (off & ~15);
              REQUIRE(content.count(gbyte) == 1);
              REQUIRE(content[gbyte].first == part * BN + k && content[gbyte].second == c);
              for (int d = 0; d < 8; d += 4) banks[lane >> 5][((off + d) / 4) % 64].insert((off + d) / 4);
            }
            for (int half = 0; half < 2; ++half)
              for (auto& kv : banks[half]) REQUIRE(kv.second.size() == 1);
          }
  std::printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_stored_ds_chunk_order(tmp_path):
    src = tmp_path / "check.cpp"
    exe = tmp_path / "check"
    src.write_text(CHECK)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
