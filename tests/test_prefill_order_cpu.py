"""Host-side check of the prefill attention's work order (no GPU).

The causal prefill attention dispatches its work items (whole query tiles
and the two key-range pieces of split tiles) longest first.  For segments
with contiguous positions the kernel maps a block index to its item in
closed form (`tile_reaching`, `prefill_item_lpt` in k_attn.hip).  This test
compiles that exact source text as host C++ and checks, over many prompt
lengths, start positions and split thresholds, that the mapping is a
bijection onto the items and that their key-tile counts never increase
along the dispatch order.
"""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "qwen2_decoder_forward_amd", "csrc", "k_attn.hip")

HARNESS = r"""
#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <vector>
using std::max;
using std::min;
constexpr int kPreKeys = 64;
%s
int main() {
  long checked = 0;
  for (int p0 = 0; p0 < 700; p0 += 23)
    for (int M = 1; M <= 4200; M += (M < 160 ? 1 : 41)) {
      const int T = (M + 31) / 32;
      auto nt = [&](int t) { return (p0 + min(32 * t + 31, M - 1)) / kPreKeys + 1; };
      const int kmax = nt(T - 1);
      for (int lim : {0, (kmax + 1) / 2, (kmax + 2) / 3, (kmax + 3) / 4, kmax}) {
        int sf = T;  // split tiles: the last ones, each with two nonempty pieces
        while (sf > 0 && nt(sf - 1) > lim && nt(sf - 1) >= 2) --sf;
        PreSeg sg{};
        sg.M = M;
        sg.n_tiles = T;
        sg.split_from = sf;
        sg.p0 = p0;
        const int n = T + (T - sf);
        std::vector<int> seen(3 * T + 2, 0);
        int prev = 1 << 30;
        for (int wi = 0; wi < n; ++wi) {
          int tile = -9, piece = -9;
          prefill_item_lpt(sg, wi, tile, piece);
          if (tile < 0 || tile >= T || piece < -1 || piece > 1 || (piece == -1) != (tile < sf)) {
            printf("bad item: p0 %%d M %%d sf %%d wi %%d -> tile %%d piece %%d\n", p0, M, sf, wi, tile, piece);
            return 1;
          }
          const int w = piece == -1 ? nt(tile) : piece == 0 ? (nt(tile) + 1) / 2 : nt(tile) / 2;
          const int key = piece == -1 ? tile : T + 2 * (tile - sf) + piece;
          if (seen[key]++) {
            printf("item twice: p0 %%d M %%d sf %%d wi %%d\n", p0, M, sf, wi);
            return 1;
          }
          if (w > prev) {
            printf("order: p0 %%d M %%d sf %%d wi %%d work %%d after %%d\n", p0, M, sf, wi, w, prev);
            return 1;
          }
          prev = w;
          ++checked;
        }
      }
    }
  printf("ok %%ld\n", checked);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_prefill_lpt_order_is_a_descending_bijection(tmp_path):
    s = open(SRC).read()
    a, b = s.index("struct PreSeg {"), s.index("struct AttnPreP {")
    code = s[a:b].replace("__device__ __forceinline__", "static inline").replace("__device__ inline",
                                                                                  "static inline")
    assert "prefill_item_lpt" in code and "tile_reaching" in code
    cpp = tmp_path / "order.cpp"
    cpp.write_text(HARNESS % code)
    exe = tmp_path / "order"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), str(cpp)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
