"""The kernels' work-item orders (csrc/schedule.h) checked on the CPU.

The header's functions decide which item each workgroup or wave takes: the
prefill's XCD chunks, the backward's four-at-a-time batch-head groups and
the decode split kernel's block ranges.  An order that is not a permutation
would leave tiles uncomputed (or computed twice) only for the grid shapes
that reach the faulty case, so the header is compiled for the host with
hipcc and each order is checked over many shapes:
  * remap_item and group_heads_on_xcd are permutations of the grid;
  * with chunking, the workgroups of one chunk share an XCD (i mod 8);
  * with head groups, every XCD keeps the batch-heads equal to it mod 8,
    takes them four at a time and walks each group's tiles in rank order
    (longest first);
  * the decode ranges partition the block list, each used wave gets a
    non-empty range, and wave_of(b) names the range that holds b.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_34_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CHECKER = r"""
#include <cstdio>
#include <cstdlib>
#include <vector>
#include "schedule.h"
using namespace attn;

static long checks = 0;
#define EXPECT(c, ...) do { ++checks; if (!(c)) { std::printf("FAIL: " __VA_ARGS__); \
  std::printf("\n"); std::exit(1); } } while (0)

static void prefill(int n, int c) {
  std::vector<int> seen(n, 0), xcd_of_chunk(n, -1);
  const bool active = c > 1 && n % (8 * c) == 0;
  for (int i = 0; i < n; ++i) {
    const int j = remap_item(i, n, c);
    EXPECT(j >= 0 && j < n, "remap_item(%d, %d, %d) = %d out of range", i, n, c, j);
    EXPECT(!seen[j]++, "remap_item(., %d, %d) takes item %d twice", n, c, j);
    if (!active) {
      EXPECT(j == i, "remap_item(%d, %d, %d) = %d, expected the identity", i, n, c, j);
    } else {
      int& x = xcd_of_chunk[j / c];
      if (x < 0) x = i & 7;
      EXPECT(x == (i & 7), "chunk %d of n=%d c=%d spans XCDs %d and %d", j / c, n, c, x, i & 7);
    }
  }
}

static void backward(int bh, int nt) {
  const int n = bh * nt;
  std::vector<int> seen(n, 0);
  for (int i = 0; i < n; ++i) {
    const int r = group_heads_on_xcd(i, bh, nt);
    EXPECT(r >= 0 && r < n, "group_heads_on_xcd(%d, %d, %d) = %d out of range", i, bh, nt, r);
    EXPECT(!seen[r]++, "group_heads_on_xcd(., %d, %d) takes item %d twice", bh, nt, r);
    if (bh % 32 != 0) EXPECT(r == i, "bh=%d: expected the identity", bh);
  }
  if (bh % 32 != 0) return;
  for (int x = 0; x < 8; ++x) {
    // positions of XCD x in dispatch order: workgroups x, x + 8, ...
    const int per_xcd = n / 8, group = 4 * nt;
    for (int g = 0; g * group < per_xcd; ++g) {
      std::vector<int> heads;
      int last_rank = -1;
      for (int pos = g * group; pos < (g + 1) * group; ++pos) {
        const int r = group_heads_on_xcd(pos * 8 + x, bh, nt);
        const int rank = r / bh, head = r % bh;
        EXPECT(head % 8 == x, "bh=%d nt=%d: XCD %d takes batch-head %d", bh, nt, x, head);
        EXPECT(rank >= last_rank, "bh=%d nt=%d: XCD %d group %d goes back to rank %d", bh, nt,
               x, g, rank);
        last_rank = rank;
        bool known = false;
        for (int h : heads) known |= (h == head);
        if (!known) heads.push_back(head);
      }
      EXPECT(heads.size() == 4, "bh=%d nt=%d: XCD %d group %d holds %d batch-heads", bh, nt, x,
             g, (int)heads.size());
    }
  }
}

static void decode(long long T, int Wl) {
  const int W = used_waves(T, Wl);
  EXPECT(W >= 1 && W <= Wl, "used_waves(%lld, %d) = %d", T, Wl, W);
  EXPECT(W == Wl || (long long)W * kDecMinBlocks >= T, "used_waves(%lld, %d) = %d too few", T,
         Wl, W);
  EXPECT((long long)(W - 1) * kDecMinBlocks < T, "used_waves(%lld, %d) = %d too many", T, Wl, W);
  EXPECT(range_start(0, T, W) == 0 && range_start(W, T, W) == T, "ranges of T=%lld W=%d", T, W);
  for (int w = 0; w < W; ++w)
    EXPECT(range_start(w + 1, T, W) > range_start(w, T, W), "T=%lld W=%d: wave %d has no blocks",
           T, W, w);
  const long long step = T > 200000 ? T / 100003 : 1;
  for (long long b = 0; b < T; b += step) {
    const int w = wave_of(b, T, W);
    EXPECT(w >= 0 && w < W && range_start(w, T, W) <= b && b < range_start(w + 1, T, W),
           "wave_of(%lld, %lld, %d) = %d", b, T, W, w);
  }
  const int w = wave_of(T - 1, T, W);
  EXPECT(w == W - 1, "wave_of(last block of %lld, %d) = %d", T, W, w);
}

int main() {
  for (int n = 1; n <= 2048; ++n)
    for (int c : {0, 1, 2, 3, 4, 8}) prefill(n, c);
  for (int n : {4096, 8192, 16384, 65536})
    for (int c : {2, 4, 8}) prefill(n, c);
  for (int bh = 1; bh <= 160; ++bh)
    for (int nt = 1; nt <= 20; ++nt) backward(bh, nt);
  for (int bh : {256, 512})
    for (int nt : {1, 7, 64, 128}) backward(bh, nt);
  for (long long T = 1; T <= 3000; ++T)
    for (int W : {1, 7, 64, 2048}) decode(T, W);
  for (long long T : {16383LL, 278528LL, 2228224LL, 1073741827LL})
    for (int W : {2048, 1999}) decode(T, W);
  std::printf("ok %ld checks\n", checks);
  return 0;
}
"""


@pytest.mark.timeout(300)
def test_work_item_orders(tmp_path):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not available")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    src = tmp_path / "schedule_check.cpp"
    src.write_text(CHECKER)
    exe = tmp_path / "schedule_check"
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O2",
                    "-I" + CSRC, str(src), "-o", str(exe)], check=True, capture_output=True,
                   text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    assert res.stdout.startswith("ok "), res.stdout[-2000:]
