// Work-item orders of the kernels' grids: which item a workgroup (or wave)
// takes.  They are pure integer functions, compiled for the host as well as
// the device, so that their properties (each order is a permutation, each
// XCD keeps the items it should, the decode ranges partition the block list)
// can be checked on the CPU for many grid shapes.
//
// A workgroup with linear index i runs on XCD i % 8 (workgroups are dealt
// round-robin to the eight XCDs, each with its own 4 MB L2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kXcds = 8;   // the shifts and masks below assume 8

// ---- prefill ----
// Items are numbered longest-first (query tile descending when causal), then
// batch, then head; consecutive heads of a GQA group are consecutive items.
// With chunk = c > 1 (and num_items a multiple of 8c), chunks of c
// consecutive items are dealt round-robin to the XCDs, so the c workgroups of
// a chunk run on the same XCD and share its L2.  Otherwise item = i.
__host__ __device__ inline int remap_item(int i, int num_items, int chunk) {
  if (chunk <= 1 || (num_items % (kXcds * chunk)) != 0) return i;
  const int x = i & 7, pos = i >> 3;
  const int round = pos / chunk, within = pos - round * chunk;
  return (round * kXcds + x) * chunk + within;
}

// ---- backward ----
// The dK/dV and dQ grids number their items (tile rank, batch-head), the
// longest tiles first under the causal mask, so each XCD gets the
// batch-heads equal to it mod 8.  When the batch-head count bh is a multiple
// of 32, each XCD instead takes its batch-heads four at a time: every tile of
// four batch-heads, longest first, before any tile of the next four.  The
// tiles running together then read the Q/dO (or K/V) rows of four
// batch-heads rather than of all of them, which the XCD's L2 can hold, and
// the longest-first order still holds within each group of four.  (All of
// an XCD's tiles for two batch-heads at once cut the fetches further, but
// mixed long and short tiles in every round and ran 10 % slower.)  Returns
// the item rank * bh + batch-head of workgroup blk (grid = ntile * bh).
__host__ __device__ inline int group_heads_on_xcd(int blk, int bh, int ntile) {
  if ((bh & 31) != 0) return blk;
  const int x = blk & 7, pos = blk >> 3;
  const int per = 4 * ntile, g = pos / per, w = pos - g * per;
  return (w >> 2) * bh + (g * 4 + (w & 3)) * 8 + x;
}

// ---- decode ----
// The split kernel's persistent waves cut the flattened list of T (sequence,
// KV head, block) entries into contiguous ranges.
// Waves that take part for a list of T blocks: every wave gets at least
// kDecMinBlocks blocks (fewer waves, fewer units cut between them), at most
// the W launched.
constexpr int kDecMinBlocks = 8;
__host__ __device__ inline int used_waves(int64_t T, int W) {
  const int64_t w = (T + kDecMinBlocks - 1) / kDecMinBlocks;
  return w < W ? (int)w : W;
}

// Range of wave w in the flattened block list: [w T / W, (w + 1) T / W).
__host__ __device__ inline int64_t range_start(int w, int64_t T, int W) {
  return (int64_t)w * T / W;
}

// The wave whose range holds block b (0 <= b < T): the last w whose range
// starts at or before b.
__host__ __device__ inline int wave_of(int64_t b, int64_t T, int W) {
  int w = (int)(b * W / T);   // range_start(w) <= b already
  while (w + 1 < W && range_start(w + 1, T, W) <= b) ++w;
  return w;
}

}  // namespace attn
