// Paged single-token decode: each sequence's one query row attends to all of
// its cached tokens, read through a block table (PagedAttention, tutorial
// "Chapter 3 Advanced principles", section 3.0: fixed-size KV blocks and a
// per-sequence table of physical block ids; shared prefixes are repeated ids).
//
// Work decomposition (split-K over a flattened block list).  A "unit" is one
// (sequence, KV head) pair; it owns ceil(context / 16) blocks and serves the
// GQA group of query heads that read that KV head, so every K/V byte is
// fetched once.  All units' blocks, in (sequence, KV head, block) order, form
// one list of T blocks that is cut into W equal contiguous ranges, one per
// persistent wave.  A wave streams its range through a ring of RING blocks of
// K and V loads that runs on across unit boundaries, so the memory pipeline
// fills once per wave instead of once per unit.
//   * a unit that lies entirely inside one wave's range is finished there:
//     normalised output and log-sum-exp are written directly;
//   * a unit cut by range boundaries leaves one partial (unnormalised O, max,
//     sum) per wave it touches -- at most two per wave: the head segment
//     (unit begun in an earlier range) and the tail segment (unit continued in
//     a later range);
//   * the combine kernel merges a cut unit's partials by their log-sum-exp,
//     the same rescaling by exp(m_p - M) that the online softmax applies
//     between key blocks.
// Per block: q.K^T for 16 tokens on the matrix cores (v_mfma_f32_16x16x32,
// query heads as A rows zero padded to 16, K read straight from memory in the
// B-operand layout), online softmax with a lazily raised reference max, and
// P.V on the vector ALUs as packed dot products over token pairs.
//
// Tokens at or past the context length are never multiplied: their scores are
// replaced (not scaled) by -inf and their V rows are zeroed before use, so
// whatever a partially filled block holds past the end cannot reach the
// output.  Nothing depends on physical block ids except addresses, so results
// are bit-identical under any block table.
#include <algorithm>

#include "common.h"
#include "schedule.h"

namespace attn {

constexpr int kDecBS = 16;          // tokens per KV block
constexpr int kDecMaxWaves = 2048;  // persistent waves: 8 per CU on 256 CUs (2 per SIMD)

// Blocks of a sequence.
__device__ inline int seq_blocks(int ctx) { return ctx > 0 ? (ctx + kDecBS - 1) / kDecBS : 0; }
// Blocks of one (sequence, KV head) unit: the sequence's blocks from table
// entry fb on (fb = 0, or in shared-prefix decode the blocks of the group's
// prefix, which the prefix kernel covers).
__device__ inline int unit_blocks(int ctx, int fb) {
  const int nb = seq_blocks(ctx) - fb;
  return nb > 0 ? nb : 0;
}
__device__ inline int first_block_of(const DecodeParams& p, int s) {
  return p.first_block != nullptr ? p.first_block[s] : 0;
}

// Total unit blocks over all sequences and those of sequences before `s`,
// reduced across the 64 lanes of the calling wave (the results are uniform).
__device__ inline void seq_block_sums(const DecodeParams& p, int s, int lane, int64_t& before,
                                      int64_t& total) {
  before = 0;
  total = 0;
  for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
    const int ss = s0 + lane;
    const int nb = (ss < p.num_seqs) ? unit_blocks(p.context_lens[ss], first_block_of(p, ss)) : 0;
    int a = (ss < s) ? nb : 0, t = nb;
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) {
      a += __shfl_xor(a, sh);
      t += __shfl_xor(t, sh);
    }
    before += __builtin_amdgcn_readfirstlane(a);
    total += __builtin_amdgcn_readfirstlane(t);
  }
}

template <typename TT, int D, int GP, int RING>
// Two waves per SIMD (8 per CU) while the output partials (GP heads x D
// columns) are small enough, one for larger ones, which need the registers.
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64),
                          amdgpu_waves_per_eu(GP * D <= 512 ? 2 : 1, GP * D <= 512 ? 2 : 1)))
void paged_decode_split_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  constexpr int KST = D / 32;            // k-steps of q.K^T (16x16x32)
  constexpr int CH = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROWS = 64 / CH;          // V rows per 16-byte load instruction
  constexpr int VST = kDecBS / ROWS;     // V load instructions per block
  // the reference max is raised only when it grows by more than TAU (log2
  // units); probabilities stay below 2^TAU and O is rescaled rarely
  constexpr float TAU = 8.0f;
  static_assert(GP % 4 == 0 && GP <= 16, "padded group");
  // wave-private exchange: rounded probabilities [head][token], rescale
  // factors, final max and sums per head
  __shared__ __attribute__((aligned(16))) uint16_t xp16[GP * kDecBS];
  __shared__ __attribute__((aligned(16))) float xm[2 * GP];

  const int w = blockIdx.x;
  const int lane = threadIdx.x;
  const int group = p.group;
  const float c = p.scale_log2;

  // list spans of 64 sequences (one round of loads): this lane's context,
  // first table entry, span and the inclusive prefix sum of spans
  struct Round {
    int ctx, fb;
    int64_t span, incl;
  };
  auto load_round = [&](int s0) {
    Round r;
    const int ss = s0 + lane;
    r.ctx = ss < p.num_seqs ? p.context_lens[ss] : 0;
    r.fb = ss < p.num_seqs ? first_block_of(p, ss) : 0;
    r.span = (int64_t)unit_blocks(r.ctx, r.fb) * p.h_kv;
    r.incl = r.span;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int64_t t = __shfl_up(r.incl, sh);
      if (lane >= sh) r.incl += t;
    }
    return r;
  };
  auto lane_value = [](int64_t v, int l) {
    return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((int)v, l));
  };
  // the first round serves both the list length (up to 64 sequences) and
  // the seek below, so the wave starts after one round trip
  const Round r0 = load_round(0);
  int64_t nlist;   // blocks in the list
  if (p.num_seqs <= 64) {
    nlist = lane_value(r0.incl, 63);
  } else {
    int64_t unused_before, total_seq_blocks;
    seq_block_sums(p, 0, lane, unused_before, total_seq_blocks);
    nlist = total_seq_blocks * p.h_kv;
  }
  if (nlist == 0) return;
  const int W = used_waves(nlist, gridDim.x);
  if (w >= W) return;
  const int64_t b0 = range_start(w, nlist, W), b1 = range_start(w + 1, nlist, W);
  if (b0 >= b1) return;

  // position in the unit list: unit (s, kvh), its blocks, context and first
  // table entry, the list position of its first block and the block within it
  struct Cursor {
    int s, kvh, nblk, ctx, fb;
    int64_t ustart;
    int lb;
  };
  // list position b -> cursor: the lane whose span holds b is picked by a
  // ballot, 64 sequences per round (the first round is already loaded)
  auto seek = [&](int64_t b) {
    Cursor cu{};
    int64_t base = 0;
    for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
      const Round r = s0 == 0 ? r0 : load_round(s0);
      const int64_t lo = base + r.incl - r.span;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(r.span > 0 && b >= lo && b < lo + r.span);
      if (hit != 0) {
        const int l = (int)__builtin_ctzll(hit);
        cu.s = s0 + l;
        cu.ctx = __builtin_amdgcn_readlane(r.ctx, l);
        cu.fb = __builtin_amdgcn_readlane(r.fb, l);
        cu.nblk = unit_blocks(cu.ctx, cu.fb);
        const int64_t pos = lane_value(lo, l);
        cu.kvh = (int)((b - pos) / cu.nblk);
        cu.ustart = pos + (int64_t)cu.kvh * cu.nblk;
        cu.lb = (int)(b - cu.ustart);
        return cu;
      }
      base += lane_value(r.incl, 63);
    }
    return cu;   // not reached: b lies inside the list
  };
  auto advance = [&](Cursor& cu) {
    if (++cu.lb < cu.nblk) return;
    cu.ustart += cu.nblk;
    cu.lb = 0;
    if (++cu.kvh < p.h_kv) return;
    cu.kvh = 0;
    do {   // next sequence with blocks (past the end: a harmless dummy unit)
      ++cu.s;
      const bool in = cu.s < p.num_seqs;
      cu.ctx = in ? ld_meta(p.context_lens, cu.s) : 1;
      cu.fb = (in && p.first_block != nullptr) ? ld_meta(p.first_block, cu.s) : 0;
      cu.nblk = unit_blocks(cu.ctx, cu.fb);
    } while (cu.nblk == 0);
  };

  const char* kc = (const char*)p.k_cache;
  const char* vc = (const char*)p.v_cache;
  const int64_t blk_bytes = (int64_t)kDecBS * D * 2;

  // per-lane byte offsets within a (block, kv head) tile of 16 x D
  //   K, B operand: token lane % 16, d = 32 st + 8 (lane / 16)
  //   V, for the vector products: load st brings token
  //   2 (lane / CH) + (st & 1) + (st >> 1) * 2 ROWS, d = 8 (lane % CH), so that
  //   loads 2u and 2u+1 hold two adjacent tokens of the same 8 columns
  const uint32_t kl = (uint32_t)((lane & 15) * D + (lane >> 4) * 8) * 2u;
  const int vrow = lane / CH;
  auto vtok = [&](int st) { return 2 * vrow + (st & 1) + (st >> 1) * 2 * ROWS; };
  const uint32_t vl = (uint32_t)(2 * vrow * D + (lane % CH) * 8) * 2u;

  u32x4 kr[RING][KST], vr[RING][VST];
  // Loads of one (block, KV head) tile through buffer resources based at the
  // tile (scalar base, every lane offset inside it), marked non-temporal: each
  // K/V byte is read once, and streaming it past the caches keeps them for
  // the data that is reused.  A refill past the end of
  // the range uses an empty resource: the loads still issue, in the same
  // order, but return zeros without touching memory.
  auto issue = [&](const Cursor& cu, int slot, bool real) {
    const char* kb = kc;
    const char* vb = vc;
    if (real) {
      const int64_t phys =
          ld_meta(p.block_table, (int64_t)cu.s * p.max_blocks_per_seq + cu.fb + cu.lb);
      kb += (phys * p.h_kv + cu.kvh) * blk_bytes;
      vb += (phys * p.h_kv + cu.kvh) * blk_bytes;
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, real ? (uint32_t)blk_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, real ? (uint32_t)blk_bytes : 0u);
#pragma unroll
    for (int st = 0; st < KST; ++st) kr[slot][st] = buf_load16_nt(rk, kl + st * 64);
#pragma unroll
    for (int st = 0; st < VST; ++st)
      vr[slot][st] = buf_load16_nt(rv, vl + ((st & 1) + (st >> 1) * 2 * ROWS) * D * 2);
  };
  // query heads of a unit as the A operand of S = Q K^T (rows = heads, zero padded)
  u32x4 qa[KST];
  auto load_q = [&](const Cursor& cu) {
    const int g = lane & 15;
    const T* qg =
        (const T*)p.q + ((int64_t)cu.s * p.h_q + cu.kvh * group + g) * D + (lane >> 4) * 8;
#pragma unroll
    for (int st = 0; st < KST; ++st) {
      qa[st] = u32x4{0, 0, 0, 0};
      if (g < group) qa[st] = *(const u32x4*)(qg + 32 * st);
    }
    // Drain here, once per unit (vmcnt(0); expcnt and lgkmcnt unconstrained).
    // The Q loads are issued after the K/V loads in flight; waiting for them
    // at each block would drain the whole ring every block.
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };

  // running state of the current unit: reference max of the heads of this
  // lane's 16-lane row (heads (lane/16)*4 + r), per-lane partial sums of the
  // rounded probabilities, output partials (heads x 8 columns of chunk lane%CH)
  const int grow_row = lane >> 4;
  const bool score_lane = grow_row * 4 < GP;
  float m_ref[4], l_part[4];
  float oa[GP][8];
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_ref[r] = -INFINITY;
      l_part[r] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) oa[g][e] = 0.f;
  };

  auto process = [&](const Cursor& cu, int slot) {
    // ---- scores of 16 tokens x (up to 16) heads on the matrix cores ----
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KST; ++st) acc = TT::mma16(qa[st], kr[slot][st], acc);
    // lane holds token lb*16 + lane%16, heads (lane/16)*4 + r (log2 units);
    // tokens past the context are replaced by -inf (never multiplied)
    const int tbase = (cu.fb + cu.lb) * kDecBS;
    const bool tv = tbase + (lane & 15) < cu.ctx;
    float sc[4];
    bool grow = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = tv ? acc[r] * c : -INFINITY;
      grow = grow || (score_lane && sc[r] > m_ref[r] + TAU);
    }
    // ---- rare: a score passed its head's reference by more than TAU ----
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      float alpha[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float bm = row16_max(sc[r]);
        const bool up = bm > m_ref[r] + TAU;
        alpha[r] = fast_exp2(up ? m_ref[r] - bm : 0.f);
        m_ref[r] = up ? bm : m_ref[r];
        l_part[r] *= alpha[r];
      }
      if ((lane & 15) == 0 && score_lane)
        *(f32x4*)(xm + grow_row * 4) = f32x4{alpha[0], alpha[1], alpha[2], alpha[3]};
      lds_order();
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 a = *(const f32x4*)(xm + g4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) oa[g4 + r][e] *= a[r];
      }
    }
    // probabilities relative to the reference, rounded as they enter P V,
    // to LDS as [head][token]; l sums the rounded values
    if (score_lane) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mm = (m_ref[r] == -INFINITY) ? 0.f : m_ref[r];
        const uint32_t wv = TT::pack2(fast_exp2(sc[r] - mm), 0.f);
        l_part[r] = TT::sum2(wv, l_part[r]);
        xp16[(grow_row * 4 + r) * kDecBS + (lane & 15)] = (uint16_t)wv;
      }
    }
    lds_order();
    // ---- O += p v with packed dot products over token pairs ----
    const bool last = tbase + kDecBS > cu.ctx;
#pragma unroll
    for (int u = 0; u < VST / 2; ++u) {
      const int t0 = vtok(2 * u);   // t1 = t0 + 1
      u32x4 va = vr[slot][2 * u], vb2 = vr[slot][2 * u + 1];
      if (last) {
        if (tbase + t0 >= cu.ctx) va = u32x4{0, 0, 0, 0};
        if (tbase + t0 + 1 >= cu.ctx) vb2 = u32x4{0, 0, 0, 0};
      }
      uint32_t vp[8];   // (v[t0][d], v[t1][d]) pairs for the 8 columns
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vp[2 * k] = join_lo16(va[k], vb2[k]);
        vp[2 * k + 1] = join_hi16(va[k], vb2[k]);
      }
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const uint32_t pp = *(const uint32_t*)(xp16 + g * kDecBS + t0);
#pragma unroll
        for (int e = 0; e < 8; ++e) oa[g][e] = TT::dot2(vp[e], pp, oa[g][e]);
      }
    }
  };

  // ---- finish this wave's segment [seg_start, seg_end) of a unit ----
  auto finish = [&](const Cursor& cu, int64_t seg_start, int64_t seg_end) {
    // the wave holding a unit's first block records where its partials are:
    // this wave and the count of waves the unit spans
    if (seg_start == cu.ustart && lane == 0) {
      const int wl = wave_of(cu.ustart + cu.nblk - 1, nlist, W);
      int32_t* ui = p.ws_unit + ((int64_t)cu.s * p.h_kv + cu.kvh) * 2;
      ui[0] = w;
      ui[1] = wl - w + 1;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) l_part[r] = row16_sum(l_part[r]);
    if ((lane & 15) == 0 && score_lane) {
      *(f32x4*)(xm + grow_row * 4) = f32x4{m_ref[0], m_ref[1], m_ref[2], m_ref[3]};
      *(f32x4*)(xm + GP + grow_row * 4) = f32x4{l_part[0], l_part[1], l_part[2], l_part[3]};
    }
    lds_order();
    // sum O over the lanes sharing a column chunk
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = oa[g][e];
        for (int sh = CH; sh < 64; sh <<= 1) x += __shfl_xor(x, sh);
        oa[g][e] = x;
      }
    const bool whole = seg_start == cu.ustart && seg_end == cu.ustart + cu.nblk;
    // partial slot: 0 = unit begun in an earlier range, 1 = continued later
    const int jslot = (seg_start > cu.ustart) ? 0 : 1;
    if (lane < CH) {
      for (int g = 0; g < group; ++g) {
        const float l = xm[GP + g], mg = xm[g];
        const int head = cu.kvh * group + g;
        if (whole && cu.fb > 0) {
          // the rest of this sequence's context is a shared prefix: the
          // combine merges this with the prefix kernel's partials
          const int64_t row = (int64_t)cu.s * p.h_q + head;
          float* dst = p.ws_suf_o + row * D + lane * 8;
          *(f32x4*)dst = f32x4{oa[g][0], oa[g][1], oa[g][2], oa[g][3]};
          *(f32x4*)(dst + 4) = f32x4{oa[g][4], oa[g][5], oa[g][6], oa[g][7]};
          if (lane == 0) {
            p.ws_suf_ml[row * 2 + 0] = mg;
            p.ws_suf_ml[row * 2 + 1] = l;
          }
        } else if (whole) {
          const float inv = 1.f / l;
          T* og = (T*)p.o + ((int64_t)cu.s * p.h_q + head) * D + lane * 8;
          u32x4 wv;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            wv[k] = TT::pack2(oa[g][2 * k] * inv, oa[g][2 * k + 1] * inv);
          *(u32x4*)og = wv;
          if (p.lse != nullptr && lane == 0)
            p.lse[(int64_t)cu.s * p.h_q + head] = (mg + __log2f(l)) * kLn2;
        } else {
          const int64_t slot = ((int64_t)w * 2 + jslot) * group + g;
          float* dst = p.ws_o + slot * D + lane * 8;
          *(f32x4*)dst = f32x4{oa[g][0], oa[g][1], oa[g][2], oa[g][3]};
          *(f32x4*)(dst + 4) = f32x4{oa[g][4], oa[g][5], oa[g][6], oa[g][7]};
          if (lane == 0) {
            p.ws_ml[slot * 2 + 0] = mg;
            p.ws_ml[slot * 2 + 1] = l;
          }
        }
      }
    }
  };

  // ---- stream [b0, b1) through the ring ----
  const int n = (int)(b1 - b0);
  Cursor icur = seek(b0);   // next block to load
  Cursor pcur = icur;       // next block to process
#pragma unroll
  for (int j = 0; j < RING; ++j) {
    issue(icur, j, j < n);
    if (j < n) advance(icur);
  }
  load_q(pcur);
  reset();
  int64_t seg_start = b0;
  // one block: process it, refill its ring slot with the block RING ahead,
  // and close the unit (or this wave's range) when it ends here
  auto step = [&](int k, int j, bool refill) {
    process(pcur, j);
    if (refill) {
      const bool real = k + RING < n;
      issue(icur, j, real);
      if (real) advance(icur);
    }
    if (pcur.lb == pcur.nblk - 1 || k == n - 1) {
      finish(pcur, seg_start, b0 + k + 1);
      if (k + 1 < n) {
        advance(pcur);
        seg_start = b0 + k + 1;
        load_q(pcur);
        reset();
      }
    } else {
      advance(pcur);
    }
  };
  // steady state: every slot is refilled (with an empty load past the end),
  // so the loads are always issued in the same order and each block waits
  // only for its own loads
  int i = 0;
  for (; i + RING <= n; i += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) step(i + j, j, true);
  }
  // the last (fewer than RING) blocks are already in the ring
#pragma unroll
  for (int t = 0; t < RING - 1; ++t)
    if (i + t < n) step(i + t, t, false);
}

// One workgroup of 64 threads per (query head, sequence).  Sequences with an
// empty context get o = 0, lse = -inf.  The others have their partial results
// merged, in this order:
//   * shared-prefix decode: the prefix kernel's partials, one per chunk of the
//     group's prefix;
//   * the sequence's own unit (its blocks past the prefix): nothing if it has
//     none; one partial if it was finished inside one wave (none when there is
//     no prefix either: the split kernel then wrote the output itself);
//     otherwise (w0, slot 1) from the wave where the unit starts, then
//     (w, slot 0) for each following wave up to the one where it ends.  The
//     split kernel recorded w0 and the count.
// Every index comes from one round of loads; lane k then reads the (m, l) of
// partial k while the O rows of the first eight partials are fetched, so a
// merge of up to eight partials costs two dependent memory round trips.
template <typename TT, int D>
__global__ __launch_bounds__(64) void paged_decode_combine_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  constexpr int CPL = D / 64;   // output columns per lane
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int kvh = h / p.group, g = h - kvh * p.group;
  T* og = (T*)p.o + ((int64_t)s * p.h_q + h) * D;
  const int ctx = p.context_lens[s];
  int fb = 0, grp = 0, mi = 0;
  if (p.first_block != nullptr) {
    fb = p.first_block[s];
    grp = p.seq_group[s];
    mi = p.seq_member[s];
  }
  int w0 = 0, nu = 0;
  if (p.ws_unit != nullptr) {
    const int2 ui = *(const int2*)(p.ws_unit + ((int64_t)s * p.h_kv + kvh) * 2);
    w0 = ui.x;
    nu = ui.y;
  }
  if (seq_blocks(ctx) == 0) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) og[lane * CPL + c] = (T)0.f;
    if (p.lse != nullptr && lane == 0) p.lse[(int64_t)s * p.h_q + h] = -INFINITY;
    return;
  }
  const int nb = unit_blocks(ctx, fb);
  // prefix partials: item (group, kvh, query tile, chunk k), query column c
  int n_pre = 0;
  int64_t pre_row0 = 0;
  if (fb > 0) {
    const int qi = mi * p.group + g;
    n_pre = (fb + p.chunk_blocks - 1) / p.chunk_blocks;
    pre_row0 = ((((int64_t)grp * p.h_kv + kvh) * p.n_rt + (qi >> 5)) * p.n_ch) * 32 + (qi & 31);
  }
  const int n_unit = nb > 0 ? nu : 0;
  const bool unit_whole = n_unit == 1;
  if (n_pre == 0 && unit_whole) return;   // finished inside one wave
  const int np = n_pre + n_unit;
  // partial k: its O row and (m, l) pair
  auto part = [&](int k, const float*& o, const float*& ml) {
    int64_t row;
    if (k < n_pre) {
      row = pre_row0 + (int64_t)k * 32;
      o = p.ws_pre_o;
      ml = p.ws_pre_ml;
    } else if (unit_whole) {
      row = (int64_t)s * p.h_q + h;
      o = p.ws_suf_o;
      ml = p.ws_suf_ml;
    } else {
      k -= n_pre;
      row = (k == 0 ? (int64_t)w0 * 2 + 1 : (int64_t)(w0 + k) * 2) * p.group + g;
      o = p.ws_o;
      ml = p.ws_ml;
    }
    o += row * D;
    ml += row * 2;
  };
  auto load_o = [&](int k, float* v) {
    const float *po, *pml;
    part(k, po, pml);
    const float* src = po + lane * CPL;
    if constexpr (CPL == 2) {
      const float2 t = *(const float2*)src;
      v[0] = t.x;
      v[1] = t.y;
    } else {
      v[0] = src[0];
    }
  };
  // (m, l) of partial `lane` and the O rows of partials 0..7 (clamped)
  float mk = -INFINITY, lk = 0.f;
  if (lane < np) {
    const float *po, *pml;
    part(lane, po, pml);
    const float2 v = *(const float2*)pml;
    mk = v.x;
    lk = v.y;
  }
  float v0[8][CPL];
#pragma unroll
  for (int j = 0; j < 8; ++j) load_o(j < np ? j : np - 1, v0[j]);
  // more than 64 partials: lane folds partials lane + 64, lane + 128, ...
  // into an online (m, l); their weights are reloaded in the sum below
  float ml = mk == -INFINITY ? -INFINITY : mk, ll = mk == -INFINITY ? 0.f : lk;
  for (int k = lane + 64; k < np; k += 64) {
    const float *po, *pml;
    part(k, po, pml);
    const float2 v = *(const float2*)pml;
    if (v.x == -INFINITY) continue;   // a chunk with no visible token
    const float mn = fmaxf(ml, v.x);
    ll = ll * fast_exp2(ml - mn) + v.y * fast_exp2(v.x - mn);
    ml = mn;
  }
  float M = ml;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
  float L = ml == -INFINITY ? 0.f : ll * fast_exp2(ml - M);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) L += __shfl_xor(L, sh);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  // O = sum_k 2^(m_k - M) O_k / L, eight partials per round trip
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int c0 = 0; c0 < np; c0 += 64) {
    float mw = mk;   // m of partial c0 + lane; 0 weight marks "none"
    if (c0 > 0) {
      mw = -INFINITY;
      if (c0 + lane < np) {
        const float *po, *pml;
        part(c0 + lane, po, pml);
        mw = pml[0];
      }
    }
    const float wl = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
    const int n = np - c0 < 64 ? np - c0 : 64;
    for (int j0 = 0; j0 < n; j0 += 8) {
      float wk[8], v[8][CPL];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = j0 + j < n ? j0 + j : n - 1;   // clamped: always a valid partial
        wk[j] = j0 + j < n ? __shfl(wl, kk) : 0.f;
        if (c0 == 0 && j0 == 0) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) v[j][c] = v0[j][c];
        } else {
          load_o(c0 + kk, v[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += wk[j] != 0.f ? wk[j] * v[j][c] : 0.f;
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) og[lane * CPL + c] = (T)(acc[c] * inv);
  if (p.lse != nullptr && lane == 0)
    p.lse[(int64_t)s * p.h_q + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// Shared-prefix decode, the prefix part: the sequences of a group read their
// common prefix from the same blocks (tutorial "Chapter 3 Advanced
// principles", section 3.0: shared prefixes are repeated block ids), so each
// prefix block is read once for the whole group instead of once per
// sequence.  One workgroup of four waves per item (group, KV head, tile of 32
// queries, chunk of chunk_blocks prefix blocks); the queries of a tile are the
// (member, head) pairs of the group that read this KV head, member-major.
// Wave w takes blocks w, w + 4, ... of the chunk.  Per block of 16 tokens:
//   * S^T = K Q^T on the matrix cores (16x16x32, two 16-query tiles): K is
//     loaded straight into the A-operand layout, Q^T stays in registers as the
//     B operand; each lane holds one query column and four of its tokens;
//   * online softmax per query column with a lazily raised reference max (it
//     moves only when a score passes it by more than TAU, in log2 units);
//   * the probabilities, rounded to the input type, are already the B
//     operand of O^T += V^T P^T (16x16x16); V goes through LDS to be read
//     transposed (ds_read_b64_tr_b16), four tokens of one column per lane.
// At the end the four waves merge their (m, l, O) in LDS in a fixed order and
// the item writes one partial per query: unnormalised O, m and l.  Tokens at
// or past a query's context length are masked, so a context shorter than the
// prefix is still exact (the prefix blocks must hold real data).
//
// Work item (g, 0, 0, 0) of every group also records each member's prefix
// length in blocks and its group for the split and combine kernels, which run
// after this one.
template <typename TT, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void paged_decode_prefix_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  constexpr int NW = 4;                  // waves per workgroup
  constexpr int KST = D / 32;            // k-steps of S^T = K Q^T (16x16x32)
  constexpr int CH = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROWS = 64 / CH;          // rows per 16-byte load instruction
  constexpr int VST = kDecBS / ROWS;     // V load instructions per block
  constexpr int DT = D / 16;             // 16-row tiles of O^T
  constexpr int RING = 2;                // blocks in flight per wave
  constexpr int OP = D + 4;              // padded row of the merge area (floats)
  constexpr float TAU = 8.0f;
  // LDS: per wave two V staging tiles [16][D] during the loop; afterwards the
  // same memory holds each wave's scaled O [32][OP] for the merge
  constexpr int VBYTES = NW * 2 * kDecBS * D * 2;
  constexpr int OBYTES = NW * 32 * OP * 4;
  __shared__ __attribute__((aligned(16))) char smem[VBYTES > OBYTES ? VBYTES : OBYTES];
  __shared__ __attribute__((aligned(16))) float mls[NW][32][2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int item = blockIdx.x;
  const int ch = item % p.n_ch;
  item /= p.n_ch;
  const int rt = item % p.n_rt;
  item /= p.n_rt;
  const int kvh = item % p.h_kv;
  const int grp = item / p.h_kv;
  const int gs = p.group_starts[grp], ge = p.group_starts[grp + 1];
  // Prefix blocks covered here: whole blocks of the prefix, within the first
  // member's context (its table row is the one read, and every slot of those
  // blocks holds real data) and within the chunks launched.  Whatever is not
  // covered -- also every member past the query tiles launched -- is left to
  // the split kernel, which reads each sequence's own blocks, so a too-small
  // host bound costs speed, not correctness.
  const int ctx0 = ge > gs ? p.context_lens[gs] : 0;
  int pblocks = max(0, min(p.prefix_lens[grp], ctx0)) / kDecBS;
  pblocks = min(pblocks, min(p.n_ch * p.chunk_blocks, p.max_blocks_per_seq));
  if (kvh == 0 && rt == 0 && ch == 0) {
    for (int m = gs + tid; m < ge; m += 256) {
      const bool covered = (int64_t)(m - gs + 1) * p.group <= (int64_t)p.n_rt * 32;
      p.seq_meta[m] = covered ? pblocks : 0;
      p.seq_meta[p.num_seqs + m] = grp;
      p.seq_meta[2 * p.num_seqs + m] = m - gs;
    }
  }
  const int j0 = ch * p.chunk_blocks;
  const int j1 = min(pblocks, j0 + p.chunk_blocks);
  const int rows = (ge - gs) * p.group;
  if (j0 >= j1 || rt * 32 >= rows) return;
  const float c = p.scale_log2;

  // ---- the query columns of this lane: c = qt * 16 + lane % 16 ----
  u32x4 qb[2][KST];
  int ctxq[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = rt * 32 + qt * 16 + (lane & 15);
    const bool valid = qi < rows;
    const int m = valid ? qi / p.group : 0;
    const int s = gs + m;
    const int head = kvh * p.group + (qi - m * p.group);
    ctxq[qt] = valid ? p.context_lens[s] : 0;
    const T* qg = (const T*)p.q + ((int64_t)s * p.h_q + head) * D + (lane >> 4) * 8;
#pragma unroll
    for (int st = 0; st < KST; ++st) {
      qb[qt][st] = u32x4{0, 0, 0, 0};
      if (valid) qb[qt][st] = *(const u32x4*)(qg + 32 * st);
    }
  }

  // ---- loads of one prefix block: K into the A-operand layout (token
  // lane % 16, d = 32 st + 8 (lane / 16)), V rows as they are in memory ----
  const char* kc = (const char*)p.k_cache;
  const char* vc = (const char*)p.v_cache;
  const int64_t blk_bytes = (int64_t)kDecBS * D * 2;
  const uint32_t kl = (uint32_t)((lane & 15) * D + (lane >> 4) * 8) * 2u;
  const uint32_t vl = (uint32_t)((lane / CH) * D + (lane % CH) * 8) * 2u;
  const int mine = (j1 - j0 - w + NW - 1) / NW;   // this wave's blocks: j0 + w + NW i
  const int64_t trow = (int64_t)gs * p.max_blocks_per_seq;
  u32x4 kr[RING][KST], vr[RING][VST];
  // a refill past this wave's blocks uses an empty resource: the loads still
  // issue, in the same order, but return zeros without touching memory
  auto issue = [&](int i, int slot) {
    const bool real = i < mine;
    const char* kb = kc;
    const char* vb = vc;
    if (real) {
      const int64_t phys = ld_meta(p.block_table, trow + j0 + w + NW * i);
      kb += (phys * p.h_kv + kvh) * blk_bytes;
      vb += (phys * p.h_kv + kvh) * blk_bytes;
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, real ? (uint32_t)blk_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, real ? (uint32_t)blk_bytes : 0u);
#pragma unroll
    for (int st = 0; st < KST; ++st) kr[slot][st] = buf_load16(rk, kl + st * 64);
#pragma unroll
    for (int st = 0; st < VST; ++st) vr[slot][st] = buf_load16(rv, vl + st * ROWS * D * 2);
  };

  // ---- LDS V staging, [token][d] with 16-byte chunk c of row r stored at
  // c ^ vsw(r), so that the transposing reads of 16 rows hit distinct banks ----
  uint16_t* vst = (uint16_t*)smem + w * 2 * kDecBS * D;
  auto vsw = [](int r) { return (2 * r) & (CH - 1); };
  const int vw_row = lane / CH, vw_chunk = lane % CH;
  // transposing read of O^T tile dt: within each 16-lane group (g4 = lane / 16)
  // lane i = 4 j + q points at token 4 g4 + j, columns 16 dt + 4 q .. + 3;
  // the read leaves lane i with tokens 4 g4 .. 4 g4 + 3 of column 16 dt + i
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2), tr_q = lane & 3;
  auto tr_ofs = [&](int dt) {
    return tr_row * D + (((2 * dt + (tr_q >> 1)) ^ vsw(tr_row)) * 8) + (tr_q & 1) * 4;
  };

  float m_ref[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};
  f32x4 oacc[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt][0] = oacc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](int i, int slot) {
    const int j = j0 + w + NW * i;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < KST; ++st)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) acc[qt] = TT::mma16(kr[slot][st], qb[qt][st], acc[qt]);
    // lane: query column qt * 16 + lane % 16, tokens tb + r
    const int tb = j * kDecBS + 4 * (lane >> 4);
    float sc[2][4];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[qt][r] = tb + r < ctxq[qt] ? acc[qt][r] * c : -INFINITY;
        grow = grow || sc[qt][r] > m_ref[qt] + TAU;
      }
    // ---- rare: a score passed its column's reference by more than TAU ----
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float bm = fmaxf(fmaxf(sc[qt][0], sc[qt][1]), fmaxf(sc[qt][2], sc[qt][3]));
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const bool up = bm > m_ref[qt] + TAU;
        const float alpha = fast_exp2(up ? m_ref[qt] - bm : 0.f);
        m_ref[qt] = up ? bm : m_ref[qt];
        l_part[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
      }
    }
    // probabilities relative to the reference, rounded as they enter P V
    u32x2 pb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float mm = m_ref[qt] == -INFINITY ? 0.f : m_ref[qt];
      pb[qt].x = TT::pack2(fast_exp2(sc[qt][0] - mm), fast_exp2(sc[qt][1] - mm));
      pb[qt].y = TT::pack2(fast_exp2(sc[qt][2] - mm), fast_exp2(sc[qt][3] - mm));
      l_part[qt] = TT::sum2(pb[qt].y, TT::sum2(pb[qt].x, l_part[qt]));
    }
    // V to LDS, then O^T += V^T P^T
    uint16_t* vt = vst + (i & 1) * kDecBS * D;
    lds_order();
#pragma unroll
    for (int st = 0; st < VST; ++st) {
      const int r = st * ROWS + vw_row;
      *(u32x4*)(vt + r * D + ((vw_chunk ^ vsw(r)) * 8)) = vr[slot][st];
    }
    lds_order();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vt + tr_ofs(dt))));
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) oacc[dt][qt] = TT::mma16k16(a, pb[qt], oacc[dt][qt]);
    }
  };

  // ---- stream this wave's blocks through the ring ----
#pragma unroll
  for (int r = 0; r < RING; ++r) issue(r, r);
  int i = 0;
  for (; i + RING <= mine; i += RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      process(i + r, r);
      issue(i + r + RING, r);
    }
  }
#pragma unroll
  for (int r = 0; r < RING - 1; ++r)
    if (i + r < mine) process(i + r, r);

  // ---- merge the four waves: M = max m_w, O = sum 2^(m_w - M) O_w ----
  float l_col[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float x = l_part[qt];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    l_col[qt] = x;
  }
  __syncthreads();   // every wave is done with its V staging
  if (lane < 16) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      mls[w][qt * 16 + lane][0] = m_ref[qt];
      mls[w][qt * 16 + lane][1] = l_col[qt];
    }
  }
  __syncthreads();
  float* mo = (float*)smem;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int col = qt * 16 + (lane & 15);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, mls[v][col][0]);
    const float f = m_ref[qt] == -INFINITY ? 0.f : fast_exp2(m_ref[qt] - M);
    float* dst = mo + (w * 32 + col) * OP + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *(f32x4*)(dst + 16 * dt) = oacc[dt][qt] * f;
  }
  __syncthreads();
  // wave w writes query columns 8 w .. 8 w + 7: 8 lanes per column, D / 8
  // consecutive floats per lane
  {
    constexpr int PL = D / 8;
    const int col = w * 8 + (lane >> 3), d0 = (lane & 7) * PL;
    if (rt * 32 + col < rows) {
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < NW; ++v) M = fmaxf(M, mls[v][col][0]);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float mv = mls[v][col][0];
        L += mv == -INFINITY ? 0.f : mls[v][col][1] * fast_exp2(mv - M);
      }
      const int64_t row = ((((int64_t)grp * p.h_kv + kvh) * p.n_rt + rt) * p.n_ch + ch) * 32 + col;
      float* dst = p.ws_pre_o + row * D + d0;
#pragma unroll
      for (int e = 0; e < PL; e += 4) {
        f32x4 x = *(const f32x4*)(mo + col * OP + d0 + e);
#pragma unroll
        for (int v = 1; v < NW; ++v) x += *(const f32x4*)(mo + (v * 32 + col) * OP + d0 + e);
        *(f32x4*)(dst + e) = x;
      }
      if ((lane & 7) == 0) {
        p.ws_pre_ml[row * 2 + 0] = M;
        p.ws_pre_ml[row * 2 + 1] = L;
      }
    }
  }
}

// Persistent waves for these sizes: one per block of the largest possible
// list, at most kDecMaxWaves.
int decode_waves(int num_seqs, int h_kv, int max_context_len) {
  const int64_t tmax = (int64_t)num_seqs * h_kv * ((max_context_len + kDecBS - 1) / kDecBS);
  return (int)(tmax < kDecMaxWaves ? (tmax > 0 ? tmax : 1) : kDecMaxWaves);
}

size_t decode_workspace_bytes(int num_seqs, int h_q, int h_kv, int head_dim, int max_context_len) {
  if (num_seqs <= 0 || h_q <= 0 || h_kv <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      h_q % h_kv != 0)
    return 0;
  const int64_t slots = (int64_t)decode_waves(num_seqs, h_kv, max_context_len) * 2 * (h_q / h_kv);
  // partial O rows, their (m, l) pairs, then (first wave, wave count) per unit
  return (size_t)(slots * head_dim * 4 + slots * 2 * 4 + (int64_t)num_seqs * h_kv * 2 * 4);
}

template <typename TT, int D, int GP>
static hipError_t launch_decode_t(const DecodeParams& p, int W, hipStream_t stream) {
  // One block of K and V (8 KiB at d = 128) in flight per wave: the next
  // block's loads go out as soon as this one is processed, and the two waves
  // of each SIMD keep about 16 MB in flight over the chip.  A two-block ring
  // (32 MB in flight) measured 2% slower.
  constexpr int RING = 1;
  // as many waves as are resident at once (one per SIMD when GP x D > 512),
  // so that no wave waits for another to finish before it starts
  if (GP * D > 512 && W > kDecMaxWaves / 2) W = kDecMaxWaves / 2;
  hipLaunchKernelGGL((paged_decode_split_kernel<TT, D, GP, RING>), dim3(W), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((paged_decode_combine_kernel<TT, D>), dim3(p.h_q, p.num_seqs), dim3(64), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename TT>
static hipError_t launch_decode_d(const DecodeParams& p, int W, hipStream_t stream) {
  const int gp = p.group <= 4 ? 4 : (p.group <= 8 ? 8 : 16);
  if (p.head_dim == 64) {
    if (gp == 4) return launch_decode_t<TT, 64, 4>(p, W, stream);
    if (gp == 8) return launch_decode_t<TT, 64, 8>(p, W, stream);
    return launch_decode_t<TT, 64, 16>(p, W, stream);
  }
  if (gp == 4) return launch_decode_t<TT, 128, 4>(p, W, stream);
  if (gp == 8) return launch_decode_t<TT, 128, 8>(p, W, stream);
  return launch_decode_t<TT, 128, 16>(p, W, stream);
}

hipError_t launch_decode(int dtype, const DecodeParams& p, int max_context_len,
                         hipStream_t stream) {
  const int W = decode_waves(p.num_seqs, p.h_kv, max_context_len);
  if (dtype == 2) return launch_decode_d<BF16>(p, W, stream);
  return launch_decode_d<F16>(p, W, stream);
}

// Shared-prefix decode: how the prefix work is cut.  Query tiles of 32 cover
// the largest group; chunks are sized so that the largest possible prefix
// work gives about 512 workgroups (two per CU), with 8 to 64 blocks per
// chunk (a multiple of the 4 waves).
SharedPlan shared_plan(int num_groups, int max_group_size, int h_q, int h_kv,
                       int max_prefix_len) {
  SharedPlan pl{};
  const int64_t rows = (int64_t)max_group_size * (h_q / h_kv);
  pl.n_rt = (int)std::max<int64_t>(1, (rows + 31) / 32);
  const int64_t pb = std::max(0, max_prefix_len) / kDecBS;
  const int64_t total = (int64_t)num_groups * h_kv * pl.n_rt * pb;
  int64_t cb = (total + 511) / 512;
  cb = (cb + 3) / 4 * 4;
  pl.chunk_blocks = (int)std::min<int64_t>(64, std::max<int64_t>(8, cb));
  pl.n_ch = (int)std::max<int64_t>(1, (pb + pl.chunk_blocks - 1) / pl.chunk_blocks);
  pl.items = (int64_t)num_groups * h_kv * pl.n_rt * pl.n_ch;
  return pl;
}

template <typename TT>
static hipError_t launch_prefix_d(const DecodeParams& p, int64_t items, hipStream_t stream) {
  if (p.head_dim == 64)
    hipLaunchKernelGGL((paged_decode_prefix_kernel<TT, 64>), dim3((unsigned)items), dim3(256), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((paged_decode_prefix_kernel<TT, 128>), dim3((unsigned)items), dim3(256), 0,
                       stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_shared(int dtype, const DecodeParams& p, int64_t items,
                                int max_context_len, hipStream_t stream) {
  const hipError_t e = dtype == 2 ? launch_prefix_d<BF16>(p, items, stream)
                                  : launch_prefix_d<F16>(p, items, stream);
  if (e != hipSuccess) return e;
  return launch_decode(dtype, p, max_context_len, stream);
}

}  // namespace attn
