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
#include "common.h"

namespace attn {

constexpr int kDecBS = 16;          // tokens per KV block
constexpr int kDecMaxWaves = 2048;  // persistent waves: 8 per CU on 256 CUs (2 per SIMD)

// Blocks of a sequence (one unit per KV head).
__device__ inline int seq_blocks(int ctx) { return ctx > 0 ? (ctx + kDecBS - 1) / kDecBS : 0; }

// Range of wave w in the flattened block list: [w T / W, (w + 1) T / W).
__device__ inline int64_t range_start(int w, int64_t T, int W) { return (int64_t)w * T / W; }

// The wave whose range holds block b (0 <= b < T): the last w whose range
// starts at or before b.
__device__ inline int wave_of(int64_t b, int64_t T, int W) {
  int w = (int)(b * W / T);   // range_start(w) <= b already
  while (w + 1 < W && range_start(w + 1, T, W) <= b) ++w;
  return w;
}

// Read-only metadata (context lengths, block table) is read through the
// constant address space: at a wave-uniform index that is a scalar load, which
// keeps the cursor in scalar registers and lets the vector-memory counter track
// K/V loads only.
__device__ inline int ld_meta(const int32_t* ptr, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)ptr)[i];
}

// Total blocks over all sequences and the blocks of sequences before `s`,
// reduced across the 64 lanes of the calling wave (the results are uniform).
__device__ inline void seq_block_sums(const DecodeParams& p, int s, int lane, int64_t& before,
                                      int64_t& total) {
  before = 0;
  total = 0;
  for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
    const int ss = s0 + lane;
    const int nb = (ss < p.num_seqs) ? seq_blocks(p.context_lens[ss]) : 0;
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

  const int w = blockIdx.x, W = gridDim.x;
  const int lane = threadIdx.x;
  const int group = p.group;
  const float c = p.scale_log2;

  int64_t unused_before, total_seq_blocks;
  seq_block_sums(p, 0, lane, unused_before, total_seq_blocks);
  const int64_t nlist = total_seq_blocks * p.h_kv;   // blocks in the list
  if (nlist == 0) return;
  const int64_t b0 = range_start(w, nlist, W), b1 = range_start(w + 1, nlist, W);
  if (b0 >= b1) return;

  // position in the unit list: unit (s, kvh), its blocks and context, the
  // list position of its first block and the block within it
  struct Cursor {
    int s, kvh, nblk, ctx;
    int64_t ustart;
    int lb;
  };
  // list position b -> cursor: the sequences' list spans are prefix-summed
  // across the wave, 64 sequences per round of loads, and the lane whose span
  // holds b is picked by a ballot
  auto seek = [&](int64_t b) {
    Cursor cu{};
    int64_t base = 0;
    for (int s0 = 0; s0 < p.num_seqs; s0 += 64) {
      const int ss = s0 + lane;
      const int ctx = ss < p.num_seqs ? p.context_lens[ss] : 0;
      const int64_t span = (int64_t)seq_blocks(ctx) * p.h_kv;
      int64_t incl = span;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) {
        const int64_t t = __shfl_up(incl, sh);
        if (lane >= sh) incl += t;
      }
      const int64_t lo = base + incl - span;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(span > 0 && b >= lo && b < lo + span);
      if (hit != 0) {
        const int l = (int)__builtin_ctzll(hit);
        cu.s = s0 + l;
        cu.ctx = __builtin_amdgcn_readlane(ctx, l);
        cu.nblk = seq_blocks(cu.ctx);
        const int64_t pos = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(lo >> 32), l) << 32) |
                                      (uint32_t)__builtin_amdgcn_readlane((int)lo, l));
        cu.kvh = (int)((b - pos) / cu.nblk);
        cu.ustart = pos + (int64_t)cu.kvh * cu.nblk;
        cu.lb = (int)(b - cu.ustart);
        return cu;
      }
      const int64_t tot = __shfl(incl, 63);
      base += (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(tot >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)tot));
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
      cu.ctx = (cu.s < p.num_seqs) ? ld_meta(p.context_lens, cu.s) : 1;
      cu.nblk = seq_blocks(cu.ctx);
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
  // tile (scalar base, every lane offset inside it).  A refill past the end of
  // the range uses an empty resource: the loads still issue, in the same
  // order, but return zeros without touching memory.
  auto issue = [&](const Cursor& cu, int slot, bool real) {
    const char* kb = kc;
    const char* vb = vc;
    if (real) {
      const int64_t phys = ld_meta(p.block_table, (int64_t)cu.s * p.max_blocks_per_seq + cu.lb);
      kb += (phys * p.h_kv + cu.kvh) * blk_bytes;
      vb += (phys * p.h_kv + cu.kvh) * blk_bytes;
    }
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, real ? (uint32_t)blk_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, real ? (uint32_t)blk_bytes : 0u);
#pragma unroll
    for (int st = 0; st < KST; ++st) kr[slot][st] = buf_load16(rk, kl + st * 64);
#pragma unroll
    for (int st = 0; st < VST; ++st)
      vr[slot][st] = buf_load16(rv, vl + ((st & 1) + (st >> 1) * 2 * ROWS) * D * 2);
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
    const int tbase = cu.lb * kDecBS;
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
        if (whole) {
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
// empty context get o = 0, lse = -inf; units cut by range boundaries get their
// partials merged: (w0, slot 1) from the wave where the unit starts, then
// (w, slot 0) for the following waves up to the one where it ends.  Lane k
// reads the (m, l) of partial k; the weights 2^(m_k - M) are then broadcast
// and the O rows of eight partials are loaded at once, so the whole merge
// costs a few dependent memory round trips whatever the number of partials.
template <typename TT, int D>
__global__ __launch_bounds__(64) void paged_decode_combine_kernel(DecodeParams p, int W) {
  typedef typename TT::elem T;
  constexpr int CPL = D / 64;   // output columns per lane
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int kvh = h / p.group, g = h - kvh * p.group;
  T* og = (T*)p.o + ((int64_t)s * p.h_q + h) * D;
  const int nb = seq_blocks(p.context_lens[s]);
  if (nb == 0) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) og[lane * CPL + c] = (T)0.f;
    if (p.lse != nullptr && lane == 0) p.lse[(int64_t)s * p.h_q + h] = -INFINITY;
    return;
  }
  int64_t before, total;
  seq_block_sums(p, s, lane, before, total);
  const int64_t T_ = total * p.h_kv;
  const int64_t ustart = before * p.h_kv + (int64_t)kvh * nb;
  const int w0 = wave_of(ustart, T_, W), w1 = wave_of(ustart + nb - 1, T_, W);
  if (w0 == w1) return;   // finished inside one wave
  const int np = w1 - w0 + 1;
  // waves with an empty range (more waves than blocks) hold no partial
  auto has_part = [&](int k) {
    return k == 0 || range_start(w0 + k, T_, W) < range_start(w0 + k + 1, T_, W);
  };
  auto slot_of = [&](int k) -> int64_t {
    return k == 0 ? ((int64_t)w0 * 2 + 1) * p.group + g : ((int64_t)(w0 + k) * 2) * p.group + g;
  };
  // pass 1: per-lane online merge of (m, l) over partials lane, lane + 64, ...
  float ml = -INFINITY, ll = 0.f;
  for (int k = lane; k < np; k += 64) {
    if (!has_part(k)) continue;
    const float2 v = *(const float2*)(p.ws_ml + slot_of(k) * 2);
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
  const float inv = 1.f / L;
  // pass 2: O = sum_k 2^(m_k - M) O_k / L, eight partials per round trip
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int c0 = 0; c0 < np; c0 += 64) {
    const int k = c0 + lane;
    float wl = 0.f;   // 0 marks "no partial": such slots are skipped, not scaled
    if (k < np && has_part(k)) wl = fast_exp2(p.ws_ml[slot_of(k) * 2] - M);
    const int n = np - c0 < 64 ? np - c0 : 64;
    for (int j0 = 0; j0 < n; j0 += 8) {
      float wk[8], v[8][CPL];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = j0 + j < n ? j0 + j : n - 1;   // clamped: always a valid slot
        wk[j] = j0 + j < n ? __shfl(wl, kk) : 0.f;
        const float* src = p.ws_o + slot_of(c0 + kk) * D + lane * CPL;
        if constexpr (CPL == 2) {
          const float2 t = *(const float2*)src;
          v[j][0] = t.x;
          v[j][1] = t.y;
        } else {
          v[j][0] = src[0];
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
  if (p.lse != nullptr && lane == 0) p.lse[(int64_t)s * p.h_q + h] = (M + __log2f(L)) * kLn2;
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
  return (size_t)(slots * head_dim * 4 + slots * 2 * 4);
}

template <typename TT, int D, int GP>
static hipError_t launch_decode_t(const DecodeParams& p, int W, hipStream_t stream) {
  constexpr int RING = 2;
  // as many waves as are resident at once (one per SIMD when GP x D > 512),
  // so that no wave waits for another to finish before it starts
  if (GP * D > 512 && W > kDecMaxWaves / 2) W = kDecMaxWaves / 2;
  hipLaunchKernelGGL((paged_decode_split_kernel<TT, D, GP, RING>), dim3(W), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((paged_decode_combine_kernel<TT, D>), dim3(p.h_q, p.num_seqs), dim3(64), 0,
                     stream, p, W);
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

}  // namespace attn
