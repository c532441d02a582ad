// Prefill kernels: exact attention O = softmax(Q K^T * scale) V in one fused,
// tiled pass with the online-softmax update ("Other people's interview
// notes", question "explain FlashAttention", part 2), never writing the
// N x N score or probability matrix to device memory.
//
// 16-bit kernel (bf16 / fp16), gfx950 matrix cores:
//   * a workgroup of 8 waves owns 256 query rows: 128 rows of each of two
//     query heads that read the same KV head (GQA), or 256 rows of one head.
//     Each wave owns 32 rows, whose Q fragment stays in VGPRs for the whole
//     kernel.  Every K/V tile staged in LDS serves all 256 rows, which halves
//     the L2-to-LDS traffic of a 128-row workgroup;
//   * the loop walks the visible key range in BN = 64 tiles.  K and V tiles
//     go from memory straight into LDS (buffer loads with the LDS bit), laid
//     out [key][d] with 16-byte chunks permuted per row against bank
//     conflicts; the K operand is one 16-byte LDS read per lane, the V
//     operand two transposing 8-byte reads.  Two stages: tile j+1 lands while
//     tile j is computed.  The stages are separate LDS arrays, so the
//     compiler can see that a stage being read is not the one being filled;
//   * scores are produced transposed, S^T = K Q^T (v_mfma_f32_32x32x16), so
//     every lane holds one query column and 16 of its keys; the row max needs
//     one exchange with lane l^32 and nothing else.  The same registers, once
//     exponentiated and rounded, are directly the B operand of
//     O^T = V^T P^T, which leaves each lane owning one query's output column:
//     the rescale by exp(m_old - m_new) is a per-lane multiply;
//   * softmax runs in the exp2 domain with scale*log2(e) folded into one
//     multiply; l is kept per lane and summed with lane l^32 at the end;
//     O is divided by l once, in the epilogue;
//   * causal: only the key tiles a workgroup can see are visited, the mask is
//     applied only on tiles that cross the diagonal, a wave stops computing
//     once every later key is masked for all of its rows, and workgroups are
//     issued longest first.  Work items that share K/V (the query heads of
//     one GQA group) are kept together on one XCD.
//
// fp32 kernel: plain fp32 arithmetic on the vector ALUs (the fp32 matrix
// rate equals the vector rate on this chip); four lanes share a query row.
#include "common.h"
#include "schedule.h"

namespace attn {

// ----------------------------------------------------------------------------
// 16-bit matrix-core kernel
// ----------------------------------------------------------------------------
// PAGED: K and V are read from a paged KV cache ([blocks][h_kv][16][D])
// through each sequence's block table, its context length sets n_k, and the
// n_q query rows are the last n_q tokens of that context.
// NW waves per workgroup, 32 query rows each.  The workgroup's 32 NW rows
// are p.hpw heads (of one KV head's group) x bm = 32 NW / p.hpw consecutive
// query rows; all of them read the same K/V tiles, so each tile staged in LDS
// serves 32 NW rows.
template <typename TT, int D, bool CAUSAL, bool PAGED, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma_kernel(FwdParams p) {
  typedef typename TT::elem T;
  constexpr int NT = 64 * NW;             // threads
  constexpr int BN = 64;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int TILE = BN * D;            // elements per K or V tile (no padding)
  constexpr int LOADS = BN * CPR / NT;    // 16-byte direct loads per thread per tile
  constexpr int QT = 32 * NW / BN;        // BN-row tiles of the workgroup's Q rows
  constexpr int NS = D / 16;              // k-steps of one S^T half (8 for d = 128)
  constexpr int NQK = 2 * NS;             // QK matrix ops per tile
  constexpr int NPV = (D / 32) * (BN / 16);  // PV matrix ops per tile
  constexpr int PFD = 3;                  // LDS operand prefetch distance, in slots
  // Probabilities are taken relative to a per-row reference m that moves
  // only when it has to (the division by l in the epilogue uses the same
  // reference, so the result does not depend on it): when a row's maximum
  // exceeds m by more than GROW (log2 units), m is set to that maximum plus
  // HEAD and O and l are rescaled; until then every probability stays below
  // 2^GROW.  For bf16 (fp32 exponent range) the headroom lets the maximum
  // rise by HEAD + GROW before the next rescale: probabilities are at most
  // 2^-HEAD relative to m's maximum, and terms more than HEAD + 66 below the
  // row maximum, which flush to zero, weigh less than 2^-52 in total.  fp16
  // probabilities must stay in fp16 range, so there m is the maximum itself.
  constexpr float HEAD = TT::kIsBf16 ? 60.f : 0.f;
  constexpr float GROW = TT::kIsBf16 ? 40.f : 8.f;
  static_assert(LOADS * NT == BN * CPR, "tile split");
  static_assert(QT == 2 || QT == 4, "Q staging");
  static_assert(32 % (NQK + NPV) == 0, "slot plan");
  // One array per stage: the tile loads write LDS directly, and the compiler
  // only knows that a stage being read is not the one being filled when they
  // are distinct objects (otherwise it waits for the loads before each read).
  __shared__ __attribute__((aligned(16))) uint16_t ks_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ks_lds1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vs_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vs_lds1[TILE];
  auto kst = [&](int st) -> uint16_t* { return st ? ks_lds1 : ks_lds0; };
  auto vst = [&](int st) -> uint16_t* { return st ? vs_lds1 : vs_lds0; };
  // Q tiles 2 and 3 (eight waves) are staged here, tiles 0 and 1 in the V stages
  __shared__ __attribute__((aligned(16))) uint16_t qx_lds[QT > 2 ? (QT - 2) * TILE : 8];
  auto qst = [&](int t) -> uint16_t* { return t < 2 ? vst(t) : qx_lds + (t - 2) * TILE; };
  // paged: this sequence's block table row, staged once so that the tile
  // loads do not wait on table reads from memory
  constexpr int kTabLds = PAGED ? 2048 : 1;
  __shared__ __attribute__((aligned(16))) int32_t tab_lds[kTabLds < 4 ? 4 : kTabLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int col = lane & 31;   // query column of this lane
  const int hi = lane >> 5;    // which half of the k slots / key rows

  const int item = remap_item(blockIdx.x, p.num_items, p.xcd_chunk);
  const int hpw = p.hpw;                  // heads of this workgroup
  const int bm = 32 * NW / hpw;           // query rows per head
  const int wph = NW / hpw;               // waves per head
  const int hgroups = p.h_q / hpw;
  const int bh = p.batch * hgroups;
  const int rank = item / bh;
  const int rem = item - rank * bh;
  const int b = rem / hgroups;
  const int h0 = (rem - b * hgroups) * hpw;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - rank) : rank;
  const int q0 = qt * bm;
  const int kvh = h0 / p.group;
  // This wave's 32 rows are row block rb of the workgroup's list (head
  // h0 + rb / wph, query rows q0 + 32 (rb % wph) ...).  The waves sharing a
  // SIMD (w and w + NW/2) take blocks rb and NW - 1 - rb, so that under a
  // causal mask each SIMD gets an equal share of the key tiles the waves
  // skip.
  const int rb = wave < NW / 2 ? wave : 3 * NW / 2 - 1 - wave;
  const int h = h0 + rb / wph;
  const int wr0 = q0 + (rb % wph) * 32;
  // keys of this sequence
  const int nk = PAGED ? __builtin_amdgcn_readfirstlane(p.context_lens[b]) : p.n_k;
  const int off = nk - p.n_q;

  int kend = nk;
  if (CAUSAL) {
    const int qlast = min(q0 + bm, p.n_q) - 1;
    kend = min(nk, max(0, qlast + off + 1));
  }
  const int ntiles = (kend + BN - 1) / BN;

  const T* Kg = (const T*)p.k + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const T* Vg = (const T*)p.v + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  // row pitch, bytes (paged: rows of one block of one KV head are contiguous)
  const uint32_t krow = PAGED ? (uint32_t)D * 2u : (uint32_t)p.ks_n * 2u;
  const uint32_t vrow = PAGED ? (uint32_t)D * 2u : (uint32_t)p.vs_n * 2u;

  // Q fragment (B operand of S^T = K Q^T): column = query, k = d.  Filled
  // in the prologue through LDS (see below).
  const int qrow = wr0 + col;
  u32x4 qf[NS];

  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY;  // reference max, log2 units (same in lanes l, l^32)
  float l_run = 0.f;        // running sum over this lane's keys
  const float c = p.scale_log2;

  // ---- tiles go HBM -> LDS directly (no registers) ----
  // LDS tile layout: row-major, 16-byte chunks permuted within each row so
  // that the column-wise operand reads hit distinct banks:
  //   K: chunk c of row r sits at c ^ (r % 16)   (16 rows x 1 chunk per read)
  //   V: chunk c of row r sits at c ^ 4 (r % 4)  (4 rows x 4 chunks per read
  //                                                of 32 lanes)
  // A direct load writes 64 consecutive 16-byte LDS slots per wave
  // instruction, so every lane fetches the global chunk that belongs in its
  // slot.
  auto kswz = [](int r) { return (r & 15) & (CPR - 1); };
  auto vswz = [](int r) { return (4 * (r & 3)) & (CPR - 1); };
  uint32_t kgo[LOADS], vgo[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int row = slot / CPR, pc = slot % CPR;
    // paged: offsets within the row's 16-row block (tiles start on block edges)
    const int brow = PAGED ? (row & 15) : row;
    kgo[i] = (uint32_t)brow * krow + (uint32_t)((pc ^ kswz(row)) * 16);
    vgo[i] = (uint32_t)brow * vrow + (uint32_t)((pc ^ vswz(row)) * 16);
  }
  // Paged: the rows of one direct-load instruction (64 / CPR of them) lie in
  // one 16-row block, so each instruction gets a resource based at its block
  // of this KV head, whose extent stops at the context (later slots, and
  // blocks past the last, read as zero).
  const int nblk = (nk + 15) >> 4;
  // The four blocks of tile kt are table entries 4 kt .. 4 kt + 3: one
  // 16-byte read of the staged row (or of the table, past the staged part).
  auto tile_blocks = [&](int kt) -> i32x4 {
    const int lb0 = kt * (BN / 16);
    if (lb0 + 4 <= kTabLds) return *(const i32x4*)(tab_lds + lb0);
    i32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = lb0 + j < nblk ? ld_meta(p.block_table, (int64_t)b * p.max_blocks_per_seq + lb0 + j) : 0;
    return r;
  };
  auto tile_ids = [&](int kt) -> i32x4 {
    if constexpr (PAGED) return tile_blocks(kt);
    return i32x4{0, 0, 0, 0};
  };
  auto block_rsrc = [&](const void* cache, int lb, int phys) {
    const char* base = (const char*)cache;
    uint32_t ext = 0;
    if (lb < nblk) {
      base += ((int64_t)__builtin_amdgcn_readfirstlane(phys) * p.h_kv + kvh) * 16 * D * 2;
      ext = (uint32_t)min(16, nk - lb * 16) * (uint32_t)D * 2u;
    }
    return make_rsrc(base, __builtin_amdgcn_readfirstlane(ext));
  };
  // Per-lane offsets stay fixed; each tile gets a buffer resource based at its
  // first row (scalar arithmetic) whose extent is what is left of the slice,
  // so rows past n_k load as zero.  Paged: `ids` are the tile's block ids
  // (tile_blocks), read by the caller before the barrier that precedes the
  // loads, so that the barrier's wait covers the table read.
  auto load_k = [&](int kt, int stage, const i32x4 ids) {
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        // block of this instruction's rows (64 / CPR of them)
        const int j = (i * NW + (wave & (NW - 1))) * (64 / CPR) / 16;
        buf_load16_lds(block_rsrc(p.k, kt * (BN / 16) + j, ids[j]),
                       kst(stage) + (i * NW + wave) * 512, kgo[i]);
      }
      return;
    }
    const uint32_t o = (uint32_t)(kt * BN) * krow;
    const uint32_t rem_b = __builtin_amdgcn_readfirstlane(p.k_bytes > o ? p.k_bytes - o : 0u);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr((const char*)Kg + o), rem_b);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) buf_load16_lds(r, kst(stage) + (i * NW + wave) * 512, kgo[i]);
  };
  // The workgroup's Q rows (QT tiles of BN rows, each of one head) go
  // through the V stages, which are idle until the first tile, and qx_lds:
  // in the K layout, loaded the same coalesced way (rows past n_q read as
  // zero).
  const uint32_t qrowb = (uint32_t)p.qs_n * 2u;
  auto load_q = [&](int t) {
    const int ht = h0 + (t * BN) / bm;
    const T* Qg = (const T*)p.q + (int64_t)b * p.qs_b + (int64_t)ht * p.qs_h;
    const uint32_t o = (uint32_t)(q0 + (t * BN) % bm) * qrowb;
    const uint32_t rem_b = __builtin_amdgcn_readfirstlane(p.q_bytes > o ? p.q_bytes - o : 0u);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr((const char*)Qg + o), rem_b);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int row = slot / CPR, pc = slot % CPR;
      buf_load16_lds(r, qst(t) + (i * NW + wave) * 512,
                     (uint32_t)row * qrowb + (uint32_t)((pc ^ kswz(row)) * 16));
    }
  };
  auto load_v = [&](int kt, int stage, const i32x4 ids) {
    if constexpr (PAGED) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int j = (i * NW + (wave & (NW - 1))) * (64 / CPR) / 16;
        buf_load16_lds(block_rsrc(p.v, kt * (BN / 16) + j, ids[j]),
                       vst(stage) + (i * NW + wave) * 512, vgo[i]);
      }
      return;
    }
    const uint32_t o = (uint32_t)(kt * BN) * vrow;
    const uint32_t rem_b = __builtin_amdgcn_readfirstlane(p.v_bytes > o ? p.v_bytes - o : 0u);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr((const char*)Vg + o), rem_b);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) buf_load16_lds(r, vst(stage) + (i * NW + wave) * 512, vgo[i]);
  };
  // Direct loads complete into LDS asynchronously: wait for them, then
  // barrier, before any wave reads the stage.
  auto wait_loads_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- LDS read addresses, fixed per lane (elements) ----
  // K operand of S^T = K Q^T, k-step s: row col (+32 for the second half),
  // logical chunk 2s + hi.
  int kofs[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kofs[s] = col * D + (((2 * s + hi) ^ kswz(col)) * 8);
  // V operand of O^T = V^T P^T through the transposing LDS read: within each
  // group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces
  // loaded by lanes 4j + i/4 (j = 0..3).  Lane 4j + q of the group therefore
  // points at key (slot base + j) and d (group base + 4q); every lane ends up
  // with four keys of one d column.  Keys of the second read are 8 further;
  // k-steps add 16 rows.  (Row offsets that are multiples of 4 leave the
  // swizzle unchanged, so they fold into immediates.)
  const int vi = lane & 15, vg = lane >> 4;
  const int v_row0 = (vg >> 1) * 4 + (vi >> 2);
  int vofs[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const int el = t * 32 + (vg & 1) * 16 + (vi & 3) * 4;
    vofs[t] = v_row0 * D + ((((el >> 3) ^ vswz(v_row0)) * 8) + (el & 7));
  }

  // last key visible to this lane's query, clamped to the sequence
  const int klast = CAUSAL ? min(qrow + off, nk - 1) : nk - 1;
  // last key tile holding a key that one of this wave's rows sees (-1: none);
  // the wave skips the products of later tiles (their probabilities are 0)
  int last_w = wr0 < p.n_q ? ntiles - 1 : -1;
  if (CAUSAL && last_w >= 0) {
    const int kmax = min(min(wr0 + 31, p.n_q - 1) + off, nk - 1);
    last_w = kmax < 0 ? -1 : min(last_w, kmax / BN);
  }
  last_w = __builtin_amdgcn_readfirstlane(last_w);   // uniform: the loop exits below are per wave

  if (ntiles > 0) {
    if constexpr (PAGED) {
      const int n = min(nblk, kTabLds);
      for (int i = tid; i < n; i += NT)
        tab_lds[i] = p.block_table[(int64_t)b * p.max_blocks_per_seq + i];
      __syncthreads();
    }
    // ---- prologue: Q through LDS, K_0 and K_1 staged, S_0 ----
#pragma unroll
    for (int t = 0; t < QT; ++t) load_q(t);
    load_k(0, 0, tile_ids(0));
    load_k(1, 1, tile_ids(1));
    wait_loads_and_sync();
    {
      // this wave's 32 rows sit in Q tile rb / 2, rows 32 (rb % 2) + ...
      const uint16_t* qb = qst(rb >> 1) + (rb & 1) * 32 * D;
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4*)(qb + kofs[s]);
    }
    f32x16 st_cur[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st_cur[sub][r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        st_cur[sub] = TT::mma32(*(const u32x4*)(ks_lds0 + sub * 32 * D + kofs[s]), qf[s], st_cur[sub]);
    }
    float smax_cur = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax_cur = fmaxf(smax_cur, st_cur[sub][r]);
    u32x4 pb_prev[4];   // P_{kt-1}, the B operand of its P V
#pragma unroll
    for (int i = 0; i < 4; ++i) pb_prev[i] = u32x4{0, 0, 0, 0};
    float pend_alpha = 1.f;
    bool pend_grow = false;
    // every wave holds its Q fragment (read from the V stages) and is done
    // with K stage 0 before tile 0 refills them
    __syncthreads();

    // One tile: the softmax of S_kt, S_{kt+1} = K_{kt+1} Q^T and its row
    // max, and (PV) O += P_{kt-1} V_{kt-1}; tile 0 has no P V.  Reads stage
    // S (K_{kt+1}, V_{kt-1}); loads go to stage S ^ 1.
    auto tile = [&](const int kt, auto SC, auto PVC) {
      constexpr int S = decltype(SC)::value;
      constexpr bool PV = decltype(PVC)::value != 0;
      // K_{kt+2} replaces K_kt (read for S_kt last tile); V_kt replaces
      // V_{kt-2} (read for its P V last tile)
      const i32x4 idk = tile_ids(kt + 2), idv = tile_ids(kt);
      // all waves are done with the stage refilled below, and the tiles
      // loaded last time have landed
      if (kt > 0) wait_loads_and_sync();
      load_k(kt + 2, S ^ 1, idk);
      load_v(kt, S ^ 1, idv);
      // O holds P_{kt-2} V_{kt-2}: move it to the reference of tile kt-1
      if (PV && pend_grow) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[t][r] *= pend_alpha;
      }
      float alpha, neg_m;
      bool grow;
      {
        const int k0 = kt * BN;
        const bool need_mask = (k0 + BN > nk) || (CAUSAL && (k0 + BN - 1 > q0 + off));
        if (need_mask) {
          // key of register r in half `sub`: k0 + hi*4 + sub*32 + (r/4)*8 + r%4
          const int lim = klast - (k0 + hi * 4);
          smax_cur = -INFINITY;
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rel = sub * 32 + (r >> 2) * 8 + (r & 3);
              st_cur[sub][r] = (rel <= lim) ? st_cur[sub][r] : -INFINITY;
              smax_cur = fmaxf(smax_cur, st_cur[sub][r]);
            }
        }
        const float tmax = pair_max32(smax_cur) * c;
        grow = tmax > m_run + GROW;
        // lanes that do not grow keep their reference (alpha = 1, which also
        // covers rows that have not seen a visible key, m = -inf); a row
        // leaving -inf gets alpha = 0
        const float m_new = tmax + HEAD;
        alpha = fast_exp2(grow ? m_run - m_new : 0.f);
        m_run = grow ? m_new : m_run;
        neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
      }

      // ---- the slots: one matrix op each (S_{kt+1} then O += P_{kt-1}
      // V_{kt-1}), its LDS operand fetched PFD slots ahead, and a share of
      // the vector ops of the softmax of S_kt / the row max of S_{kt+1} ----
      const uint16_t* kb = kst(S);
      const uint16_t* vb = vst(S);
      auto fetch = [&](int i) -> u32x4 {
        if (i < NQK) return *(const u32x4*)(kb + (i / NS) * 32 * D + kofs[i % NS]);
        const int j = i - NQK, t = j / (BN / 16), ks = j % (BN / 16);
        const uint16_t* a = vb + ks * 16 * D + vofs[t];
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(a)));
        const u32x2 hi8 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(a + 8 * D)));
        return u32x4{lo.x, lo.y, hi8.x, hi8.y};
      };
      constexpr int NSLOT = NQK + NPV;
      // slots that issue a matrix op: [0, NA)
      constexpr int NA = PV ? NSLOT : NQK;
      f32x16 st_next[2];
      u32x4 pb_cur[4];
      float psum = 0.f, pe_prev = 0.f, smax_next = -INFINITY;
      // softmax of S_kt, probability e (32 per lane), packed in pairs
      auto softmax_elem = [&](int e) {
        const int sub = e / 16, r = e % 16;
        // the empty volatile statements keep this slot's vector work
        // between this slot's neighbours in the instruction stream
        float x = st_cur[sub][r];
        asm volatile("" : "+v"(x));
        float pe = fast_exp2(fmaf(x, c, neg_m));
        asm volatile("" : "+v"(pe));
        if (r & 1) {
          // (pinned here too: otherwise the compiler sinks the packs and the
          // dependent chain of sums to the top of the next tile, where no
          // matrix op runs beside them)
          uint32_t w = TT::pack2(pe_prev, pe);
          asm volatile("" : "+v"(w));
          // l sums the rounded values that enter P V, so the normalisation
          // matches the weights actually applied
          psum = TT::sum2(w, psum);
          asm volatile("" : "+v"(psum));
          pb_cur[sub * 2 + (r >> 3)][(r & 7) >> 1] = w;
        }
        pe_prev = pe;
      };
      u32x4 opnd[NSLOT];
#pragma unroll
      for (int i = 0; i < PFD; ++i) opnd[i] = fetch(i);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + PFD < NA) opnd[i + PFD] = fetch(i + PFD);
        if (i < NQK) {
          const int sub = i / NS, s = i % NS;
          if (s == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st_next[sub][r] = 0.f;
          }
          st_next[sub] = TT::mma32(opnd[i], qf[s], st_next[sub]);
        } else {
          const int j = i - NQK, t = j / (BN / 16), ks = j % (BN / 16);
          oacc[t] = TT::mma32(opnd[i], pb_prev[ks], oacc[t]);
        }
#pragma unroll
        for (int e = i * 32 / NA; e < (i + 1) * 32 / NA; ++e) softmax_elem(e);
        // row max of S_{kt+1}, once its products have landed
        if (i >= NQK) {
          const int j = i - NQK;                 // 0..NPV-1
          const int e0 = j * 32 / NPV, e1 = (j + 1) * 32 / NPV;
#pragma unroll
          for (int e = e0; e < e1; ++e) smax_next = fmaxf(smax_next, st_next[e / 16][e % 16]);
          asm volatile("" : "+v"(smax_next));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!PV) {
#pragma unroll
        for (int e = 0; e < 32; ++e) smax_next = fmaxf(smax_next, st_next[e / 16][e % 16]);
      }
      l_run = l_run * alpha + psum;
      pend_alpha = alpha;
      pend_grow = __builtin_amdgcn_ballot_w64(grow) != 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb_prev[i] = pb_cur[i];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) st_cur[sub] = st_next[sub];
      smax_cur = smax_next;
    };
    using T1 = IntC<1>;
    using T0 = IntC<0>;
    // the wave's last P V, O += P_L V_L, from the V stage of tile L
    auto last_pv = [&](int L) {
      if (pend_grow) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[t][r] *= pend_alpha;
      }
      const uint16_t* vb = vst(L & 1);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks) {
          const uint16_t* a = vb + ks * 16 * D + vofs[t];
          const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(a)));
          const u32x2 hi8 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(a + 8 * D)));
          oacc[t] = TT::mma32(u32x4{lo.x, lo.y, hi8.x, hi8.y}, pb_prev[ks], oacc[t]);
        }
    };

    // The wave computes tiles 0 .. L = last_w (tile 0 has no P V).  Its
    // last P V, P_L V_L, comes in tile L + 1, before that tile's loads are
    // issued (so no load into LDS is in flight while it reads V_L), or after
    // the loop when L is the last tile.  From then on the wave only issues
    // its share of the remaining tile loads and joins their barriers.  Tile
    // kt reads stage (kt & 1) ^ 1.
    const int L = last_w;
    int kt = 0;
    if (L >= 0) {
      tile(0, T1(), T0());
      for (kt = 1; kt + 1 <= L; kt += 2) {
        tile(kt, T0(), T1());
        tile(kt + 1, T1(), T1());
      }
      if (kt <= L) {
        tile(kt, T0(), T1());
        ++kt;
      }
    }
    // (a wave with no visible key starts here at tile 0, which, as for the
    // others, has no barrier: every wave passes the same barriers)
    for (; kt < ntiles; ++kt) {   // tile kt fills stage kt & 1
      const i32x4 idk = tile_ids(kt + 2), idv = tile_ids(kt);
      if (kt > 0) wait_loads_and_sync();
      if (L >= 0 && kt == L + 1) last_pv(L);
      load_k(kt + 2, kt & 1, idk);
      load_v(kt, kt & 1, idv);
    }
    wait_loads_and_sync();
    if (L >= 0 && L == ntiles - 1) last_pv(L);
  }

  // ---- epilogue: O = O^T / l, LSE ----
  const float l_tot = pair_sum32(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  {
    // Each wave's 32 output rows go through LDS (16-byte chunk c of row r
    // at c ^ (r % CPR), against bank conflicts) so that each store
    // instruction writes whole rows instead of 8-byte pieces of 32 rows.  Two
    // waves share each K or V stage.
    static_assert(NW <= 8 && 64 * D <= TILE, "O staging fits the K and V stages");
    __syncthreads();            // every wave is done with the K/V stages
    uint16_t* ow = ((wave >> 1) & 3) < 2 ? kst(wave >> 1) : vst((wave >> 1) - 2);
    ow += (wave & 1) * 32 * D;
    auto oswz = [](int r) { return r & (CPR - 1); };
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = TT::pack2(oacc[t][4 * g + 0] * inv, oacc[t][4 * g + 1] * inv);
        w.y = TT::pack2(oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv);
        *(u32x2*)(ow + col * D + (((4 * t + g) ^ oswz(col)) * 8) + hi * 4) = w;
      }
    lds_order();
    // lane l: chunk l % CPR of row (l / CPR) + (64 / CPR) i of this wave's rows
    constexpr int RPI = 64 / CPR;   // rows per store instruction
    T* Ob = (T*)p.o + (int64_t)b * p.os_b + (int64_t)h * p.os_h;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CPR;
      const int grow = wr0 + r;
      const u32x4 v = *(const u32x4*)(ow + r * D + (((lane % CPR) ^ oswz(r)) * 8));
      // non-temporal: O is not read back here, and lines it leaves dirty in
      // the caches would be written back during whatever kernel runs next
      if (grow < p.n_q)
        __builtin_nontemporal_store(v, (u32x4*)(Ob + (int64_t)grow * p.os_n + (lane % CPR) * 8));
    }
  }
  if (qrow < p.n_q) {
    if (p.lse != nullptr && hi == 0) {
      p.lse[((int64_t)b * p.h_q + h) * p.n_q + qrow] =
          (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ----------------------------------------------------------------------------
// fp32 kernel
// ----------------------------------------------------------------------------
// A workgroup of 256 threads owns 64 query rows of one (batch, head); the
// four lanes of a quad share a row and each holds D/4 of its q and o.  Keys
// are visited in tiles of 32 staged in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdParams p) {
  constexpr int BMF = 64, BNF = 32, DQ = D / 4;
  __shared__ float ks[BNF][D + 4];
  __shared__ float vs[BNF][D + 4];
  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const int b = blockIdx.z, h = blockIdx.y;
  const int q0 = blockIdx.x * BMF;
  const int kvh = h / p.group;
  const int off = p.n_k - p.n_q;
  const int qrow = q0 + qi;

  const float* Qg = (const float*)p.q + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h;
  const float* Kg = (const float*)p.k + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const float* Vg = (const float*)p.v + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;

  float qv[DQ], ov[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    qv[c] = (qrow < p.n_q) ? Qg[(int64_t)qrow * p.qs_n + part * DQ + c] : 0.f;
    ov[c] = 0.f;
  }
  int kend = p.n_k;
  if (CAUSAL) {
    const int qlast = min(q0 + BMF, p.n_q) - 1;
    kend = min(p.n_k, max(0, qlast + off + 1));
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int k0 = 0; k0 < kend; k0 += BNF) {
    __syncthreads();
    for (int idx = tid; idx < BNF * D; idx += 256) {
      const int r = idx / D, c = idx % D;
      const int key = k0 + r;
      ks[r][c] = (key < p.n_k) ? Kg[(int64_t)key * p.ks_n + c] : 0.f;
      vs[r][c] = (key < p.n_k) ? Vg[(int64_t)key * p.vs_n + c] : 0.f;
    }
    __syncthreads();
    float s[BNF];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c) acc = fmaf(qv[c], ks[j][part * DQ + c], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = k0 + j;
      const bool vis = (key < p.n_k) && (!CAUSAL || key <= qrow + off);
      s[j] = vis ? acc * p.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < DQ; ++c) ov[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      const float pj = exp2f(s[j] - m_use);
      l_run += pj;
#pragma unroll
      for (int c = 0; c < DQ; ++c) ov[c] = fmaf(pj, vs[j][part * DQ + c], ov[c]);
    }
    m_run = m_new;
  }
  if (qrow < p.n_q) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    float* Og = (float*)p.o + (int64_t)b * p.os_b + (int64_t)qrow * p.os_n + (int64_t)h * p.os_h;
#pragma unroll
    for (int c = 0; c < DQ; ++c) Og[part * DQ + c] = ov[c] * inv;
    if (p.lse != nullptr && part == 0)
      p.lse[((int64_t)b * p.h_q + h) * p.n_q + qrow] =
          (l_run > 0.f) ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// ----------------------------------------------------------------------------
// host-side launchers
// ----------------------------------------------------------------------------
template <typename TT, int D, bool CAUSAL, bool PAGED>
static hipError_t launch_mfma(FwdParams p, hipStream_t stream) {
  constexpr int NW = 8;   // waves per workgroup: 256 query rows share each K/V tile
  // two heads of one KV head's group per workgroup when the group allows,
  // else 256 rows of one head
  p.hpw = (p.group % 2 == 0) ? 2 : 1;
  const int bm = 32 * NW / p.hpw;
  p.n_qtiles = (p.n_q + bm - 1) / bm;
  p.num_items = p.n_qtiles * p.batch * (p.h_q / p.hpw);
  p.xcd_chunk = p.group / p.hpw > 1 ? p.group / p.hpw : 1;
  // bytes from the first row of a (batch, kv head) slice to the end of its last row
  p.k_bytes = p.n_k > 0 ? (uint32_t)(((int64_t)(p.n_k - 1) * p.ks_n + D) * 2) : 0u;
  p.v_bytes = p.n_k > 0 ? (uint32_t)(((int64_t)(p.n_k - 1) * p.vs_n + D) * 2) : 0u;
  p.q_bytes = p.n_q > 0 ? (uint32_t)(((int64_t)(p.n_q - 1) * p.qs_n + D) * 2) : 0u;
  hipLaunchKernelGGL((attn_fwd_mfma_kernel<TT, D, CAUSAL, PAGED, NW>), dim3(p.num_items),
                     dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool PAGED>
static hipError_t launch_f32(FwdParams p, hipStream_t stream) {
  dim3 grid((p.n_q + 63) / 64, p.h_q, p.batch);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// dtype: 0 f32, 1 f16, 2 bf16.  Returns the launch status.
hipError_t launch_prefill(int dtype, int head_dim, bool causal, const FwdParams& p,
                          hipStream_t stream) {
#define ATTN_DISPATCH_D(FN, ...)                                                 \
  (head_dim == 64 ? (causal ? FN<__VA_ARGS__ 64, true, false>(p, stream)         \
                            : FN<__VA_ARGS__ 64, false, false>(p, stream))       \
                  : (causal ? FN<__VA_ARGS__ 128, true, false>(p, stream)        \
                            : FN<__VA_ARGS__ 128, false, false>(p, stream)))
  if (dtype == 2) return ATTN_DISPATCH_D(launch_mfma, BF16,);
  if (dtype == 1) return ATTN_DISPATCH_D(launch_mfma, F16,);
  return ATTN_DISPATCH_D(launch_f32, );
#undef ATTN_DISPATCH_D
}

// Prefill over a paged KV cache (bf16 / fp16).
hipError_t launch_prefill_paged(int dtype, int head_dim, bool causal, const FwdParams& p,
                                hipStream_t stream) {
#define ATTN_DISPATCH_P(TT)                                                    \
  (head_dim == 64 ? (causal ? launch_mfma<TT, 64, true, true>(p, stream)       \
                            : launch_mfma<TT, 64, false, true>(p, stream))     \
                  : (causal ? launch_mfma<TT, 128, true, true>(p, stream)      \
                            : launch_mfma<TT, 128, false, true>(p, stream)))
  if (dtype == 2) return ATTN_DISPATCH_P(BF16);
  return ATTN_DISPATCH_P(F16);
#undef ATTN_DISPATCH_P
}

}  // namespace attn
