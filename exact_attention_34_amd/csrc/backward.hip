// Backward pass of exact attention (bf16 / fp16, gfx950 matrix cores).
//
// The forward pass keeps no N x N matrix, so the backward pass recomputes
// the probabilities tile by tile from Q, K and the forward log-sum-exp
// ("Other people's interview notes", question "explain FlashAttention",
// part 3: recomputation instead of storing P; the codelogiq.de FAQ table,
// row on intermediate storage).  With S = scale Q K^T, P = softmax(S) and an
// upstream gradient dO, the chain rule gives
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O),
//     dQ = scale dS K,  dK = scale dS^T Q,
// where rowsum(P * dP) = rowsum(dO * O) because O = P V.  P itself is
// exp(S - lse) with the forward pass's per-row log-sum-exp: no running max is
// needed the second time.
//
// Three kernels, none of them with atomics, so results are deterministic:
//   * attn_bwd_delta_kernel: delta = rowsum(dO * O) per query row (fp32),
//     and the forward log-sum-exp converted to log2 units;
//   * attn_bwd_dkdv_kernel: a workgroup owns 128 keys of one (batch, KV head)
//     and walks every query tile of every query head of the GQA group that
//     can see them; dK and dV accumulate in registers (eight waves: 32 keys
//     x half of each query tile per wave);
//   * attn_bwd_dq_kernel: a workgroup owns 128 query rows of one (batch,
//     head) (32 per wave) and walks the key tiles they can see; dQ
//     accumulates in registers.
// Both main kernels use v_mfma_f32_32x32x16 with fp32 accumulation.  In the
// key-owning kernel S = Q K^T leaves each lane one key column and 16 query
// rows, so the rounded P and dS are directly the B operands of
// dV^T = dO^T P and dK^T = Q^T dS; in the query-owning kernel S^T = K Q^T
// leaves each lane one query column, and dS^T is the B operand of
// dQ^T = K^T dS^T.  The transposed operands (dO^T, Q^T, K^T) are read from
// row-major LDS tiles with ds_read_b64_tr_b16.
#include "common.h"
#include "schedule.h"

namespace attn {

// ----------------------------------------------------------------------------
// delta = rowsum(dO * O)
// ----------------------------------------------------------------------------
// Rows are taken in (position, head) order, so that with the usual
// [batch][position][head][d] layout a workgroup reads one contiguous stretch.
template <typename TT, int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  typedef typename TT::elem T;
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;   // rows per pass of the workgroup
  constexpr int PASSES = 4;        // rows of a thread, loaded together
  const int tid = threadIdx.x, c = tid % CPR;
  const int b = blockIdx.y;
  const int64_t nrows = (int64_t)p.n_q * p.h_q;
  const T* Ob = (const T*)p.o + (int64_t)b * p.os_b + c * 8;
  const T* Gb = (const T*)p.dout + (int64_t)b * p.dos_b + c * 8;
  u32x4 o[PASSES], g[PASSES];
  int64_t row[PASSES];
  float lse[PASSES];
  // every load of the thread (its O and dO chunks, and for the first lane of
  // a row the row's log-sum-exp) is issued before any is used
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    const int64_t r = ((int64_t)blockIdx.x * PASSES + i) * RPP + tid / CPR;
    const int n = (int)(r / p.h_q);
    const int h = (int)(r - (int64_t)n * p.h_q);
    row[i] = r < nrows ? ((int64_t)b * p.h_q + h) * p.n_q + n : -1;
    o[i] = g[i] = u32x4{0, 0, 0, 0};
    lse[i] = 0.f;
    if (r < nrows) {
      o[i] = *(const u32x4*)(Ob + (int64_t)n * p.os_n + (int64_t)h * p.os_h);
      g[i] = *(const u32x4*)(Gb + (int64_t)n * p.dos_n + (int64_t)h * p.dos_h);
      if (c == 0) lse[i] = p.lse[row[i]];
    }
  }
#pragma unroll
  for (int i = 0; i < PASSES; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = TT::dot2(o[i][k], g[i][k], acc);
#pragma unroll
    for (int sh = 1; sh < CPR; sh <<= 1) acc += __shfl_xor(acc, sh);
    if (c == 0 && row[i] >= 0) {
      p.delta[row[i]] = acc;
      // the log-sum-exp in log2 units, as the probabilities are recomputed
      p.lse2[row[i]] = lse[i] * kLog2e;
    }
  }
}

// LDS tiles of these kernels are row-major [row][d] with 16-byte chunk c of
// row r stored at c ^ tswz(r), filled by direct buffer -> LDS loads (each lane
// fetches the global chunk that belongs in its LDS slot).  The tiles are read
// two ways, and the permutation keeps both free of bank conflicts:
//   * row reads: 16 bytes of one row per lane, one chunk of 32 consecutive
//     rows; tswz is a bijection on r % 16 (d = 128), or on the rows of one
//     parity within 16 (d = 64, two 128-byte rows per 256 bytes of banks);
//   * transposing reads (below): 32 lanes read 4 consecutive rows (4k ..
//     4k + 3) x 4 consecutive chunks (4t .. 4t + 3); the bits of tswz above
//     the low two differ between those rows, so the 16 chunks land in
//     distinct banks.
// d = 128: tswz(r) = 4 (r % 4) + (r / 4) % 4 (a rotation of r % 16).
// d = 64:  tswz(r) = 4 ((r / 2) % 2) + (r / 4) % 4.
template <int CPR>
__device__ inline int tswz(int r) {
  if (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-lane offsets (elements) of the transposing reads of a 32-column block t
// of such a tile: within each 16-lane group (g = lane / 16, i = lane % 16)
// lane 4 j + q points at row 4 (g / 2) + j and columns t*32 + 16 (g % 2) + 4 q
// .. + 3; ds_read_b64_tr_b16 then leaves lane i with rows 4 (g / 2) .. + 3 of
// column t*32 + 16 (g % 2) + i.  The second read of a 16-row k-step is 8 rows
// further; adding 16 rows leaves the permutation unchanged.
// tr_base gives block 0's first read; the others follow by flipping bits
// (tr_ofs): block t changes only chunk bits 2..3, which move bits 5..6 of the
// offset, and the rows 8 further have the permutation XOR 2 (chunk bit 1,
// offset bit 4) and add 8 D, a bit that is clear in every first-read row.
// Likewise the row read of k-step s is k-step 0's offset XOR 16 s.  So a
// tile's offsets cost one XOR each from two per-lane values.
template <int D>
__device__ inline int tr_base(int lane) {
  constexpr int CPR = D / 8;
  const int vi = lane & 15, vg = lane >> 4;
  const int r = (vg >> 1) * 4 + (vi >> 2);
  const int el = (vg & 1) * 16 + (vi & 3) * 4;
  return r * D + (((el >> 3) ^ tswz<CPR>(r)) * 8) + (el & 7);
}
template <int D>
__device__ inline int tr_ofs(int base, int t, int half) {
  return base ^ (32 * t) ^ (half ? (16 | 8 * D) : 0);
}
// Row-read offset of k-step 0 (row `row`, chunk `hi`).
template <int D>
__device__ inline int row_base(int row, int hi) {
  return row * D + ((hi ^ tswz<D / 8>(row)) * 8);
}

// A operand of a 32x32x16 product whose k index runs over 16 rows of a tile
// (rows 4 (lane / 32) + 0..3 and 8 + 4 (lane / 32) + 0..3) and whose m index is
// the 32 columns of block t.
__device__ inline u32x4 tr_operand(const uint16_t* base, int ofs0, int ofs1) {
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + ofs0)));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(base + ofs1)));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Stage a wave's 32 x D output block (lane = output row `col`, accumulator
// rows = columns t*32 + 8 j + 4 hi + i) through LDS and store it as whole
// rows: out row `row0 + r` at `dst + (row0 + r) * stride`, rows >= n skipped.
template <typename TT, int D>
__device__ inline void store_rows(const f32x16 (&acc)[D / 32], float mul, uint16_t* stage,
                                  int lane, typename TT::elem* dst, int64_t stride, int row0,
                                  int n) {
  constexpr int CPR = D / 8;
  constexpr int OP = D + 8;   // padded row, elements
  const int col = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w.x = TT::pack2(acc[t][4 * g + 0] * mul, acc[t][4 * g + 1] * mul);
      w.y = TT::pack2(acc[t][4 * g + 2] * mul, acc[t][4 * g + 3] * mul);
      *(u32x2*)(stage + col * OP + t * 32 + g * 8 + hi * 4) = w;
    }
  lds_order();
  constexpr int RPI = 64 / CPR;   // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;
    const u32x4 v = *(const u32x4*)(stage + r * OP + (lane % CPR) * 8);
    if (row0 + r < n) *(u32x4*)(dst + (int64_t)(row0 + r) * stride + (lane % CPR) * 8) = v;
  }
  lds_order();
}

// ----------------------------------------------------------------------------
// dK, dV: a workgroup per (128 keys, batch, KV head)
// ----------------------------------------------------------------------------
// Eight waves, two per SIMD: wave w owns keys 32 (w % 4) .. + 31 of the tile
// and, of every 64-row query tile, rows 32 (w / 4) .. + 31.  The two waves of
// a key group hold partial dK and dV, summed through LDS at the end (in a
// fixed order, so the result is deterministic).
template <typename TT, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(BwdParams p) {
  typedef typename TT::elem T;
  constexpr int BK = 128, BQ = 64;        // keys per workgroup, queries per tile
  constexpr int NT = 512;                 // threads
  constexpr int CPR = D / 8;
  constexpr int NS = D / 16;              // k-steps over d
  constexpr int TILE = BQ * D;            // elements of a Q or dO tile
  constexpr int LOADS = BQ * CPR / NT;    // direct loads per thread per tile
  static_assert(LOADS * NT == BQ * CPR, "tile split");
  // One array per stage (Q, dO, log-sum-exp and delta rows), named at compile
  // time, so that the compiler can see that the stage being read is not the
  // one the direct loads are filling; with a runtime stage index into one
  // array it waits for the next tile's loads before the first read of every
  // tile.  The four tile arrays are reused at the end for the partial sums
  // and the output staging, one per key group.
  __shared__ __attribute__((aligned(16))) uint16_t q_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t q_lds1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t o_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t o_lds1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[BK * D];   // this tile's V, [key][d]
  __shared__ __attribute__((aligned(16))) float lse_lds0[BQ];
  __shared__ __attribute__((aligned(16))) float lse_lds1[BQ];
  __shared__ __attribute__((aligned(16))) float dl_lds0[BQ];
  __shared__ __attribute__((aligned(16))) float dl_lds1[BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3, rh = wave >> 2;   // key group, query-row half
  const int col = lane & 31, hi = lane >> 5;
  // items: key tile (the first tiles see the most queries when causal), batch, KV head
  const int bh = p.batch * p.h_kv;
  const int blk = group_heads_on_xcd(blockIdx.x, bh, p.n_kt);
  const int kt = blk / bh, rem = blk - kt * bh;
  const int b = rem / p.h_kv, kvh = rem - b * p.h_kv;
  const int k0 = kt * BK;
  const int kcol = k0 + kw * 32 + col;   // this lane's key
  const int off = p.n_k - p.n_q;
  const float c = p.scale_log2;

  // K fragment: B operand of S = Q K^T (column = key, k = d chunk 2 s + hi),
  // held in registers; V (the B operand of dP = dO V^T) is read from LDS
  const T* Kg = (const T*)p.k + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const T* Vg = (const T*)p.v + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  u32x4 kf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = u32x4{0, 0, 0, 0};
    if (kcol < p.n_k) kf[s] = *(const u32x4*)(Kg + (int64_t)kcol * p.ks_n + (2 * s + hi) * 8);
  }
  {
    // V rows k0 .. k0 + 127 in the tile layout (rows past n_k read as zero)
    const uint32_t vrow = (uint32_t)p.vs_n * 2u, ov = (uint32_t)k0 * vrow;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(
        (const char*)Vg + ov, __builtin_amdgcn_readfirstlane(p.v_bytes > ov ? p.v_bytes - ov : 0u));
#pragma unroll
    for (int i = 0; i < BK * CPR / NT; ++i) {
      const int slot = (i * 8 + wave) * 64 + lane;
      const int row = slot / CPR, pc = slot % CPR;
      buf_load16_lds(rv, v_lds + (i * 8 + wave) * 512,
                     (uint32_t)row * vrow + (uint32_t)((pc ^ tswz<CPR>(row)) * 16));
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[t][r] = dv[t][r] = 0.f;

  // query tiles that see a key of this tile: q >= k0 - off when causal
  const int qt0 = CAUSAL ? max(0, k0 - off) / BQ : 0;
  const int nqt = (p.n_q + BQ - 1) / BQ;
  const int per_head = nqt > qt0 ? nqt - qt0 : 0;
  const int ntiles = per_head * p.group;

  // per-lane LDS offsets of k-step 0 and of transposing-read block 0; each
  // tile derives its offsets from these with one XOR apiece
  const int kbase0 = row_base<D>(rh * 32 + col, hi);
  const int tbase0 = tr_base<D>(lane);

  // direct loads of the Q and dO tiles and of the tile's lse and delta rows.
  // Load i of a wave covers rows (8 i + wave) RPI + lane / CPR, lane % CPR
  // naming the LDS chunk; a row's swizzle depends on the row mod 16 alone,
  // which does not change with i, so each lane's byte offset is fixed and
  // the rest is a uniform offset per load.
  constexpr int RPI = 64 / CPR;   // rows per load instruction
  static_assert((8 * RPI) % 16 == 0, "a load index step keeps the row mod 16");
  const uint32_t qrowb = (uint32_t)p.qs_n * 2u, orowb = (uint32_t)p.dos_n * 2u;
  auto load_tile = [&](int idx, auto SC) {
    constexpr int ST = decltype(SC)::value;
    // the lane's offsets, derived per tile (a few instructions) rather than
    // held in registers across the loop: the empty statement hides the lane
    // index from loop-invariant hoisting
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lrow = ln / CPR, lpc = ln % CPR;
    const uint32_t cb = (uint32_t)((lpc ^ tswz<CPR>(wave * RPI + lrow)) * 16);
    const uint32_t vq = (uint32_t)lrow * qrowb + cb, vo = (uint32_t)lrow * orowb + cb;
    uint16_t* qd = ST ? q_lds1 : q_lds0;
    uint16_t* od = ST ? o_lds1 : o_lds0;
    const int h = kvh * p.group + idx / per_head;
    const int q0 = (qt0 + idx % per_head) * BQ;
    const T* Qg = (const T*)p.q + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h;
    const T* Og = (const T*)p.dout + (int64_t)b * p.dos_b + (int64_t)h * p.dos_h;
    const uint32_t oq = (uint32_t)q0 * qrowb, oo = (uint32_t)q0 * orowb;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(
        uniform_ptr((const char*)Qg + oq),
        __builtin_amdgcn_readfirstlane(p.q_bytes > oq ? p.q_bytes - oq : 0u));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(
        uniform_ptr((const char*)Og + oo),
        __builtin_amdgcn_readfirstlane(p.do_bytes > oo ? p.do_bytes - oo : 0u));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t r0 = (uint32_t)((i * 8 + wave) * RPI);
      buf_load16_lds(rq, qd + (i * 8 + wave) * 512, vq, r0 * qrowb);
      buf_load16_lds(ro, od + (i * 8 + wave) * 512, vo, r0 * orowb);
    }
    // rows past n_q read as zero: their Q and dO rows are zero too, so they
    // contribute nothing whatever their probabilities
    if (wave == 0) {
      const int64_t row = ((int64_t)b * p.h_q + h) * p.n_q + q0;
      const uint32_t nb = __builtin_amdgcn_readfirstlane((uint32_t)(p.n_q - q0) * 4u);
      buf_load4_lds(make_rsrc(uniform_ptr(p.lse2 + row), nb), ST ? lse_lds1 : lse_lds0,
                    (uint32_t)lane * 4u);
      buf_load4_lds(make_rsrc(uniform_ptr(p.delta + row), nb), ST ? dl_lds1 : dl_lds0,
                    (uint32_t)lane * 4u);
    }
  };

  // one query tile, read from stage S (tile idx lands in stage idx & 1)
  auto step = [&](const int idx, auto SC) {
    constexpr int S = decltype(SC)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // tile idx landed; every wave is done with stage S ^ 1
    if (idx + 1 < ntiles) load_tile(idx + 1, IntC<S ^ 1>());
    const int q0 = (qt0 + idx % per_head) * BQ + rh * 32;   // this wave's first row
    const uint16_t* qb = S ? q_lds1 : q_lds0;
    const uint16_t* ob = S ? o_lds1 : o_lds0;
    const float* lsb = S ? lse_lds1 : lse_lds0;
    const float* dlb = S ? dl_lds1 : dl_lds0;
    // rows whose visible keys do not cover this wave's keys need the mask
    const bool need_mask = CAUSAL && (q0 + off < k0 + kw * 32 + 31);
    // LDS read offsets, derived here rather than held across the loop (the
    // empty statement keeps the compiler from hoisting them)
    int kb0 = kbase0, tb0 = tbase0;
    asm volatile("" : "+v"(kb0), "+v"(tb0));
    int kofs[NS];   // row reads: row col of this wave's 32 query rows, chunk 2 s + hi
#pragma unroll
    for (int s = 0; s < NS; ++s) kofs[s] = kb0 ^ (16 * s);
    // V rows of this wave's keys: the Q row offsets moved by (kw - rh) 32 rows
    const uint16_t* vb = v_lds + (kw - rh) * 32 * D;
    // One matrix product per slot, its LDS operand fetched PFD slots ahead:
    // S = Q K^T and dP = dO V^T alternate over the k-steps (slots 0 ..
    // NSD-1), then, once P and dS are formed, dV^T += dO^T P and
    // dK^T += Q^T dS alternate over (k-step, column block).
    constexpr int DT = D / 32;
    constexpr int NSD = 2 * NS, NVK = 4 * DT, NSLOT = NSD + NVK;
    constexpr int PFD = 3;
    auto fetch = [&](int i) -> u32x4 {
      if (i < NSD) return *(const u32x4*)(((i & 1) ? ob : qb) + kofs[i >> 1]);
      const int j = i - NSD, ks = j / (2 * DT), t = (j >> 1) % DT;
      return tr_operand(((j & 1) ? qb : ob) + (rh * 2 + ks) * 16 * D, tr_ofs<D>(tb0, t, 0),
                        tr_ofs<D>(tb0, t, 1));
    };
    // the B operand of a dP slot (V rows), fetched with its A operand
    auto fetch_v = [&](int i) -> u32x4 {
      return (i < NSD && (i & 1)) ? *(const u32x4*)(vb + kofs[i >> 1]) : u32x4{0, 0, 0, 0};
    };
    u32x4 opnd[NSLOT], opv[NSLOT];
#pragma unroll
    for (int i = 0; i < PFD; ++i) {
      opnd[i] = fetch(i);
      opv[i] = fetch_v(i);
    }
    f32x16 sacc, dpacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = dpacc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < NSD; ++i) {
      opnd[i + PFD] = fetch(i + PFD);
      opv[i + PFD] = fetch_v(i + PFD);
      if (i & 1)
        dpacc = TT::mma32(opnd[i], opv[i], dpacc);
      else
        sacc = TT::mma32(opnd[i], kf[i >> 1], sacc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane: key kcol, query rows q0 + 8 j + 4 hi + i (register 4 j + i);
    // P = 2^(S c - lse log2 e) with the log-sum-exp stored in log2 units.
    // Tiles whose keys every row of the wave sees skip the mask (the choice
    // is uniform per wave).
    u32x4 pp[2], ps[2];
    auto probs = [&](auto MC) {
      constexpr bool MASK = decltype(MC)::value != 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 lv = *(const f32x4*)(lsb + rh * 32 + 8 * j + 4 * hi);
        const f32x4 dl = *(const f32x4*)(dlb + rh * 32 + 8 * j + 4 * hi);
        float pv[4], dsv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          const float e = fast_exp2(fmaf(sacc[r], c, -lv[i]));
          pv[i] = (!MASK || kcol <= q0 + 8 * j + 4 * hi + i + off) ? e : 0.f;
          dsv[i] = pv[i] * (dpacc[r] - dl[i]);
        }
        // k-step j / 2 of the 32 query rows, values 4 (j % 2) .. + 3
        pp[j >> 1][(j & 1) * 2 + 0] = TT::pack2(pv[0], pv[1]);
        pp[j >> 1][(j & 1) * 2 + 1] = TT::pack2(pv[2], pv[3]);
        ps[j >> 1][(j & 1) * 2 + 0] = TT::pack2(dsv[0], dsv[1]);
        ps[j >> 1][(j & 1) * 2 + 1] = TT::pack2(dsv[2], dsv[3]);
      }
    };
    if (need_mask)
      probs(IntC<1>());
    else
      probs(IntC<0>());
    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P, dK^T += Q^T dS (scale applied at the end)
#pragma unroll
    for (int i = NSD; i < NSLOT; ++i) {
      if (i + PFD < NSLOT) opnd[i + PFD] = fetch(i + PFD);
      const int j = i - NSD, ks = j / (2 * DT), t = (j >> 1) % DT;
      if (j & 1)
        dk[t] = TT::mma32(opnd[i], ps[ks], dk[t]);
      else
        dv[t] = TT::mma32(opnd[i], pp[ks], dv[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (ntiles > 0) load_tile(0, IntC<0>());
  for (int idx = 0; idx < ntiles; idx += 2) {
    step(idx, IntC<0>());
    if (idx + 1 < ntiles) step(idx + 1, IntC<1>());
  }

  // ---- epilogue: sum the two row halves of each key group, then write
  // dK = scale dK^T^T and dV = dV^T^T as whole rows through LDS ----
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // every wave is done with the tiles
  // key group kw's region: one of the four tile arrays
  uint16_t* region = kw == 0 ? q_lds0 : kw == 1 ? q_lds1 : kw == 2 ? o_lds0 : o_lds1;
  float* part = (float*)region;   // [t][4 floats of 16][lane][4]
  static_assert((D / 32) * 16 * 64 * 4 <= TILE * 2, "partial sums fit");
  auto merge = [&](f32x16 (&acc)[D / 32]) {
    if (rh == 1) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(f32x4*)(part + ((t * 4 + e) * 64 + lane) * 4) =
              f32x4{acc[t][4 * e], acc[t][4 * e + 1], acc[t][4 * e + 2], acc[t][4 * e + 3]};
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4 x = *(const f32x4*)(part + ((t * 4 + e) * 64 + lane) * 4);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[t][4 * e + u] += x[u];
        }
    }
    __syncthreads();
  };
  merge(dk);
  merge(dv);
  if (rh == 0) {
    uint16_t* stage = region;
    static_assert(32 * (D + 8) <= TILE, "output staging fits");
    T* dKg = (T*)p.dk + (int64_t)b * p.dks_b + (int64_t)kvh * p.dks_h;
    T* dVg = (T*)p.dv + (int64_t)b * p.dvs_b + (int64_t)kvh * p.dvs_h;
    store_rows<TT, D>(dk, p.scale, stage, lane, dKg, p.dks_n, k0 + kw * 32, p.n_k);
    store_rows<TT, D>(dv, 1.f, stage, lane, dVg, p.dvs_n, k0 + kw * 32, p.n_k);
  }
}

// ----------------------------------------------------------------------------
// dQ: a workgroup per (128 query rows, batch, head)
// ----------------------------------------------------------------------------
template <typename TT, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(BwdParams p) {
  typedef typename TT::elem T;
  constexpr int BM = 128, BN = 64;
  constexpr int CPR = D / 8;
  constexpr int NS = D / 16;
  constexpr int TILE = BN * D;
  constexpr int LOADS = BN * CPR / 256;
  // one array per stage, so that the compiler can see that the stage being
  // read is not the one the direct loads are filling
  __shared__ __attribute__((aligned(16))) uint16_t ks_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ks_lds1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vs_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vs_lds1[TILE];
  auto kst = [&](int st) -> uint16_t* { return st ? ks_lds1 : ks_lds0; };
  auto vst = [&](int st) -> uint16_t* { return st ? vs_lds1 : vs_lds0; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  // items: query tile (longest first when causal), batch, head
  const int bh = p.batch * p.h_q;
  const int blk = group_heads_on_xcd(blockIdx.x, bh, p.n_qt);
  const int rank = blk / bh, rem = blk - rank * bh;
  const int b = rem / p.h_q, h = rem - b * p.h_q;
  const int qt = CAUSAL ? (p.n_qt - 1 - rank) : rank;
  const int q0 = qt * BM;
  const int kvh = h / p.group;
  const int off = p.n_k - p.n_q;
  int kend = p.n_k;
  if (CAUSAL) {
    const int qlast = min(q0 + BM, p.n_q) - 1;
    kend = min(p.n_k, max(0, qlast + off + 1));
  }
  const int ntiles = (kend + BN - 1) / BN;
  const int qrow = q0 + wave * 32 + col;   // this lane's query
  const bool qvalid = qrow < p.n_q;
  const float c = p.scale_log2;

  // Q^T and dO^T fragments: B operands of S^T = K Q^T and dP^T = V dO^T
  const T* Qg = (const T*)p.q + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h;
  const T* Og = (const T*)p.dout + (int64_t)b * p.dos_b + (int64_t)h * p.dos_h;
  u32x4 qf[NS], of[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = of[s] = u32x4{0, 0, 0, 0};
    if (qvalid) {
      qf[s] = *(const u32x4*)(Qg + (int64_t)qrow * p.qs_n + (2 * s + hi) * 8);
      of[s] = *(const u32x4*)(Og + (int64_t)qrow * p.dos_n + (2 * s + hi) * 8);
    }
  }
  // a row past n_q has zero Q and dO: a zero lse and delta keep its (unused)
  // column finite
  float lse2 = 0.f, dl = 0.f;
  if (qvalid) {
    const int64_t row = ((int64_t)b * p.h_q + h) * p.n_q + qrow;
    lse2 = p.lse2[row];
    dl = p.delta[row];
  }
  // per-lane LDS offsets of k-step 0 and of transposing-read block 0
  const int kbase0 = row_base<D>(col, hi);
  const int tbase0 = tr_base<D>(lane);
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[t][r] = 0.f;

  const T* Kg = (const T*)p.k + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const T* Vg = (const T*)p.v + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;
  const uint32_t krow = (uint32_t)p.ks_n * 2u, vrow = (uint32_t)p.vs_n * 2u;
  uint32_t kgo[LOADS], vgo[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int row = slot / CPR, pc = slot % CPR;
    kgo[i] = (uint32_t)row * krow + (uint32_t)((pc ^ tswz<CPR>(row)) * 16);
    vgo[i] = (uint32_t)row * vrow + (uint32_t)((pc ^ tswz<CPR>(row)) * 16);
  }
  auto load_kv = [&](int kt, int stage) {
    const uint32_t ok = (uint32_t)(kt * BN) * krow, ov = (uint32_t)(kt * BN) * vrow;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(
        uniform_ptr((const char*)Kg + ok),
        __builtin_amdgcn_readfirstlane(p.k_bytes > ok ? p.k_bytes - ok : 0u));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(
        uniform_ptr((const char*)Vg + ov),
        __builtin_amdgcn_readfirstlane(p.v_bytes > ov ? p.v_bytes - ov : 0u));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      buf_load16_lds(rk, kst(stage) + (i * 4 + wave) * 512, kgo[i]);
      buf_load16_lds(rv, vst(stage) + (i * 4 + wave) * 512, vgo[i]);
    }
  };

  // one key tile, read from stage S (tile kt lands in stage kt & 1)
  auto step = [&](const int kt, auto SC) {
    constexpr int S = decltype(SC)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < ntiles) load_kv(kt + 1, S ^ 1);
    const uint16_t* kb = kst(S);
    const uint16_t* vb = vst(S);
    const int k0 = kt * BN;
    const bool need_mask = (k0 + BN > p.n_k) || (CAUSAL && (k0 + BN - 1 > q0 + off));
    // LDS read offsets, derived here rather than held across the loop
    int kb0 = kbase0, tb0 = tbase0;
    asm volatile("" : "+v"(kb0), "+v"(tb0));
    int kofs[NS];   // row reads: key row (lane % 32), chunk 2 s + lane / 32
#pragma unroll
    for (int s = 0; s < NS; ++s) kofs[s] = kb0 ^ (16 * s);
    // One matrix product per slot, its LDS operand fetched PFD slots ahead:
    // for each 32-key half, S^T = K Q^T and dP^T = V dO^T alternate over
    // the k-steps (then that half's dS^T is formed); then dQ^T += K^T dS^T
    // over (k-step, column block).
    constexpr int DT = D / 32;
    constexpr int NSD = 2 * NS, NQ = (BN / 16) * DT, NSLOT = 2 * NSD + NQ;
    constexpr int PFD = 3;
    auto fetch = [&](int i) -> u32x4 {
      if (i < 2 * NSD) {
        const int sub = i / NSD, j = i % NSD;
        return *(const u32x4*)(((j & 1) ? vb : kb) + sub * 32 * D + kofs[j >> 1]);
      }
      const int j = i - 2 * NSD, ks = j / DT, t = j % DT;
      return tr_operand(kb + ks * 16 * D, tr_ofs<D>(tb0, t, 0), tr_ofs<D>(tb0, t, 1));
    };
    u32x4 opnd[NSLOT];
#pragma unroll
    for (int i = 0; i < PFD; ++i) opnd[i] = fetch(i);
    u32x4 dsb[4];   // dS^T: B operand of dQ^T += K^T dS^T, one per 16-key k-step
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = dpacc[r] = 0.f;
#pragma unroll
      for (int j = 0; j < NSD; ++j) {
        const int i = sub * NSD + j;
        opnd[i + PFD] = fetch(i + PFD);
        if (j & 1)
          dpacc = TT::mma32(opnd[i], of[j >> 1], dpacc);
        else
          sacc = TT::mma32(opnd[i], qf[j >> 1], sacc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane: query qrow, keys k0 + sub*32 + 8 j + 4 hi + i (register 4 j + i);
      // tiles inside every row's visible range skip the mask (uniform choice)
      auto grads = [&](auto MC) {
        constexpr bool MASK = decltype(MC)::value != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dsv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            const int key = k0 + sub * 32 + 8 * j + 4 * hi + i;
            const float e = fast_exp2(fmaf(sacc[r], c, -lse2));
            const bool vis = !MASK || (key < p.n_k && (!CAUSAL || key <= qrow + off));
            dsv[i] = (vis ? e : 0.f) * (dpacc[r] - dl);
          }
          dsb[sub * 2 + (j >> 1)][(j & 1) * 2 + 0] = TT::pack2(dsv[0], dsv[1]);
          dsb[sub * 2 + (j >> 1)][(j & 1) * 2 + 1] = TT::pack2(dsv[2], dsv[3]);
        }
      };
      if (need_mask)
        grads(IntC<1>());
      else
        grads(IntC<0>());
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 2 * NSD; i < NSLOT; ++i) {
      if (i + PFD < NSLOT) opnd[i + PFD] = fetch(i + PFD);
      const int j = i - 2 * NSD, ks = j / DT, t = j % DT;
      dq[t] = TT::mma32(opnd[i], dsb[ks], dq[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (ntiles > 0) load_kv(0, 0);
  int kt = 0;
  for (; kt + 1 < ntiles; kt += 2) {
    step(kt, IntC<0>());
    step(kt + 1, IntC<1>());
  }
  if (kt < ntiles) step(kt, IntC<0>());

  // ---- epilogue: dQ = scale dQ^T^T, whole rows through LDS ----
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint16_t* stage = wave < 2 ? kst(wave) : vst(wave - 2);
  static_assert(32 * (D + 8) <= TILE, "a wave's output rows fit one stage");
  T* dQg = (T*)p.dq + (int64_t)b * p.dqs_b + (int64_t)h * p.dqs_h;
  store_rows<TT, D>(dq, p.scale, stage, lane, dQg, p.dqs_n, q0 + wave * 32, p.n_q);
}

// ----------------------------------------------------------------------------
// host-side launch
// ----------------------------------------------------------------------------
template <typename TT, int D, bool CAUSAL>
static hipError_t launch_bwd_t(BwdParams p, hipStream_t stream) {
  constexpr int RPB = 4 * 256 / (D / 8);   // rows per delta workgroup
  p.n_qt = (p.n_q + 127) / 128;
  p.n_kt = (p.n_k + 127) / 128;
  // with no query rows dK = dV = 0; with no keys dQ = 0 (the kernels write
  // the zeros); empty grids are not launched
  hipError_t e = hipSuccess;
  if (p.n_q > 0) {
    const int64_t rows = (int64_t)p.n_q * p.h_q;
    hipLaunchKernelGGL((attn_bwd_delta_kernel<TT, D>), dim3((unsigned)((rows + RPB - 1) / RPB), p.batch),
                       dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.n_k > 0) {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<TT, D, CAUSAL>), dim3(p.n_kt * p.batch * p.h_kv),
                       dim3(512), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.n_q > 0) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<TT, D, CAUSAL>), dim3(p.n_qt * p.batch * p.h_q),
                       dim3(256), 0, stream, p);
    e = hipGetLastError();
  }
  return e;
}

// dtype: 1 f16, 2 bf16.
hipError_t launch_backward(int dtype, int head_dim, bool causal, const BwdParams& p,
                           hipStream_t stream) {
#define ATTN_BWD_D(TT)                                                        \
  (head_dim == 64 ? (causal ? launch_bwd_t<TT, 64, true>(p, stream)           \
                            : launch_bwd_t<TT, 64, false>(p, stream))         \
                  : (causal ? launch_bwd_t<TT, 128, true>(p, stream)          \
                            : launch_bwd_t<TT, 128, false>(p, stream)))
  if (dtype == 2) return ATTN_BWD_D(BF16);
  return ATTN_BWD_D(F16);
#undef ATTN_BWD_D
}

}  // namespace attn
