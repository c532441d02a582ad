// Paged single-token decode: each sequence's one query row attends to all of
// its cached tokens, read through a block table (PagedAttention, tutorial
// "Chapter 3 Advanced principles", section 3.0: fixed-size KV blocks and a
// per-sequence table of physical block ids; shared prefixes are repeated ids).
//
// Split kernel, one workgroup per (context partition of 512 tokens, KV head,
// sequence); the GQA group of query heads that read this KV head is handled
// together, so every K/V byte is fetched from HBM once per partition:
//   phase A  each wave takes 8 blocks of 16 tokens; for every block the 16 x d
//            K tile is read straight from HBM in the B-operand layout of
//            v_mfma_f32_16x16x32 (token = lane % 16) and multiplied by the
//            query heads (A operand rows, zero padded to 16); the scaled
//            scores go to LDS;
//   softmax  the partition's max and sum per head are reduced through LDS
//            (the two-pass form of the definition, restricted to the
//            partition); scores become probabilities in place;
//   phase B  each wave re-walks its blocks reading V with fully coalesced
//            16-byte loads (4 tokens x 256 bytes per instruction) and
//            accumulates p * v in fp32 on the vector ALUs;
//   merge    lanes, then waves, are summed in a fixed order through LDS.  A
//            sequence with a single partition is normalised and written here;
//            otherwise the unnormalised partial output with its (max, sum) goes
//            to the workspace.
// Combine kernel, one workgroup per (head, sequence): the partitions are merged
// by their log-sum-exp -- the same rescaling by exp(m_p - M) that the online
// softmax applies between key blocks.
//
// Tokens at or past the context length are never multiplied: their scores are
// replaced (not scaled) by -inf and their V rows are not loaded, so whatever a
// partially filled block holds past the end cannot reach the output.  Nothing
// depends on physical block ids except addresses, so results are bit-identical
// under any block table.
#include "common.h"

namespace attn {

constexpr int kDecBS = 16;     // tokens per KV block
constexpr int kDecPart = 512;  // tokens per partition

template <typename TT, int D, int GP, int RING>
__global__ __launch_bounds__(64) void paged_decode_split_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  constexpr int NB = kDecPart / kDecBS;  // 32 blocks per partition
  constexpr int KST = D / 32;            // k-steps of q.K^T (16x16x32)
  constexpr int CH = D / 8;              // 16-byte chunks per K/V row
  constexpr int ROWS = 64 / CH;          // V rows per 16-byte load instruction
  constexpr int VST = kDecBS / ROWS;     // V load instructions per block
  // the reference max is raised only when it grows by more than TAU (log2
  // units); probabilities stay below 2^TAU and O is rescaled rarely
  constexpr float TAU = 8.0f;
  static_assert(GP % 4 == 0 && GP <= 16, "padded group");
  // wave-private exchange: probabilities [token][head], block maxima and
  // final sums per head
  __shared__ __attribute__((aligned(16))) float xp[kDecBS * GP];
  __shared__ __attribute__((aligned(16))) float xm[2 * GP];

  const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x;
  const int ctx = p.context_lens[s];
  const int group = p.group;
  const int head0 = kvh * group;

  if (ctx <= 0) {
    // empty context: o = 0, lse = -inf (written once, by partition 0)
    if (part == 0) {
      T* og = (T*)p.o + ((int64_t)s * p.h_q + head0) * D;
      for (int i = lane; i < group * D; i += 64) og[i] = (T)0.f;
      if (p.lse != nullptr && lane < group) p.lse[(int64_t)s * p.h_q + head0 + lane] = -INFINITY;
    }
    return;
  }
  const int tok0 = part * kDecPart;
  if (tok0 >= ctx) return;
  const int ntok = min(kDecPart, ctx - tok0);
  const int nblk = (ntok + kDecBS - 1) / kDecBS;
  const int nparts = (ctx + kDecPart - 1) / kDecPart;
  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq + tok0 / kDecBS;
  const char* kc = (const char*)p.k_cache;
  const char* vc = (const char*)p.v_cache;
  const int64_t blk_bytes = (int64_t)kDecBS * D * 2;
  const float c = p.scale_log2;

  // query heads as the A operand of S = Q K^T (rows = heads, zero padded)
  u32x4 qa[KST];
  {
    const int g = lane & 15;
    const T* qg = (const T*)p.q + ((int64_t)s * p.h_q + head0 + g) * D + (lane >> 4) * 8;
#pragma unroll
    for (int st = 0; st < KST; ++st) {
      qa[st] = u32x4{0, 0, 0, 0};
      if (g < group) qa[st] = *(const u32x4*)(qg + 32 * st);
    }
  }
  // per-lane byte offsets within a (block, kv head) tile of 16 x D
  //   K, B operand: token lane % 16, d = 32 st + 8 (lane / 16)
  //   V, for the vector products: token ROWS st + lane / CH, d = 8 (lane % CH)
  const uint32_t kl = (uint32_t)((lane & 15) * D + (lane >> 4) * 8) * 2u;
  const int vrow = lane / CH, vch = lane % CH;
  const uint32_t vl = (uint32_t)(vrow * D + vch * 8) * 2u;

  u32x4 kr[RING][KST], vr[RING][VST];
  auto issue = [&](int lb, int slot) {
    const int64_t phys = table[lb];
    const char* kb = kc + (phys * p.h_kv + kvh) * blk_bytes + kl;
    const char* vb = vc + (phys * p.h_kv + kvh) * blk_bytes + vl;
#pragma unroll
    for (int st = 0; st < KST; ++st) kr[slot][st] = *(const u32x4*)(kb + st * 64);
#pragma unroll
    for (int st = 0; st < VST; ++st) vr[slot][st] = *(const u32x4*)(vb + st * ROWS * D * 2);
  };

  // running state: reference max per head (identical in all lanes),
  // per-lane partial sums of probabilities and output partials
  float m_ref[GP];
  float l_part[4];    // heads (lane/16)*4 + r, over this lane's tokens
  float oa[GP][8];    // heads x 8 d of column chunk vch, over tokens of row vrow
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    m_ref[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) oa[g][e] = 0.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) l_part[r] = 0.f;

  auto process = [&](int lb, int slot) {
    // ---- scores of 16 tokens x (up to 16) heads on the matrix cores ----
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KST; ++st) acc = TT::mma16(qa[st], kr[slot][st], acc);
    // lane holds token lb*16 + lane%16, heads (lane/16)*4 + r; tokens past
    // the context are replaced by -inf (never multiplied)
    const bool tv = tok0 + lb * kDecBS + (lane & 15) < ctx;
    float sc[4], bm[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = tv ? acc[r] : -INFINITY;
      bm[r] = sc[r];
    }
    // block max per head over the 16 tokens (lanes of one 16-lane row)
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) bm[r] = fmaxf(bm[r], __shfl_xor(bm[r], sh, 16));
    // every lane learns the block max of every head through LDS
    const int grow_row = lane >> 4;
    if ((lane & 15) == 0 && grow_row * 4 < GP) {
#pragma unroll
      for (int r = 0; r < 4; ++r) xm[grow_row * 4 + r] = bm[r] * c;
    }
    // (all lanes see the same block maxima, so `grow` is wave-uniform)
    float alpha[GP];
    bool any_grow = false;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float t = xm[g];
      const bool grow = t > m_ref[g] + TAU;
      alpha[g] = fast_exp2(grow ? m_ref[g] - t : 0.f);
      m_ref[g] = grow ? t : m_ref[g];
      any_grow = any_grow || grow;
    }
    if (any_grow) {
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) oa[g][e] *= alpha[g];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (grow_row * 4 + r < GP) l_part[r] *= alpha[grow_row * 4 + r];
    }
    float mine_m[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mine_m[r] = (grow_row * 4 + r < GP) ? m_ref[grow_row * 4 + r] : 0.f;
    // probabilities relative to the reference, to LDS as [token][head]
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mm = (mine_m[r] == -INFINITY) ? 0.f : mine_m[r];
      pr[r] = fast_exp2(fmaf(sc[r], c, -mm));
      l_part[r] += pr[r];
    }
    if (grow_row * 4 < GP)
      *(f32x4*)(xp + (lane & 15) * GP + grow_row * 4) = f32x4{pr[0], pr[1], pr[2], pr[3]};
    // ---- O += p v on the vector ALUs (V rows past the context are zero) ----
    const bool last = (tok0 + (lb + 1) * kDecBS > ctx);
#pragma unroll
    for (int st = 0; st < VST; ++st) {
      const int tok = st * ROWS + vrow;
      u32x4 vv = vr[slot][st];
      if (last && tok0 + lb * kDecBS + tok >= ctx) vv = u32x4{0, 0, 0, 0};
      float vf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vf[2 * w] = TT::lo(vv[w]);
        vf[2 * w + 1] = TT::hi(vv[w]);
      }
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 pv = *(const f32x4*)(xp + tok * GP + g4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) oa[g4 + r][e] = fmaf(pv[r], vf[e], oa[g4 + r][e]);
      }
    }
  };

  // ---- stream the partition's blocks through a ring of RING loads ----
#pragma unroll
  for (int j = 0; j < RING; ++j)
    if (j < nblk) issue(j, j);
  for (int i = 0; i < nblk; i += RING) {
#pragma unroll
    for (int j = 0; j < RING; ++j) {
      const int lb = i + j;
      if (lb < nblk) {
        process(lb, j);
        if (lb + RING < nblk) issue(lb + RING, j);
      }
    }
  }

  // ---- merge lanes: sums per head over the 16 tokens of a row, O over rows ----
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) l_part[r] += __shfl_xor(l_part[r], sh, 16);
  if ((lane & 15) == 0 && (lane >> 4) * 4 < GP) {
#pragma unroll
    for (int r = 0; r < 4; ++r) xm[GP + (lane >> 4) * 4 + r] = l_part[r];
  }
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = oa[g][e];
      for (int sh = CH; sh < 64; sh <<= 1) x += __shfl_xor(x, sh);
      oa[g][e] = x;
    }
  if (lane < CH) {
    for (int g = 0; g < group; ++g) {
      const float l = xm[GP + g];
      const int head = head0 + g;
      if (nparts == 1) {
        const float inv = 1.f / l;
        T* og = (T*)p.o + ((int64_t)s * p.h_q + head) * D + lane * 8;
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = TT::pack2(oa[g][2 * k] * inv, oa[g][2 * k + 1] * inv);
        *(u32x4*)og = w;
        if (p.lse != nullptr && lane == 0)
          p.lse[(int64_t)s * p.h_q + head] = (m_ref[g] + __log2f(l)) * kLn2;
      } else {
        const int64_t slot = ((int64_t)s * p.h_q + head) * p.max_parts + part;
        float* dst = p.ws_o + slot * D + lane * 8;
        *(f32x4*)dst = f32x4{oa[g][0], oa[g][1], oa[g][2], oa[g][3]};
        *(f32x4*)(dst + 4) = f32x4{oa[g][4], oa[g][5], oa[g][6], oa[g][7]};
        if (lane == 0) {
          p.ws_ml[slot * 2 + 0] = m_ref[g];
          p.ws_ml[slot * 2 + 1] = l;
        }
      }
    }
  }
}

// Merge the partitions of one (head, sequence): M = max_p m_p,
// O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
template <typename TT>
__global__ __launch_bounds__(128) void paged_decode_combine_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  const int h = blockIdx.x, s = blockIdx.y;
  const int ctx = p.context_lens[s];
  const int nparts = (ctx + kDecPart - 1) / kDecPart;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)s * p.h_q + h) * p.max_parts;
  float M = -INFINITY;
  for (int pp = 0; pp < nparts; ++pp) M = fmaxf(M, p.ws_ml[(base + pp) * 2]);
  float L = 0.f;
  for (int pp = 0; pp < nparts; ++pp)
    L += fast_exp2(p.ws_ml[(base + pp) * 2] - M) * p.ws_ml[(base + pp) * 2 + 1];
  for (int dd = threadIdx.x; dd < p.head_dim; dd += blockDim.x) {
    float acc = 0.f;
    for (int pp = 0; pp < nparts; ++pp)
      acc += fast_exp2(p.ws_ml[(base + pp) * 2] - M) * p.ws_o[(base + pp) * p.head_dim + dd];
    ((T*)p.o)[((int64_t)s * p.h_q + h) * p.head_dim + dd] = (T)(acc / L);
  }
  if (p.lse != nullptr && threadIdx.x == 0) p.lse[(int64_t)s * p.h_q + h] = (M + __log2f(L)) * kLn2;
}

size_t decode_workspace_bytes(int num_seqs, int h_q, int head_dim, int max_context_len) {
  if (num_seqs <= 0 || h_q <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = (max_context_len + kDecPart - 1) / kDecPart;
  if (parts <= 1) return 0;
  const int64_t slots = (int64_t)num_seqs * h_q * parts;
  return (size_t)(slots * head_dim * 4 + slots * 2 * 4);
}

int decode_max_parts(int max_context_len) {
  return max_context_len <= 0 ? 1 : (max_context_len + kDecPart - 1) / kDecPart;
}

template <typename TT, int D, int GP>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.max_parts, p.h_kv, p.num_seqs);
  constexpr int RING = GP <= 4 ? 3 : 2;
  hipLaunchKernelGGL((paged_decode_split_kernel<TT, D, GP, RING>), grid, dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.max_parts > 1) {
    hipLaunchKernelGGL((paged_decode_combine_kernel<TT>), dim3(p.h_q, p.num_seqs), dim3(128), 0,
                       stream, p);
    e = hipGetLastError();
  }
  return e;
}

template <typename TT>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const int gp = p.group <= 4 ? 4 : (p.group <= 8 ? 8 : 16);
  if (p.head_dim == 64) {
    if (gp == 4) return launch_decode_t<TT, 64, 4>(p, stream);
    if (gp == 8) return launch_decode_t<TT, 64, 8>(p, stream);
    return launch_decode_t<TT, 64, 16>(p, stream);
  }
  if (gp == 4) return launch_decode_t<TT, 128, 4>(p, stream);
  if (gp == 8) return launch_decode_t<TT, 128, 8>(p, stream);
  return launch_decode_t<TT, 128, 16>(p, stream);
}

hipError_t launch_decode(int dtype, const DecodeParams& p, hipStream_t stream) {
  if (dtype == 2) return launch_decode_d<BF16>(p, stream);
  return launch_decode_d<F16>(p, stream);
}

}  // namespace attn
