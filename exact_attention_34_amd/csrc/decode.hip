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
constexpr int kDecWaves = 4;

template <typename TT, int D, int GP>
__global__ __launch_bounds__(256) void paged_decode_split_kernel(DecodeParams p) {
  typedef typename TT::elem T;
  constexpr int NB = kDecPart / kDecBS;  // 32 blocks per partition
  constexpr int BPW = NB / kDecWaves;    // 8 blocks per wave
  constexpr int INFL = 4;                // blocks whose K loads are in flight together
  static_assert(GP % 4 == 0 && GP <= 16, "padded group");
  // scores / probabilities [token][head]; reused as the cross-wave merge buffer
  constexpr int SC_FLOATS = kDecPart * GP;
  constexpr int OB_FLOATS = kDecWaves * GP * D;
  __shared__ __attribute__((aligned(16))) float sbuf[SC_FLOATS > OB_FLOATS ? SC_FLOATS : OB_FLOATS];
  __shared__ float red[kDecWaves][GP];
  __shared__ float stat_m[GP], stat_l[GP];

  const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ctx = p.context_lens[s];
  const int group = p.group;
  const int head0 = kvh * group;

  if (ctx <= 0) {
    // empty context: o = 0, lse = -inf (written once, by partition 0)
    if (part == 0) {
      T* og = (T*)p.o + ((int64_t)s * p.h_q + head0) * D;
      for (int i = tid; i < group * D; i += 256) og[i] = (T)0.f;
      if (p.lse != nullptr && tid < group) p.lse[(int64_t)s * p.h_q + head0 + tid] = -INFINITY;
    }
    return;
  }
  const int tok0 = part * kDecPart;
  if (tok0 >= ctx) return;
  const int ntok = min(kDecPart, ctx - tok0);
  const int nblk = (ntok + kDecBS - 1) / kDecBS;
  const int nparts = (ctx + kDecPart - 1) / kDecPart;
  const int32_t* table = p.block_table + (int64_t)s * p.max_blocks_per_seq + tok0 / kDecBS;
  const T* kc = (const T*)p.k_cache;
  const T* vc = (const T*)p.v_cache;

  // ---- query heads as the A operand (rows = heads, zero padded) ----
  u32x4 qa[D / 32];
  {
    const int g = lane & 15;
    const T* qg = (const T*)p.q + ((int64_t)s * p.h_q + head0 + g) * D + (lane >> 4) * 8;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      qa[st] = u32x4{0, 0, 0, 0};
      if (g < group) qa[st] = *(const u32x4*)(qg + 32 * st);
    }
  }

  // ---- phase A: scores ----
#pragma unroll
  for (int i0 = 0; i0 < BPW; i0 += INFL) {
    u32x4 kr[INFL][D / 32];
    int lbs[INFL];
#pragma unroll
    for (int j = 0; j < INFL; ++j) {
      const int lb = wave * BPW + i0 + j;
      lbs[j] = lb;
      if (lb < nblk) {
        const int64_t phys = table[lb];
        const T* kb = kc + (phys * p.h_kv + kvh) * (kDecBS * D) + (lane & 15) * D + (lane >> 4) * 8;
#pragma unroll
        for (int st = 0; st < D / 32; ++st) kr[j][st] = *(const u32x4*)(kb + 32 * st);
      }
    }
#pragma unroll
    for (int j = 0; j < INFL; ++j) {
      const int lb = lbs[j];
      if (lb < nblk) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < D / 32; ++st) acc = TT::mma16(qa[st], kr[j][st], acc);
        // lane holds token lb*16 + lane%16, heads (lane/16)*4 + 0..3
        const int t = lb * kDecBS + (lane & 15);
        const bool tv = (tok0 + t) < ctx;
        const int g0 = (lane >> 4) * 4;
        if (g0 < GP) {
          f32x4 sv;
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[r] = tv ? acc[r] * p.scale_log2 : -INFINITY;
          *(f32x4*)(sbuf + t * GP + g0) = sv;
        }
      }
    }
  }
  __syncthreads();

  // ---- partition max per head ----
  {
    float mx[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) mx[g] = -INFINITY;
    for (int t = tid; t < ntok; t += 256) {
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        const f32x4 v = *(const f32x4*)(sbuf + t * GP + g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[g4 + r] = fmaxf(mx[g4 + r], v[r]);
      }
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], sh));
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < GP; ++g) red[wave][g] = mx[g];
    }
    __syncthreads();
    if (tid < GP) {
      float m = red[0][tid];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) m = fmaxf(m, red[w][tid]);
      stat_m[tid] = m;
    }
    __syncthreads();
  }

  // ---- probabilities in place, partition sum per head ----
  {
    float sm[GP], m[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      sm[g] = 0.f;
      m[g] = stat_m[g];
    }
    for (int t = tid; t < ntok; t += 256) {
#pragma unroll
      for (int g4 = 0; g4 < GP; g4 += 4) {
        f32x4 v = *(const f32x4*)(sbuf + t * GP + g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = fast_exp2(v[r] - m[g4 + r]);
          sm[g4 + r] += v[r];
        }
        *(f32x4*)(sbuf + t * GP + g4) = v;
      }
    }
#pragma unroll
    for (int g = 0; g < GP; ++g) {
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) sm[g] += __shfl_xor(sm[g], sh);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < GP; ++g) red[wave][g] = sm[g];
    }
    __syncthreads();
    if (tid < GP) {
      float l = red[0][tid];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) l += red[w][tid];
      stat_l[tid] = l;
    }
    // (probabilities written above are read after the next barrier)
  }

  // ---- phase B: O_part = sum_t p_t v_t ----
  const int r4 = lane >> 4;   // token row within a group of 4
  const int c16 = lane & 15;  // 8-element column chunk of d (D = 128) ...
  constexpr int CH = D / 8;   // ... chunks per row: 16 (D=128) or 8 (D=64)
  constexpr int ROWS = 64 / CH;   // token rows per load instruction: 4 or 8
  float oa[GP][8];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) oa[g][e] = 0.f;
  __syncthreads();
  {
    const int cch = lane % CH;
    const int rr = lane / CH;
#pragma unroll 2
    for (int i = 0; i < BPW; ++i) {
      const int lb = wave * BPW + i;
      if (lb >= nblk) break;
      const int64_t phys = table[lb];
      const T* vb = vc + (phys * p.h_kv + kvh) * (kDecBS * D) + cch * 8;
      u32x4 vv[kDecBS / ROWS];
#pragma unroll
      for (int st = 0; st < kDecBS / ROWS; ++st) {
        const int tok = st * ROWS + rr;
        vv[st] = u32x4{0, 0, 0, 0};
        if (tok0 + lb * kDecBS + tok < ctx) vv[st] = *(const u32x4*)(vb + tok * D);
      }
#pragma unroll
      for (int st = 0; st < kDecBS / ROWS; ++st) {
        const int t = lb * kDecBS + st * ROWS + rr;
        float vf[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vf[2 * w] = TT::lo(vv[st][w]);
          vf[2 * w + 1] = TT::hi(vv[st][w]);
        }
#pragma unroll
        for (int g4 = 0; g4 < GP; g4 += 4) {
          // tokens past the context have p = 0 exactly and v = 0
          const f32x4 pv = (tok0 + t < ctx) ? *(const f32x4*)(sbuf + t * GP + g4)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) oa[g4 + r][e] = fmaf(pv[r], vf[e], oa[g4 + r][e]);
        }
      }
    }
  }
  (void)r4;
  (void)c16;

  // ---- merge: lanes sharing a d chunk, then waves ----
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = oa[g][e];
      for (int sh = CH; sh < 64; sh <<= 1) x += __shfl_xor(x, sh);
      oa[g][e] = x;
    }
  __syncthreads();  // all waves are done reading probabilities
  if (lane < CH) {
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float* dst = sbuf + (wave * GP + g) * D + lane * 8;
      *(f32x4*)(dst) = f32x4{oa[g][0], oa[g][1], oa[g][2], oa[g][3]};
      *(f32x4*)(dst + 4) = f32x4{oa[g][4], oa[g][5], oa[g][6], oa[g][7]};
    }
  }
  __syncthreads();
  for (int idx = tid; idx < group * D; idx += 256) {
    const int g = idx / D, dd = idx - g * D;
    float acc = sbuf[(0 * GP + g) * D + dd];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) acc += sbuf[(w * GP + g) * D + dd];
    const int head = head0 + g;
    if (nparts == 1) {
      const float l = stat_l[g];
      ((T*)p.o)[((int64_t)s * p.h_q + head) * D + dd] = (T)(acc / l);
      if (p.lse != nullptr && dd == 0)
        p.lse[(int64_t)s * p.h_q + head] = (stat_m[g] + __log2f(l)) * kLn2;
    } else {
      const int64_t slot = ((int64_t)s * p.h_q + head) * p.max_parts + part;
      p.ws_o[slot * D + dd] = acc;
      if (dd == 0) {
        p.ws_ml[slot * 2 + 0] = stat_m[g];
        p.ws_ml[slot * 2 + 1] = stat_l[g];
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
  hipLaunchKernelGGL((paged_decode_split_kernel<TT, D, GP>), grid, dim3(256), 0, stream, p);
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
