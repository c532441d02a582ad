// Prefill kernels: exact attention O = softmax(Q K^T * scale) V in one fused,
// tiled pass with the online-softmax update ("Other people's interview
// notes", question "explain FlashAttention", part 2), never writing the
// N x N score or probability matrix to device memory.
//
// 16-bit kernel (bf16 / fp16), gfx950 matrix cores:
//   * a workgroup of 4 waves owns BM = 128 query rows of one (batch, head);
//     each wave owns 32 rows, whose Q fragment stays in VGPRs for the whole
//     kernel;
//   * the loop walks the visible key range in BN = 64 tiles.  K tiles are
//     copied to LDS as they are in memory ([key][d]); V tiles are transposed
//     in registers on the way in and stored [d][key], so that both products
//     read their operand with one 16-byte LDS load per lane.  Two LDS stages:
//     tile j+1 is fetched from HBM into registers while tile j is computed;
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
//     applied only on tiles that cross the diagonal, and workgroups are issued
//     longest first.  Work items that share K/V (the query heads of one GQA
//     group) are kept together on one XCD.
//
// fp32 kernel: plain fp32 arithmetic on the vector ALUs (the fp32 matrix
// rate equals the vector rate on this chip); four lanes share a query row.
#include "common.h"

namespace attn {

// ----------------------------------------------------------------------------
// work-item mapping
// ----------------------------------------------------------------------------
// Workgroup i runs on XCD i % 8.  Items are numbered longest-first (query
// tile descending when causal), then batch, then head; consecutive heads of a
// GQA group are consecutive items.  With xcd_chunk = c > 0 (and num_items a
// multiple of 8c), chunks of c consecutive items are dealt round-robin to the
// XCDs, so the c workgroups of a chunk run on the same XCD and share its L2.
__device__ inline int remap_item(int i, int num_items, int chunk) {
  if (chunk <= 1 || (num_items % (8 * chunk)) != 0) return i;
  const int x = i & 7, pos = i >> 3;
  const int round = pos / chunk, within = pos - round * chunk;
  return (round * 8 + x) * chunk + within;
}

// ----------------------------------------------------------------------------
// 16-bit matrix-core kernel
// ----------------------------------------------------------------------------
template <typename TT, int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_mfma_kernel(FwdParams p) {
  typedef typename TT::elem T;
  constexpr int BM = 128, BN = 64;
  constexpr int KLD = D + 8;   // LDS row stride of K, elements (16 B pad)
  constexpr int VLD = BN + 8;  // LDS row stride of V^T, elements (16 B pad)
  constexpr int KSZ = BN * KLD;
  constexpr int VSZ = D * VLD;
  constexpr int STAGE = KSZ + VSZ;
  constexpr int KCH = BN * D / 8 / 256;   // 16-byte K chunks per thread
  constexpr int VUNITS = (BN / 8) * (D / 4);  // (8 keys x 4 d) V units
  static_assert(KCH * 256 * 8 == BN * D, "K tile split");
  static_assert(VUNITS <= 256, "V tile split");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane
  const int hi = lane >> 5;    // which half of the k slots / key rows

  const int item = remap_item(blockIdx.x, p.num_items, p.xcd_chunk);
  const int bh = p.batch * p.h_q;
  const int rank = item / bh;
  const int rem = item - rank * bh;
  const int b = rem / p.h_q;
  const int h = rem - b * p.h_q;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - rank) : rank;
  const int q0 = qt * BM;
  const int kvh = h / p.group;
  const int off = p.n_k - p.n_q;

  int kend = p.n_k;
  if (CAUSAL) {
    const int qlast = min(q0 + BM, p.n_q) - 1;
    kend = min(p.n_k, max(0, qlast + off + 1));
  }
  const int ntiles = (kend + BN - 1) / BN;

  const T* Qg = (const T*)p.q + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h;
  const T* Kg = (const T*)p.k + (int64_t)b * p.ks_b + (int64_t)kvh * p.ks_h;
  const T* Vg = (const T*)p.v + (int64_t)b * p.vs_b + (int64_t)kvh * p.vs_h;

  // Q fragment (B operand of S^T = K Q^T): column = query, k = d.
  const int qrow = q0 + wave * 32 + col;
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    if (qrow < p.n_q) qf[s] = *(const u32x4*)(Qg + (int64_t)qrow * p.qs_n + 16 * s + hi * 8);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY;  // running max, log2 units (same in lanes l, l^32)
  float l_run = 0.f;        // running sum over this lane's keys

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[KCH];
  u32x2 vreg[8];
  // V unit of this thread: 8 keys x 4 consecutive d.  Within each group of
  // 16 keys the LDS position order is keys 0-3, 8-11, 4-7, 12-15, which is
  // the order in which the score registers of a lane feed the P^T operand.
  const int vdq = tid % (D / 4);
  const int vko = tid / (D / 4);
  const int vkey_base = (vko >> 1) * 16 + (vko & 1) * 4;

  auto gload = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      const int key = k0 + row;
      kreg[c] = u32x4{0, 0, 0, 0};
      if (key < p.n_k) kreg[c] = *(const u32x4*)(Kg + (int64_t)key * p.ks_n + ch * 8);
    }
    if (tid < VUNITS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = k0 + vkey_base + (j & 3) + (j >> 2) * 8;
        vreg[j] = u32x2{0, 0};
        if (key < p.n_k) vreg[j] = *(const u32x2*)(Vg + (int64_t)key * p.vs_n + vdq * 4);
      }
    }
  };
  auto lstore = [&](int stage) {
    uint16_t* Ks = smem + stage * STAGE;
    uint16_t* Vs = Ks + KSZ;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + 256 * c;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      *(u32x4*)(Ks + row * KLD + ch * 8) = kreg[c];
    }
    if (tid < VUNITS) {
      // transpose 8 keys x 4 d into 4 rows (one per d) of 8 keys
      u32x4 w0, w1, w2, w3;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 a = vreg[2 * w], c2 = vreg[2 * w + 1];
        w0[w] = join_lo16(a.x, c2.x);
        w1[w] = join_hi16(a.x, c2.x);
        w2[w] = join_lo16(a.y, c2.y);
        w3[w] = join_hi16(a.y, c2.y);
      }
      uint16_t* vrow = Vs + (vdq * 4) * VLD + vko * 8;
      *(u32x4*)(vrow + 0 * VLD) = w0;
      *(u32x4*)(vrow + 1 * VLD) = w1;
      *(u32x4*)(vrow + 2 * VLD) = w2;
      *(u32x4*)(vrow + 3 * VLD) = w3;
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const uint16_t* Ks = smem + stage * STAGE;
    const uint16_t* Vs = Ks + KSZ;

    // ---- S^T = K Q^T for two 32-key sub-tiles ----
    f32x16 st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[sub][r] = 0.f;
      const uint16_t* kp = Ks + (sub * 32 + col) * KLD + hi * 8;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) st[sub] = TT::mma32(*(const u32x4*)(kp + 16 * s), qf[s], st[sub]);
    }

    // ---- scale, mask, online softmax ----
    const int k0 = kt * BN;
    const bool need_mask = (k0 + BN > p.n_k) || (CAUSAL && (k0 + BN - 1 > q0 + off));
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float t = st[sub][r] * p.scale_log2;
        if (need_mask) {
          const int key = k0 + sub * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const bool vis = (key < p.n_k) && (!CAUSAL || key <= qrow + off);
          t = vis ? t : -INFINITY;
        }
        st[sub][r] = t;
        tmax = fmaxf(tmax, t);
      }
    tmax = fmaxf(tmax, xor32(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
    u32x4 pb[4];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(st[sub][r] - m_use);
        const float p1 = fast_exp2(st[sub][r + 1] - m_use);
        psum += p0 + p1;
        pb[sub * 2 + (r >> 3)][(r & 7) >> 1] = TT::pack2(p0, p1);
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const uint16_t* vp = Vs + (t * 32 + col) * VLD + hi * 8;
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks)
        oacc[t] = TT::mma32(*(const u32x4*)(vp + ks * 16), pb[ks], oacc[t]);
    }

    if (kt + 1 < ntiles) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE ----
  const float l_tot = l_run + xor32(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < p.n_q) {
    T* Og = (T*)p.o + (int64_t)b * p.os_b + (int64_t)qrow * p.os_n + (int64_t)h * p.os_h;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w.x = TT::pack2(oacc[t][4 * g + 0] * inv, oacc[t][4 * g + 1] * inv);
        w.y = TT::pack2(oacc[t][4 * g + 2] * inv, oacc[t][4 * g + 3] * inv);
        *(u32x2*)(Og + t * 32 + g * 8 + hi * 4) = w;
      }
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
template <typename TT, int D, bool CAUSAL>
static hipError_t launch_mfma(FwdParams p, hipStream_t stream) {
  constexpr int BM = 128;
  p.n_qtiles = (p.n_q + BM - 1) / BM;
  p.num_items = p.n_qtiles * p.batch * p.h_q;
  p.xcd_chunk = p.group > 1 ? p.group : 1;
  hipLaunchKernelGGL((attn_fwd_mfma_kernel<TT, D, CAUSAL>), dim3(p.num_items), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(FwdParams p, hipStream_t stream) {
  dim3 grid((p.n_q + 63) / 64, p.h_q, p.batch);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// dtype: 0 f32, 1 f16, 2 bf16.  Returns the launch status.
hipError_t launch_prefill(int dtype, int head_dim, bool causal, const FwdParams& p,
                          hipStream_t stream) {
#define ATTN_DISPATCH_D(FN, ...)                                          \
  (head_dim == 64 ? (causal ? FN<__VA_ARGS__ 64, true>(p, stream)         \
                            : FN<__VA_ARGS__ 64, false>(p, stream))       \
                  : (causal ? FN<__VA_ARGS__ 128, true>(p, stream)        \
                            : FN<__VA_ARGS__ 128, false>(p, stream)))
  if (dtype == 2) return ATTN_DISPATCH_D(launch_mfma, BF16,);
  if (dtype == 1) return ATTN_DISPATCH_D(launch_mfma, F16,);
  return ATTN_DISPATCH_D(launch_f32, );
#undef ATTN_DISPATCH_D
}

}  // namespace attn
