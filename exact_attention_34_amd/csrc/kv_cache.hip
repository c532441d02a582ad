// Paged KV cache maintenance (PagedAttention, tutorial "Chapter 3 Advanced
// principles", section 3.0: fixed-size KV blocks, a per-sequence block table,
// blocks shared between sequences and copied before a shared block is
// written):
//   * kv_write_kernel scatters the K and V rows of new tokens into their
//     physical slots (slot = block * block_size + offset);
//   * kv_copy_blocks_kernel copies whole blocks (all KV heads of K and V),
//     the device half of copy-on-write.
// Both are plain HBM copies: 16 bytes per lane, whole rows per token.
#include "common.h"

namespace attn {

struct KvWriteParams {
  const void* k_new;
  const void* v_new;
  int64_t ks_t, ks_h;   // element strides of (token, head) of k_new
  int64_t vs_t, vs_h;
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  int n_tokens, h_kv, head_dim, block_size;
  int64_t num_slots;    // num_blocks * block_size
};

// One workgroup per token; each lane moves 16-byte chunks of the token's
// h_kv rows of K and then of V.  Slots outside [0, num_slots) (-1 marks a
// padding token) are skipped.
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteParams p) {
  const int t = blockIdx.x;
  const int64_t slot = p.slots[t];
  if (slot < 0 || slot >= p.num_slots) return;
  const int64_t blk = slot / p.block_size, off = slot - blk * p.block_size;
  const int cpr = p.head_dim / 8;   // 16-byte chunks per row
  const int n = p.h_kv * cpr;
  for (int i = threadIdx.x; i < 2 * n; i += blockDim.x) {
    const bool is_v = i >= n;
    const int j = is_v ? i - n : i;
    const int h = j / cpr, c = j - h * cpr;
    const uint16_t* src = (const uint16_t*)(is_v ? p.v_new : p.k_new) +
                          (int64_t)t * (is_v ? p.vs_t : p.ks_t) +
                          (int64_t)h * (is_v ? p.vs_h : p.ks_h) + c * 8;
    uint16_t* dst = (uint16_t*)(is_v ? p.v_cache : p.k_cache) +
                    ((blk * p.h_kv + h) * p.block_size + off) * p.head_dim + c * 8;
    *(u32x4*)dst = *(const u32x4*)src;
  }
}

struct KvCopyParams {
  void* k_cache;
  void* v_cache;
  const int32_t* src;
  const int32_t* dst;
  int64_t block_elems;   // h_kv * block_size * head_dim
  int num_blocks;
};

// One workgroup per (source, destination) pair; pairs naming a block outside
// [0, num_blocks) are skipped.
__global__ __launch_bounds__(256) void kv_copy_blocks_kernel(KvCopyParams p) {
  const int i = blockIdx.x;
  const int s = p.src[i], d = p.dst[i];
  if (s < 0 || s >= p.num_blocks || d < 0 || d >= p.num_blocks) return;
  const int64_t chunks = p.block_elems / 8;
  for (int64_t c = threadIdx.x; c < 2 * chunks; c += blockDim.x) {
    const bool is_v = c >= chunks;
    const int64_t j = is_v ? c - chunks : c;
    uint16_t* base = (uint16_t*)(is_v ? p.v_cache : p.k_cache);
    *(u32x4*)(base + (int64_t)d * p.block_elems + j * 8) =
        *(const u32x4*)(base + (int64_t)s * p.block_elems + j * 8);
  }
}

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(kv_write_kernel, dim3(p.n_tokens), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_copy(const KvCopyParams& p, int n_pairs, hipStream_t stream) {
  hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3(n_pairs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
