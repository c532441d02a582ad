// Shared device-side helpers for the gfx950 attention kernels: vector types,
// matrix-core wrappers, 16-bit packing and launch parameter structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type traits: matrix-core products with fp32 accumulation and the
// fp32 -> 16-bit round-to-nearest-even packing of two values into one dword.
struct BF16 {
  typedef __bf16 elem;
  static constexpr bool kIsBf16 = true;
  // 32x32x16: A is 32 rows x 16 k, B is 16 k x 32 columns; each lane holds 8
  // consecutive k values of one row (A) / one column (B).
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // 16x16x16: each lane holds 4 consecutive k values of one row (A) / column (B)
  __device__ static inline f32x4 mma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // acc + (both packed values): the fp32 sum of the rounded probabilities
  __device__ static inline float sum2(uint32_t w, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
  }
  // acc + a.x * b.x + a.y * b.y over packed pairs, fp32 accumulation
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  }
  // widen the low / high 16-bit half of a dword to fp32 (exact)
  __device__ static inline float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
  __device__ static inline float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
};

struct F16 {
  typedef _Float16 elem;
  static constexpr bool kIsBf16 = false;
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  __device__ static inline float sum2(uint32_t w, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
  }
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
  }
  __device__ static inline float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static inline float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

// Join the low halves (lo16) / high halves (hi16) of two dwords: the result
// holds a's half in bits 0..15 and b's half in bits 16..31.
__device__ inline uint32_t join_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ inline uint32_t join_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders a wave's LDS writes before its later LDS reads of data other lanes
// wrote (possibly through a different element type).  The hardware executes
// one wave's LDS operations in order; this only stops the compiler from
// moving the reads above the writes.
__device__ inline void lds_order() { asm volatile("" ::: "memory"); }

// Value of `v` held by the lane that DPP control CTRL selects in this lane's row.
template <int CTRL>
__device__ inline float dpp_src(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xf, 0xf, false));
}
// max / sum of a value over the 16 lanes of its DPP row (lanes 16k .. 16k+15):
// xor 1, xor 2 within quads (quad_perm [1,0,3,2], [2,3,0,1]), then the
// half-row mirror and the row mirror.
__device__ inline float row16_max(float x) {
  x = fmaxf(x, dpp_src<0xB1>(x));
  x = fmaxf(x, dpp_src<0x4E>(x));
  x = fmaxf(x, dpp_src<0x141>(x));
  x = fmaxf(x, dpp_src<0x140>(x));
  return x;
}
__device__ inline float row16_sum(float x) {
  x += dpp_src<0xB1>(x);
  x += dpp_src<0x4E>(x);
  x += dpp_src<0x141>(x);
  x += dpp_src<0x140>(x);
  return x;
}

// max / sum of a value over the lane pair (l, l xor 32): v_permlane32_swap of
// x with itself leaves {x[l % 32], x[l % 32 + 32]} in the two results.
__device__ inline float pair_max32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ inline float pair_sum32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Raw buffer resource over [base, base + bytes): loads whose byte offset
// (the VGPR offset) is at or past `bytes` return zero.
// A compile-time int as a type, for passing constants to generic lambdas.
template <int V>
struct IntC {
  static constexpr int value = V;
};

// A pointer that is the same in every lane, marked as such for the compiler
// (a buffer resource must sit in scalar registers).
__device__ inline const void* uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same with the non-temporal hint (cache policy bit 1): data read once
// and streamed past.
__device__ inline u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
// 16 bytes per lane straight from memory into LDS: the wave's 64 lanes fill
// 1 KiB of consecutive LDS starting at `lds` (a wave-uniform address), lane i
// at lds + 16 i.  Completion is tracked by vmcnt.
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, 0);
}
// The same with a wave-uniform byte offset `soff` added to every lane's.
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, soff, 0, 0);
}
// 4 bytes per lane straight into LDS: the wave fills 256 consecutive bytes.
__device__ inline void buf_load4_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           off, 0, 0, 0);
}

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_n, qs_h;
  int64_t ks_b, ks_n, ks_h;
  int64_t vs_b, vs_n, vs_h;
  int64_t os_b, os_n, os_h;
  int batch, n_q, n_k, h_q, h_kv, group;
  uint32_t k_bytes, v_bytes;  // byte extent of one (batch, kv head) slice of k / v
  uint32_t q_bytes;           // byte extent of one (batch, head) slice of q
  // paged K/V (prefill over a paged cache): k and v are the caches
  const int32_t* block_table;    // [batch][max_blocks_per_seq]
  const int32_t* context_lens;   // [batch]: keys of each sequence
  int max_blocks_per_seq;
  int hpw;          // query heads per workgroup (of one KV head's group)
  int n_qtiles;     // ceil(n_q / rows per head of a workgroup)
  int num_items;    // n_qtiles * batch * h_q / hpw
  int xcd_chunk;    // work items kept together on one XCD (0 = no remap)
  float scale_log2;  // softmax_scale * log2(e)
};

// Backward pass (bf16 / fp16).  Element strides of (batch, sequence, head);
// the head_dim axis is contiguous.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // [B][Hq][Nq] natural-log log-sum-exp of the forward pass
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // [B][Hq][Nq] workspace: rowsum(dO * O)
  float* lse2;        // [B][Hq][Nq] workspace: lse * log2(e)
  int64_t qs_b, qs_n, qs_h;
  int64_t ks_b, ks_n, ks_h;
  int64_t vs_b, vs_n, vs_h;
  int64_t os_b, os_n, os_h;
  int64_t dos_b, dos_n, dos_h;
  int64_t dqs_b, dqs_n, dqs_h;
  int64_t dks_b, dks_n, dks_h;
  int64_t dvs_b, dvs_n, dvs_h;
  int batch, n_q, n_k, h_q, h_kv, group;
  uint32_t q_bytes, k_bytes, v_bytes, do_bytes;  // byte extents of one (batch, head) slice
  int n_qt, n_kt;     // query / key tiles
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
};

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* o;
  float* lse;
  float* ws_o;    // [waves][2][group][head_dim] partial outputs
  float* ws_ml;   // [waves][2][group][2]  (max in log2 units, sum)
  int32_t* ws_unit;  // [num_seqs][h_kv][2]: first wave of the unit, waves it spans
  int num_seqs, h_q, h_kv, group, head_dim;
  int max_blocks_per_seq;
  float scale_log2;
  // Shared-prefix decode only (first_block == nullptr otherwise).  Sequences
  // [group_starts[g], group_starts[g+1]) form group g; the first
  // prefix_lens[g] tokens of each are the group's common prefix, held in the
  // same blocks.  The prefix kernel fills seq_meta with each sequence's
  // prefix length in blocks (first_block), its group (seq_group) and its
  // index in the group (seq_member); the split kernel then covers only
  // blocks at or past first_block[s].
  const int32_t* group_starts;
  const int32_t* prefix_lens;
  int32_t* seq_meta;            // [3][num_seqs]
  const int32_t* first_block;   // seq_meta
  const int32_t* seq_group;     // seq_meta + num_seqs
  const int32_t* seq_member;    // seq_meta + 2 num_seqs
  float* ws_suf_o;    // [num_seqs][h_q][head_dim] suffixes finished inside one wave
  float* ws_suf_ml;   // [num_seqs][h_q][2]
  float* ws_pre_o;    // [prefix items][32][head_dim] one partial per item and query
  float* ws_pre_ml;   // [prefix items][32][2]
  int num_groups;
  int n_rt;           // 32-query tiles per (group, KV head)
  int n_ch;           // prefix chunks per (group, KV head, query tile)
  int chunk_blocks;   // prefix blocks per chunk
};

// Cut of the prefix work of shared-prefix decode (host side).
struct SharedPlan {
  int n_rt, n_ch, chunk_blocks;
  int64_t items;   // workgroups of the prefix kernel
};

// Read-only metadata (context lengths, block tables) read through the
// constant address space: at a wave-uniform index that is a scalar load, which
// keeps the value in scalar registers and leaves the vector-memory counter to
// the K/V loads.
__device__ inline int ld_meta(const int32_t* ptr, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)ptr)[i];
}

}  // namespace attn
