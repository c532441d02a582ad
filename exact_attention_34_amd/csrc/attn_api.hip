// C ABI of libattn.so (declared in include/attn.h): host-side validation and
// dispatch.  Nothing here allocates device memory or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "common.h"

namespace attn {
hipError_t launch_prefill(int dtype, int head_dim, bool causal, const FwdParams& p,
                          hipStream_t stream);
hipError_t launch_prefill_paged(int dtype, int head_dim, bool causal, const FwdParams& p,
                                hipStream_t stream);
hipError_t launch_decode(int dtype, const DecodeParams& p, int max_context_len, hipStream_t stream);
hipError_t launch_backward(int dtype, int head_dim, bool causal, const BwdParams& p,
                           hipStream_t stream);
hipError_t launch_decode_shared(int dtype, const DecodeParams& p, int64_t items,
                                int max_context_len, hipStream_t stream);
size_t decode_workspace_bytes(int num_seqs, int h_q, int h_kv, int head_dim, int max_context_len);
size_t scratch_capacity();
hipError_t scratch_address(int device, void** out);
int decode_waves(int num_seqs, int h_kv, int max_context_len);
SharedPlan shared_plan(int num_groups, int max_group_size, int h_q, int h_kv, int max_prefix_len);
struct KvWriteParams {
  const void* k_new;
  const void* v_new;
  int64_t ks_t, ks_h;
  int64_t vs_t, vs_h;
  const int32_t* slots;
  void* k_cache;
  void* v_cache;
  int n_tokens, h_kv, head_dim, block_size;
  int64_t num_slots;
};
struct KvCopyParams {
  void* k_cache;
  void* v_cache;
  const int32_t* src;
  const int32_t* dst;
  int64_t block_elems;
  int num_blocks;
};
hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream);
hipError_t launch_kv_copy(const KvCopyParams& p, int n_pairs, hipStream_t stream);
}  // namespace attn

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int elem_size(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Byte offsets of the regions of the shared-prefix decode workspace: the
// split kernel's partials first (as in plain decode), then the per-(sequence,
// head) suffix results, the prefix partials and the per-sequence metadata.
struct SharedWs {
  size_t suf_o, suf_ml, pre_o, pre_ml, meta, total;
};
SharedWs shared_ws(int num_seqs, int h_q, int head_dim, size_t split_bytes, int64_t items) {
  SharedWs w{};
  size_t off = align16(split_bytes);
  w.suf_o = off;
  off = align16(off + (size_t)num_seqs * h_q * head_dim * 4);
  w.suf_ml = off;
  off = align16(off + (size_t)num_seqs * h_q * 2 * 4);
  w.pre_o = off;
  off = align16(off + (size_t)items * 32 * head_dim * 4);
  w.pre_ml = off;
  off = align16(off + (size_t)items * 32 * 2 * 4);
  w.meta = off;
  off = align16(off + (size_t)num_seqs * 3 * 4);
  w.total = off;
  return w;
}

// Checks common to both decode entry points (everything but the workspace);
// on success fills the fields of p that plain decode uses.
int check_decode(const char* fn, int dtype, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                 void* o, float* lse, int num_seqs, int h_q, int h_kv, int head_dim,
                 int block_size, int max_blocks_per_seq, int max_context_len, int num_blocks,
                 float softmax_scale, attn::DecodeParams& p) {
  const std::string f(fn);
  if (dtype != ATTN_F16 && dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, f + ": dtype must be ATTN_F16 or ATTN_BF16");
  if (num_seqs < 0 || h_q < 0 || h_kv < 0 || head_dim < 0 || block_size < 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || num_blocks < 0)
    return fail(ATTN_ERR_SHAPE, f + ": sizes must be non-negative");
  if (h_kv == 0 || h_q == 0 || (h_q % h_kv) != 0)
    return fail(ATTN_ERR_SHAPE, f + ": h_q must be a positive multiple of h_kv");
  if (h_q / h_kv > 16)
    return fail(ATTN_ERR_UNSUPPORTED, f + ": at most 16 query heads per KV head");
  if (head_dim != 64 && head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
  if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, f + ": block_size must be 16");
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(ATTN_ERR_SHAPE, f + ": softmax_scale must be finite and positive");
  if ((int64_t)max_blocks_per_seq * block_size < (int64_t)max_context_len)
    return fail(ATTN_ERR_SHAPE, f + ": max_blocks_per_seq * block_size < max_context_len");
  if (max_context_len > 0 && num_blocks == 0)
    return fail(ATTN_ERR_SHAPE, f + ": num_blocks must be positive");
  if (num_seqs == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr || context_lens == nullptr)
    return fail(ATTN_ERR_NULL, f + ": q, o and context_lens must not be NULL");
  if (max_context_len > 0 && (k_cache == nullptr || v_cache == nullptr || block_table == nullptr))
    return fail(ATTN_ERR_NULL, f + ": k_cache, v_cache and block_table must not be NULL");
  const void* ptrs[4] = {q, k_cache, v_cache, o};
  for (const void* ptr : ptrs)
    if (ptr != nullptr && !aligned16(ptr))
      return fail(ATTN_ERR_ALIGN, f + ": q, caches and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(ATTN_ERR_ALIGN, f + ": block_table, context_lens and lse must be 4-byte aligned");
  if ((int64_t)num_seqs > 65535 || h_q > 65535)
    return fail(ATTN_ERR_UNSUPPORTED, f + ": too many sequences or heads for one launch");
  p = attn::DecodeParams{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.o = o;
  p.lse = lse;
  p.num_seqs = num_seqs;
  p.h_q = h_q;
  p.h_kv = h_kv;
  p.group = h_q / h_kv;
  p.head_dim = head_dim;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.scale_log2 = softmax_scale * attn::kLog2e;
  return ATTN_OK;
}

int check_workspace(const char* fn, void* workspace, size_t workspace_bytes, size_t need) {
  if (need == 0) return ATTN_OK;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, std::string(fn) + ": workspace of " + std::to_string(need) +
                                        " bytes required, got " + std::to_string(workspace_bytes));
  if (!aligned16(workspace))
    return fail(ATTN_ERR_ALIGN, std::string(fn) + ": workspace must be 16-byte aligned");
  return ATTN_OK;
}

// ATTN_VALIDATE set to anything but "" or "0": the paged entry points copy
// their device metadata to the host and range-check it before any launch.
// Read at every call, so a test can switch it.
bool validate_enabled() {
  const char* e = std::getenv("ATTN_VALIDATE");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// n int32 values from device memory to `out`, ordered after the work already
// on `stream` (the caller may have written them there).
int fetch_i32(const char* fn, const int32_t* dev, size_t n, std::vector<int32_t>& out,
              hipStream_t stream) {
  out.assign(n, 0);
  if (n == 0 || dev == nullptr) return ATTN_OK;
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, std::string(fn) + ": copy for ATTN_VALIDATE failed: " +
                                  hipGetErrorString(e));
  return ATTN_OK;
}

// The ATTN_VALIDATE check: host copies of the table, the context lengths
// and (shared-prefix decode) the groups, through attn_validate_paged_tables.
int validate_on_host(const char* fn, hipStream_t stream, const int32_t* block_table,
                     const int32_t* context_lens, int num_seqs, int max_blocks_per_seq,
                     int max_context_len, int num_blocks, int block_size,
                     const int32_t* group_starts, const int32_t* prefix_lens, int num_groups) {
  std::vector<int32_t> tab, ctx, gs, pl;
  int rc = fetch_i32(fn, block_table, (size_t)num_seqs * max_blocks_per_seq, tab, stream);
  if (rc == ATTN_OK) rc = fetch_i32(fn, context_lens, (size_t)num_seqs, ctx, stream);
  if (rc == ATTN_OK && group_starts != nullptr)
    rc = fetch_i32(fn, group_starts, (size_t)num_groups + 1, gs, stream);
  if (rc == ATTN_OK && prefix_lens != nullptr)
    rc = fetch_i32(fn, prefix_lens, (size_t)num_groups, pl, stream);
  if (rc != ATTN_OK) return rc;
  rc = attn_validate_paged_tables(tab.data(), ctx.data(), num_seqs, max_blocks_per_seq,
                                  max_context_len, num_blocks, block_size,
                                  group_starts != nullptr ? gs.data() : nullptr,
                                  prefix_lens != nullptr ? pl.data() : nullptr, num_groups);
  if (rc != ATTN_OK) g_last_error = std::string(fn) + " (ATTN_VALIDATE): " + g_last_error;
  return rc;
}

bool debug_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("ATTN_DEBUG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

}  // namespace

namespace attn {
// Status and message for the calling thread (used by block_manager.cpp too).
int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
}  // namespace attn

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
             int batch, int n_q, int n_k, int h_q, int h_kv, int head_dim,
             const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
             const int64_t* o_stride, float softmax_scale, int causal, void* stream) {
  try {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: dtype must be ATTN_F32, ATTN_F16 or ATTN_BF16");
    if (batch < 0 || n_q < 0 || n_k < 0 || h_q < 0 || h_kv < 0 || head_dim < 0)
      return fail(ATTN_ERR_SHAPE, "attn_fwd: sizes must be non-negative");
    if (h_kv == 0 || (h_q % h_kv) != 0)
      return fail(ATTN_ERR_SHAPE, "attn_fwd: h_q must be a positive multiple of h_kv");
    if (head_dim != 64 && head_dim != 128)
      return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: head_dim must be 64 or 128");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_SHAPE, "attn_fwd: causal must be 0 or 1");
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
      return fail(ATTN_ERR_SHAPE, "attn_fwd: softmax_scale must be finite and positive");
    if (batch == 0 || n_q == 0 || h_q == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr) return fail(ATTN_ERR_NULL, "attn_fwd: q and o must not be NULL");
    if (n_k > 0 && (k == nullptr || v == nullptr))
      return fail(ATTN_ERR_NULL, "attn_fwd: k and v must not be NULL");
    if (q_stride == nullptr || k_stride == nullptr || v_stride == nullptr || o_stride == nullptr)
      return fail(ATTN_ERR_NULL, "attn_fwd: stride arrays must not be NULL");
    const int es = elem_size(dtype);
    const void* ptrs[4] = {q, k, v, o};
    for (const void* ptr : ptrs)
      if (ptr != nullptr && !aligned16(ptr))
        return fail(ATTN_ERR_ALIGN, "attn_fwd: q, k, v and o must be 16-byte aligned");
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return fail(ATTN_ERR_ALIGN, "attn_fwd: lse must be 4-byte aligned");
    const int64_t* strides[4] = {q_stride, k_stride, v_stride, o_stride};
    for (const int64_t* st : strides)
      for (int i = 0; i < 3; ++i) {
        if (st[i] < 0) return fail(ATTN_ERR_SHAPE, "attn_fwd: strides must be non-negative");
        if ((st[i] * es) % 16 != 0)
          return fail(ATTN_ERR_ALIGN, "attn_fwd: batch/sequence/head strides must be multiples of 16 bytes");
      }

    if (n_k > 1 && (k_stride[1] < head_dim || v_stride[1] < head_dim))
      return fail(ATTN_ERR_SHAPE, "attn_fwd: k and v sequence strides must be >= head_dim");
    // K/V tiles are addressed with 32-bit byte offsets within one
    // (batch, kv head) slice, including up to one tile past its end
    if (((int64_t)n_k + 128) * std::max(k_stride[1], v_stride[1]) * es >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: one (batch, kv head) slice of k/v spans >= 2 GiB");
    if (((int64_t)n_q + 128) * q_stride[1] * es >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: one (batch, head) slice of q spans >= 2 GiB");

    attn::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.qs_b = q_stride[0]; p.qs_n = q_stride[1]; p.qs_h = q_stride[2];
    p.ks_b = k_stride[0]; p.ks_n = k_stride[1]; p.ks_h = k_stride[2];
    p.vs_b = v_stride[0]; p.vs_n = v_stride[1]; p.vs_h = v_stride[2];
    p.os_b = o_stride[0]; p.os_n = o_stride[1]; p.os_h = o_stride[2];
    p.batch = batch;
    p.n_q = n_q;
    p.n_k = n_k;
    p.h_q = h_q;
    p.h_kv = h_kv;
    p.group = h_q / h_kv;
    p.scale_log2 = softmax_scale * attn::kLog2e;
    if ((int64_t)((n_q + 63) / 64) * batch * h_q > (int64_t)1 << 31)
      return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: problem too large for one launch");
    if (debug_enabled())
      std::fprintf(stderr, "[attn] attn_fwd dtype=%d b=%d nq=%d nk=%d hq=%d hkv=%d d=%d causal=%d\n",
                   dtype, batch, n_q, n_k, h_q, h_kv, head_dim, causal);
    hipError_t e = attn::launch_prefill(dtype, head_dim, causal != 0, p,
                                        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, std::string("attn_fwd: launch failed: ") + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, "attn_fwd: unexpected host exception");
  }
}

int attn_fwd_paged(int dtype, const void* q, const int64_t* q_stride, const void* k_cache,
                   const void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                   void* o, const int64_t* o_stride, float* lse, int batch, int n_q, int h_q,
                   int h_kv, int head_dim, int block_size, int max_blocks_per_seq,
                   int max_context_len, int num_blocks, float softmax_scale, int causal,
                   void* stream) {
  const std::string f("attn_fwd_paged");
  try {
    g_last_error.clear();
    if (dtype != ATTN_F16 && dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": dtype must be ATTN_F16 or ATTN_BF16");
    if (batch < 0 || n_q < 0 || h_q < 0 || h_kv < 0 || head_dim < 0 || max_blocks_per_seq < 0 ||
        max_context_len < 0 || num_blocks < 0)
      return fail(ATTN_ERR_SHAPE, f + ": sizes must be non-negative");
    if (h_kv == 0 || (h_q % h_kv) != 0)
      return fail(ATTN_ERR_SHAPE, f + ": h_q must be a positive multiple of h_kv");
    if (head_dim != 64 && head_dim != 128)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
    if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, f + ": block_size must be 16");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_SHAPE, f + ": causal must be 0 or 1");
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
      return fail(ATTN_ERR_SHAPE, f + ": softmax_scale must be finite and positive");
    if ((int64_t)max_blocks_per_seq * block_size < (int64_t)max_context_len)
      return fail(ATTN_ERR_SHAPE, f + ": max_blocks_per_seq * block_size < max_context_len");
    if (max_context_len > 0 && num_blocks == 0)
      return fail(ATTN_ERR_SHAPE, f + ": num_blocks must be positive");
    if (batch == 0 || n_q == 0 || h_q == 0) return ATTN_OK;
    if (q == nullptr || o == nullptr || context_lens == nullptr || q_stride == nullptr ||
        o_stride == nullptr)
      return fail(ATTN_ERR_NULL, f + ": q, o, context_lens and strides must not be NULL");
    if (max_context_len > 0 && (k_cache == nullptr || v_cache == nullptr || block_table == nullptr))
      return fail(ATTN_ERR_NULL, f + ": caches and block_table must not be NULL");
    const void* ptrs[4] = {q, o, k_cache, v_cache};
    for (const void* ptr : ptrs)
      if (ptr != nullptr && !aligned16(ptr))
        return fail(ATTN_ERR_ALIGN, f + ": q, o and the caches must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
      return fail(ATTN_ERR_ALIGN, f + ": block_table, context_lens and lse must be 4-byte aligned");
    for (const int64_t* st : {q_stride, o_stride})
      for (int i = 0; i < 3; ++i)
        if (st[i] < 0 || (st[i] * 2) % 16 != 0)
          return fail(ATTN_ERR_ALIGN, f + ": strides must be non-negative multiples of 16 bytes");
    if (((int64_t)n_q + 128) * q_stride[1] * 2 >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, f + ": one (batch, head) slice of q spans >= 2 GiB");
    if ((int64_t)((n_q + 63) / 64) * batch * h_q > (int64_t)1 << 31)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": problem too large for one launch");
    if (validate_enabled()) {
      const int rc = validate_on_host("attn_fwd_paged", reinterpret_cast<hipStream_t>(stream),
                                      block_table, context_lens, batch, max_blocks_per_seq,
                                      max_context_len, num_blocks, block_size, nullptr, nullptr,
                                      0);
      if (rc != ATTN_OK) return rc;
    }
    attn::FwdParams p{};
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.o = o;
    p.lse = lse;
    p.qs_b = q_stride[0]; p.qs_n = q_stride[1]; p.qs_h = q_stride[2];
    p.os_b = o_stride[0]; p.os_n = o_stride[1]; p.os_h = o_stride[2];
    p.batch = batch;
    p.n_q = n_q;
    p.n_k = max_context_len;
    p.h_q = h_q;
    p.h_kv = h_kv;
    p.group = h_q / h_kv;
    p.block_table = block_table;
    p.context_lens = context_lens;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.scale_log2 = softmax_scale * attn::kLog2e;
    hipError_t e = attn::launch_prefill_paged(dtype, head_dim, causal != 0, p,
                                              reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, f + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, f + ": unexpected host exception");
  }
}

int paged_kv_write(int dtype, const void* k_new, const void* v_new, const int64_t* k_stride,
                   const int64_t* v_stride, const int32_t* slot_mapping, void* k_cache,
                   void* v_cache, int n_tokens, int h_kv, int head_dim, int block_size,
                   int num_blocks, void* stream) {
  const std::string f("paged_kv_write");
  try {
    g_last_error.clear();
    if (dtype != ATTN_F16 && dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": dtype must be ATTN_F16 or ATTN_BF16");
    if (n_tokens < 0 || h_kv <= 0 || num_blocks < 0)
      return fail(ATTN_ERR_SHAPE, f + ": n_tokens >= 0, h_kv > 0, num_blocks >= 0 required");
    if (head_dim != 64 && head_dim != 128)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
    if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, f + ": block_size must be 16");
    if (n_tokens == 0) return ATTN_OK;
    if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr || k_cache == nullptr ||
        v_cache == nullptr || k_stride == nullptr || v_stride == nullptr)
      return fail(ATTN_ERR_NULL, f + ": pointers must not be NULL");
    const void* ptrs[4] = {k_new, v_new, k_cache, v_cache};
    for (const void* ptr : ptrs)
      if (!aligned16(ptr)) return fail(ATTN_ERR_ALIGN, f + ": tensors must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(slot_mapping) & 3u)
      return fail(ATTN_ERR_ALIGN, f + ": slot_mapping must be 4-byte aligned");
    for (int i = 0; i < 2; ++i)
      if (k_stride[i] < 0 || v_stride[i] < 0 || (k_stride[i] * 2) % 16 || (v_stride[i] * 2) % 16)
        return fail(ATTN_ERR_ALIGN, f + ": token and head strides must be non-negative multiples of 16 bytes");
    if (n_tokens > 0x7fffffff / 2) return fail(ATTN_ERR_UNSUPPORTED, f + ": too many tokens");
    attn::KvWriteParams p{k_new, v_new, k_stride[0], k_stride[1], v_stride[0], v_stride[1],
                          slot_mapping, k_cache, v_cache, n_tokens, h_kv, head_dim, block_size,
                          (int64_t)num_blocks * block_size};
    hipError_t e = attn::launch_kv_write(p, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, f + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, f + ": unexpected host exception");
  }
}

int paged_kv_copy_blocks(int dtype, void* k_cache, void* v_cache, const int32_t* src,
                         const int32_t* dst, int n_pairs, int h_kv, int head_dim, int block_size,
                         int num_blocks, void* stream) {
  const std::string f("paged_kv_copy_blocks");
  try {
    g_last_error.clear();
    if (dtype != ATTN_F16 && dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": dtype must be ATTN_F16 or ATTN_BF16");
    if (n_pairs < 0 || h_kv <= 0 || num_blocks < 0)
      return fail(ATTN_ERR_SHAPE, f + ": n_pairs >= 0, h_kv > 0, num_blocks >= 0 required");
    if (head_dim != 64 && head_dim != 128)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
    if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, f + ": block_size must be 16");
    if (n_pairs == 0) return ATTN_OK;
    if (k_cache == nullptr || v_cache == nullptr || src == nullptr || dst == nullptr)
      return fail(ATTN_ERR_NULL, f + ": pointers must not be NULL");
    if (!aligned16(k_cache) || !aligned16(v_cache))
      return fail(ATTN_ERR_ALIGN, f + ": caches must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(src) & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u))
      return fail(ATTN_ERR_ALIGN, f + ": src and dst must be 4-byte aligned");
    attn::KvCopyParams p{k_cache, v_cache, src, dst, (int64_t)h_kv * block_size * head_dim,
                         num_blocks};
    hipError_t e = attn::launch_kv_copy(p, n_pairs, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, f + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, f + ": unexpected host exception");
  }
}

size_t attn_bwd_workspace_size(int batch, int n_q, int h_q) {
  if (batch <= 0 || n_q <= 0 || h_q <= 0) return 0;
  // delta, then the log-sum-exp in log2 units, one fp32 each per query row
  return 2 * align16((size_t)batch * h_q * n_q * 4);
}

int attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
             const void* d_o, const float* lse, void* dq, void* dk, void* dv, int batch, int n_q,
             int n_k, int h_q, int h_kv, int head_dim, const int64_t* q_stride,
             const int64_t* k_stride, const int64_t* v_stride, const int64_t* o_stride,
             const int64_t* do_stride, const int64_t* dq_stride, const int64_t* dk_stride,
             const int64_t* dv_stride, float softmax_scale, int causal, void* workspace,
             size_t workspace_bytes, void* stream) {
  const char* fn = "attn_bwd";
  try {
    g_last_error.clear();
    const std::string f(fn);
    if (dtype != ATTN_F16 && dtype != ATTN_BF16)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": dtype must be ATTN_F16 or ATTN_BF16");
    if (batch < 0 || n_q < 0 || n_k < 0 || h_q < 0 || h_kv < 0 || head_dim < 0)
      return fail(ATTN_ERR_SHAPE, f + ": sizes must be non-negative");
    if (h_kv == 0 || (h_q % h_kv) != 0)
      return fail(ATTN_ERR_SHAPE, f + ": h_q must be a positive multiple of h_kv");
    if (head_dim != 64 && head_dim != 128)
      return fail(ATTN_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_SHAPE, f + ": causal must be 0 or 1");
    if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
      return fail(ATTN_ERR_SHAPE, f + ": softmax_scale must be finite and positive");
    if (batch == 0 || h_q == 0 || (n_q == 0 && n_k == 0)) return ATTN_OK;
    const bool has_q = n_q > 0, has_k = n_k > 0;
    if (has_q && (q == nullptr || o == nullptr || d_o == nullptr || lse == nullptr || dq == nullptr))
      return fail(ATTN_ERR_NULL, f + ": q, o, d_o, lse and dq must not be NULL");
    if (has_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
      return fail(ATTN_ERR_NULL, f + ": k, v, dk and dv must not be NULL");
    if (q_stride == nullptr || k_stride == nullptr || v_stride == nullptr || o_stride == nullptr ||
        do_stride == nullptr || dq_stride == nullptr || dk_stride == nullptr ||
        dv_stride == nullptr)
      return fail(ATTN_ERR_NULL, f + ": stride arrays must not be NULL");
    const void* ptrs[9] = {q, k, v, o, d_o, dq, dk, dv, workspace};
    for (const void* ptr : ptrs)
      if (ptr != nullptr && !aligned16(ptr))
        return fail(ATTN_ERR_ALIGN, f + ": tensors and workspace must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return fail(ATTN_ERR_ALIGN, f + ": lse must be 4-byte aligned");
    const int64_t* strides[8] = {q_stride, k_stride, v_stride, o_stride,
                                 do_stride, dq_stride, dk_stride, dv_stride};
    for (const int64_t* st : strides)
      for (int i = 0; i < 3; ++i) {
        if (st[i] < 0) return fail(ATTN_ERR_SHAPE, f + ": strides must be non-negative");
        if ((st[i] * 2) % 16 != 0)
          return fail(ATTN_ERR_ALIGN, f + ": batch/sequence/head strides must be multiples of 16 bytes");
      }
    // Q, dO, K and V tiles are addressed with 32-bit byte offsets inside one
    // (batch, head) slice, including up to one tile past its end
    if (((int64_t)n_k + 128) * std::max(k_stride[1], v_stride[1]) * 2 >= ((int64_t)1 << 31) ||
        ((int64_t)n_q + 128) * std::max(q_stride[1], do_stride[1]) * 2 >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, f + ": one (batch, head) slice spans >= 2 GiB");
    if (h_q > 65535 || batch > 65535 ||
        (int64_t)((n_q + 127) / 128) * batch * h_q >= ((int64_t)1 << 31) ||
        (int64_t)((n_k + 127) / 128) * batch * h_kv >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, f + ": problem too large for one launch");
    const size_t need = attn_bwd_workspace_size(batch, n_q, h_q);
    int rc = check_workspace(fn, workspace, workspace_bytes, need);
    if (rc != ATTN_OK) return rc;

    attn::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = d_o; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.delta = static_cast<float*>(workspace);
    p.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      align16((size_t)batch * h_q * n_q * 4));
    p.qs_b = q_stride[0]; p.qs_n = q_stride[1]; p.qs_h = q_stride[2];
    p.ks_b = k_stride[0]; p.ks_n = k_stride[1]; p.ks_h = k_stride[2];
    p.vs_b = v_stride[0]; p.vs_n = v_stride[1]; p.vs_h = v_stride[2];
    p.os_b = o_stride[0]; p.os_n = o_stride[1]; p.os_h = o_stride[2];
    p.dos_b = do_stride[0]; p.dos_n = do_stride[1]; p.dos_h = do_stride[2];
    p.dqs_b = dq_stride[0]; p.dqs_n = dq_stride[1]; p.dqs_h = dq_stride[2];
    p.dks_b = dk_stride[0]; p.dks_n = dk_stride[1]; p.dks_h = dk_stride[2];
    p.dvs_b = dv_stride[0]; p.dvs_n = dv_stride[1]; p.dvs_h = dv_stride[2];
    p.batch = batch; p.n_q = n_q; p.n_k = n_k; p.h_q = h_q; p.h_kv = h_kv;
    p.group = h_q / h_kv;
    auto extent = [&](int n, int64_t pitch) -> uint32_t {
      return n > 0 ? (uint32_t)(((int64_t)(n - 1) * pitch + head_dim) * 2) : 0u;
    };
    p.q_bytes = extent(n_q, q_stride[1]);
    p.do_bytes = extent(n_q, do_stride[1]);
    p.k_bytes = extent(n_k, k_stride[1]);
    p.v_bytes = extent(n_k, v_stride[1]);
    p.scale = softmax_scale;
    p.scale_log2 = softmax_scale * attn::kLog2e;
    if (debug_enabled())
      std::fprintf(stderr, "[attn] %s dtype=%d b=%d nq=%d nk=%d hq=%d hkv=%d d=%d causal=%d\n", fn,
                   dtype, batch, n_q, n_k, h_q, h_kv, head_dim, causal);
    hipError_t e = attn::launch_backward(dtype, head_dim, causal != 0, p,
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, f + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, std::string(fn) + ": unexpected host exception");
  }
}

size_t paged_attn_decode_workspace_size(int num_seqs, int h_q, int h_kv, int head_dim,
                                        int max_context_len) {
  return attn::decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, max_context_len);
}

}  // extern "C"

namespace {

// paged_attn_decode and its variant on the library's scratch.  With
// workspace == nullptr and use_scratch set, the workspace is the scratch
// array of the stream's device (sizes beyond it are rejected first).
int decode_call(const char* fn, int dtype, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                void* o, float* lse, int num_seqs, int h_q, int h_kv, int head_dim,
                int block_size, int max_blocks_per_seq, int max_context_len, int num_blocks,
                float softmax_scale, void* workspace, size_t workspace_bytes, bool use_scratch,
                void* stream) {
  try {
    g_last_error.clear();
    attn::DecodeParams p;
    int rc = check_decode(fn, dtype, q, k_cache, v_cache, block_table, context_lens, o, lse,
                          num_seqs, h_q, h_kv, head_dim, block_size, max_blocks_per_seq,
                          max_context_len, num_blocks, softmax_scale, p);
    if (rc != ATTN_OK || num_seqs == 0) return rc;
    const size_t need = attn::decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, max_context_len);
    if (use_scratch) {
      const size_t cap = attn::scratch_capacity();
      if (need > cap)
        return fail(ATTN_ERR_WORKSPACE, std::string(fn) + ": these sizes need " +
                                            std::to_string(need) + " bytes of scratch; the "
                                            "library holds " + std::to_string(cap));
      if (need > 0) {
        int dev = -1;
        hipError_t e = stream != nullptr
                           ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev)
                           : hipGetDevice(&dev);
        if (e == hipSuccess) e = attn::scratch_address(dev, &workspace);
        if (e != hipSuccess)
          return fail(ATTN_ERR_HIP, std::string(fn) + ": scratch lookup failed: " +
                                        hipGetErrorString(e));
        workspace_bytes = cap;
      }
    }
    rc = check_workspace(fn, workspace, workspace_bytes, need);
    if (rc != ATTN_OK) return rc;
    if (need > 0) {
      const int64_t slots =
          (int64_t)attn::decode_waves(num_seqs, h_kv, max_context_len) * 2 * (h_q / h_kv);
      p.ws_o = static_cast<float*>(workspace);
      p.ws_ml = p.ws_o + slots * head_dim;
      p.ws_unit = reinterpret_cast<int32_t*>(p.ws_ml + slots * 2);
    }
    if (!use_scratch && validate_enabled()) {
      rc = validate_on_host(fn, reinterpret_cast<hipStream_t>(stream),
                            block_table, context_lens, num_seqs, max_blocks_per_seq,
                            max_context_len, num_blocks, block_size, nullptr, nullptr, 0);
      if (rc != ATTN_OK) return rc;
    }
    if (debug_enabled())
      std::fprintf(stderr, "[attn] %s dtype=%d seqs=%d hq=%d hkv=%d d=%d waves=%d\n", fn,
                   dtype, num_seqs, h_q, h_kv, head_dim,
                   attn::decode_waves(num_seqs, h_kv, max_context_len));
    hipError_t e = attn::launch_decode(dtype, p, max_context_len, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, std::string(fn) + ": unexpected host exception");
  }
}

}  // namespace

extern "C" {

int paged_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* context_lens, void* o,
                      float* lse, int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                      int max_blocks_per_seq, int max_context_len, int num_blocks,
                      float softmax_scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_call("paged_attn_decode", dtype, q, k_cache, v_cache, block_table, context_lens,
                     o, lse, num_seqs, h_q, h_kv, head_dim, block_size, max_blocks_per_seq,
                     max_context_len, num_blocks, softmax_scale, workspace, workspace_bytes,
                     false, stream);
}

int paged_attn_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens, void* o,
                              float* lse, int num_seqs, int h_q, int h_kv, int head_dim,
                              int block_size, int max_blocks_per_seq, int max_context_len,
                              int num_blocks, float softmax_scale, void* stream) {
  return decode_call("paged_attn_decode_noalloc", dtype, q, k_cache, v_cache, block_table,
                     context_lens, o, lse, num_seqs, h_q, h_kv, head_dim, block_size,
                     max_blocks_per_seq, max_context_len, num_blocks, softmax_scale, nullptr, 0,
                     true, stream);
}

size_t paged_attn_decode_shared_workspace_size(int num_seqs, int num_groups, int max_group_size,
                                               int h_q, int h_kv, int head_dim,
                                               int max_context_len, int max_prefix_len) {
  if (num_seqs <= 0 || num_groups <= 0 || max_group_size <= 0 || h_q <= 0 || h_kv <= 0 ||
      head_dim <= 0 || max_context_len < 0 || max_prefix_len < 0 || h_q % h_kv != 0)
    return 0;
  const attn::SharedPlan pl =
      attn::shared_plan(num_groups, max_group_size, h_q, h_kv, max_prefix_len);
  const size_t split = attn::decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, max_context_len);
  return shared_ws(num_seqs, h_q, head_dim, split, pl.items).total;
}

int paged_attn_decode_shared(int dtype, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* context_lens,
                             const int32_t* group_starts, const int32_t* prefix_lens, void* o,
                             float* lse, int num_seqs, int num_groups, int max_group_size,
                             int h_q, int h_kv, int head_dim, int block_size,
                             int max_blocks_per_seq, int max_context_len, int max_prefix_len,
                             int num_blocks, float softmax_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const char* fn = "paged_attn_decode_shared";
  try {
    g_last_error.clear();
    attn::DecodeParams p;
    int rc = check_decode(fn, dtype, q, k_cache, v_cache, block_table, context_lens, o, lse,
                          num_seqs, h_q, h_kv, head_dim, block_size, max_blocks_per_seq,
                          max_context_len, num_blocks, softmax_scale, p);
    if (rc != ATTN_OK) return rc;
    if (num_groups < 0 || max_group_size < 0 || max_prefix_len < 0)
      return fail(ATTN_ERR_SHAPE, std::string(fn) + ": sizes must be non-negative");
    if (num_seqs == 0) return ATTN_OK;
    if (num_groups == 0 || max_group_size == 0)
      return fail(ATTN_ERR_SHAPE, std::string(fn) + ": every sequence must be in a group");
    if (max_prefix_len > max_context_len)
      return fail(ATTN_ERR_SHAPE, std::string(fn) + ": max_prefix_len > max_context_len");
    if (group_starts == nullptr || prefix_lens == nullptr)
      return fail(ATTN_ERR_NULL, std::string(fn) + ": group_starts and prefix_lens must not be NULL");
    if ((reinterpret_cast<uintptr_t>(group_starts) & 3u) || (reinterpret_cast<uintptr_t>(prefix_lens) & 3u))
      return fail(ATTN_ERR_ALIGN, std::string(fn) + ": group_starts and prefix_lens must be 4-byte aligned");
    const attn::SharedPlan pl =
        attn::shared_plan(num_groups, max_group_size, h_q, h_kv, max_prefix_len);
    if (pl.items >= ((int64_t)1 << 31))
      return fail(ATTN_ERR_UNSUPPORTED, std::string(fn) + ": problem too large for one launch");
    const size_t split = attn::decode_workspace_bytes(num_seqs, h_q, h_kv, head_dim, max_context_len);
    const SharedWs lay = shared_ws(num_seqs, h_q, head_dim, split, pl.items);
    rc = check_workspace(fn, workspace, workspace_bytes, lay.total);
    if (rc != ATTN_OK) return rc;
    if (validate_enabled()) {
      rc = validate_on_host(fn, reinterpret_cast<hipStream_t>(stream), block_table, context_lens,
                            num_seqs, max_blocks_per_seq, max_context_len, num_blocks,
                            block_size, group_starts, prefix_lens, num_groups);
      if (rc != ATTN_OK) return rc;
    }
    char* base = static_cast<char*>(workspace);
    if (split > 0) {
      const int64_t slots =
          (int64_t)attn::decode_waves(num_seqs, h_kv, max_context_len) * 2 * (h_q / h_kv);
      p.ws_o = reinterpret_cast<float*>(base);
      p.ws_ml = p.ws_o + slots * head_dim;
      p.ws_unit = reinterpret_cast<int32_t*>(p.ws_ml + slots * 2);
    }
    p.group_starts = group_starts;
    p.prefix_lens = prefix_lens;
    p.ws_suf_o = reinterpret_cast<float*>(base + lay.suf_o);
    p.ws_suf_ml = reinterpret_cast<float*>(base + lay.suf_ml);
    p.ws_pre_o = reinterpret_cast<float*>(base + lay.pre_o);
    p.ws_pre_ml = reinterpret_cast<float*>(base + lay.pre_ml);
    p.seq_meta = reinterpret_cast<int32_t*>(base + lay.meta);
    p.first_block = p.seq_meta;
    p.seq_group = p.seq_meta + num_seqs;
    p.seq_member = p.seq_meta + 2 * num_seqs;
    p.num_groups = num_groups;
    p.n_rt = pl.n_rt;
    p.n_ch = pl.n_ch;
    p.chunk_blocks = pl.chunk_blocks;
    if (debug_enabled())
      std::fprintf(stderr,
                   "[attn] %s dtype=%d seqs=%d groups=%d hq=%d hkv=%d d=%d items=%lld "
                   "chunk=%d tiles=%d\n",
                   fn, dtype, num_seqs, num_groups, h_q, h_kv, head_dim, (long long)pl.items,
                   pl.chunk_blocks, pl.n_rt);
    hipError_t e = attn::launch_decode_shared(dtype, p, pl.items, max_context_len,
                                              reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
    return ATTN_OK;
  } catch (...) {
    return fail(ATTN_ERR_HIP, std::string(fn) + ": unexpected host exception");
  }
}

}  // extern "C"
