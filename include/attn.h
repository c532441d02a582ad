/*
 * attn.h -- C ABI of libattn.so: exact fused attention (prefill) and paged
 * single-token decode for AMD MI355X (gfx950).
 *
 * What is computed.  Both entry points compute exact scaled-dot-product
 * attention, O = softmax(Q K^T * scale) V, the definition given on the page
 * "Other people's interview notes" (zzsy.me), question "explain
 * FlashAttention", part 1.  It is evaluated in one fused, tiled pass with the
 * online-softmax update of part 2 of the same answer (running row maximum m
 * and running sum l, accumulated output rescaled by exp(m_old - m_new)), so
 * the N x N score and probability matrices are never written to device
 * memory (the codelogiq.de FAQ on FlashAttention-2 vs standard attention).
 * Decode reads a PagedAttention-style KV cache through a block table, as the
 * tutorial "Chapter 3 Advanced principles: performance model and numerical
 * stability", section 3.0, describes (fixed-size KV blocks, a per-sequence
 * table of block ids, shared prefixes expressed as repeated ids).
 *
 * Conventions the pages leave open, fixed here:
 *   - grouped-query attention: query head h reads KV head h / (h_q / h_kv);
 *   - the causal mask is bottom-right aligned: key j is visible to query row
 *     i when j <= i + (n_k - n_q) (the usual lower triangle when n_q == n_k);
 *   - a row with no visible key gets output 0 and log-sum-exp -inf;
 *   - the log-sum-exp is in natural-log units;
 *   - 16-bit outputs are rounded to nearest-even from fp32.
 *
 * Arithmetic.  16-bit inputs: products on the matrix cores with fp32
 * accumulation; softmax statistics and the output accumulator in fp32; the
 * probabilities are rounded to the input type before the P*V product.  fp32
 * inputs: fp32 throughout.
 *
 * Ownership.  Every pointer is device memory owned by the caller.  The
 * library never allocates or frees device memory and keeps no pointer after a
 * call returns.  Its mutable global state is a thread-local error message and,
 * for paged_attn_decode_noalloc only, one scratch array per GPU (a static
 * device array of the code object, ATTN_DECODE_SCRATCH_BYTES) with its looked-up
 * address.  Calls other than paged_attn_decode_noalloc are re-entrant.
 *
 * Asynchrony.  Calls only enqueue kernels on the given stream (a hipStream_t
 * passed as void*; NULL means the null stream) and never synchronise.  A
 * device-side fault caused by invalid device data (an out-of-range block id,
 * a context length above the stated maximum) surfaces at the caller's next
 * synchronisation and is undefined behaviour.  Test mode: with the
 * environment variable ATTN_VALIDATE set to a value other than "0", the
 * paged entry points (paged_attn_decode, paged_attn_decode_shared,
 * attn_fwd_paged) first copy their block table, context lengths and groups
 * to the host, waiting for the copy on the given stream, and check them with
 * attn_validate_paged_tables; a violation returns ATTN_ERR_SHAPE and launches
 * nothing.  The variable is read at every call.
 *
 * Errors.  Every entry point returns ATTN_OK or one of the codes below and
 * never aborts; no C++ exception crosses the ABI.  Arguments are validated on
 * the host before anything is launched; on an error nothing is launched and
 * attn_last_error() describes the first problem found.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 7

/* element types of q, k, v, o and the KV cache */
typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype;

/* status codes */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size is negative / inconsistent (h_q % h_kv != 0, ...) */
  ATTN_ERR_UNSUPPORTED = 3, /* a valid but unsupported dtype / head_dim / block size / group */
  ATTN_ERR_WORKSPACE = 4,   /* decode workspace missing or smaller than required */
  ATTN_ERR_ALIGN = 5,       /* a base pointer or row stride is not 16-byte aligned */
  ATTN_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  ATTN_ERR_NO_BLOCKS = 7    /* the block manager has too few free blocks (nothing changed) */
};

/* ABI version of the loaded library (ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* Message for the last non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* attn_last_error(void);

/*
 * attn_validate_paged_tables -- range-check the metadata of a paged call on
 * the host (every array is HOST memory; nothing touches the GPU).  The
 * kernels trust these values; this is the check the ATTN_VALIDATE mode runs.
 * The contract checked is the paged KV cache of the tutorial "Chapter 3
 * Advanced principles: performance model and numerical stability", section
 * 3.0: logical block t / block_size of a sequence lives in the physical block
 * its table row names, and sequences sharing a prefix name the same blocks.
 *
 *   block_table     [num_seqs][max_blocks_per_seq] int32; the first
 *                   ceil(context_lens[s] / block_size) entries of row s must
 *                   lie in [0, num_blocks) (the rest are not read).
 *   context_lens    [num_seqs] int32, each in [0, max_context_len] and
 *                   needing at most max_blocks_per_seq table entries.
 *   group_starts,   NULL (no groups) or, for paged_attn_decode_shared,
 *   prefix_lens     [num_groups + 1] and [num_groups] int32 with
 *                   group_starts[0] == 0, non-decreasing, group_starts[
 *                   num_groups] == num_seqs; prefix_lens[g] >= 0 and at most
 *                   every member's context; the first prefix_lens[g] /
 *                   block_size entries of every member's row equal the
 *                   group's first member's.
 *
 * Returns ATTN_OK, ATTN_ERR_NULL (a required array is NULL) or
 * ATTN_ERR_SHAPE; attn_last_error() names the first violation found (array,
 * index, value).
 */
int attn_validate_paged_tables(const int32_t* block_table, const int32_t* context_lens,
                               int num_seqs, int max_blocks_per_seq, int max_context_len,
                               int num_blocks, int block_size, const int32_t* group_starts,
                               const int32_t* prefix_lens, int num_groups);

/*
 * attn_fwd -- prefill: O = softmax(Q K^T * softmax_scale [+ causal mask]) V.
 *
 *   dtype          ATTN_F32, ATTN_F16 or ATTN_BF16 (q, k, v and o share it).
 *   q              [batch][n_q][h_q][head_dim] addressed by q_stride.
 *   k, v           [batch][n_k][h_kv][head_dim] addressed by k_stride / v_stride.
 *   o              [batch][n_q][h_q][head_dim] addressed by o_stride (written).
 *   lse            optional [batch][h_q][n_q] fp32, contiguous, natural-log
 *                  log-sum-exp of each row's visible logits (written); NULL
 *                  to skip.
 *   x_stride[3]    element strides of the (batch, sequence, head) dimensions;
 *                  the head_dim stride is 1.  Host arrays.
 *   head_dim       64 or 128.
 *   h_q, h_kv      h_q % h_kv == 0.
 *   softmax_scale  finite and > 0 (1/sqrt(head_dim) in the usual case).
 *   causal         0 or 1 (bottom-right aligned mask, see above).
 *   stream         hipStream_t or NULL.
 *
 * Alignment: base pointers 16-byte aligned; every sequence and head stride
 * (and batch stride) times the element size a multiple of 16 bytes.  The
 * sequence strides of k and v must be at least head_dim (rows do not
 * overlap), and one (batch, kv head) slice of k or v must span less than
 * 2 GiB.
 * batch, n_q or h_q equal to 0 is a no-op; n_k == 0 writes o = 0 and
 * lse = -inf.  Host-side errors only: ATTN_ERR_NULL, _SHAPE, _UNSUPPORTED,
 * _ALIGN; ATTN_ERR_HIP if the launch fails.
 */
int attn_fwd(int dtype,
             const void* q, const void* k, const void* v, void* o, float* lse,
             int batch, int n_q, int n_k, int h_q, int h_kv, int head_dim,
             const int64_t* q_stride, const int64_t* k_stride,
             const int64_t* v_stride, const int64_t* o_stride,
             float softmax_scale, int causal, void* stream);

/*
 * Bytes of device workspace attn_bwd needs (two fp32 per query row and head:
 * rowsum(dO * O) and the log-sum-exp in log2 units).  Returns 0 for empty or
 * invalid sizes.
 */
size_t attn_bwd_workspace_size(int batch, int n_q, int h_q);

/*
 * attn_bwd -- gradients of attn_fwd's output with respect to q, k and v, for
 * an upstream gradient d_o of the output: the backward pass with
 * recomputation of "Other people's interview notes", question "explain
 * FlashAttention", part 3 (no N x N matrix is stored by the forward pass or
 * written by this one; the probabilities are recomputed tile by tile from q,
 * k and the forward log-sum-exp).  The gradients are those of the definition
 * O = softmax(Q K^T * softmax_scale [+ causal mask]) V:
 *     dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *     dQ = softmax_scale dS K,  dK = softmax_scale dS^T Q,
 * with a KV head's dK and dV summed over the query heads that read it.
 *
 *   dtype          ATTN_F16 or ATTN_BF16 (every tensor argument shares it).
 *   q, o, d_o      [batch][n_q][h_q][head_dim]: the forward inputs, the
 *                  forward output O (as attn_fwd returned it) and dO.
 *   k, v           [batch][n_k][h_kv][head_dim].
 *   lse            [batch][h_q][n_q] fp32, contiguous: the log-sum-exp attn_fwd
 *                  returned for these inputs (natural log; -inf for rows with
 *                  no visible key).
 *   dq             like q; dk, dv like k (written; every element, zeros where
 *                  there is nothing to sum).
 *   x_stride[3]    element strides of (batch, sequence, head) of each tensor,
 *                  host arrays, head_dim stride 1 (same rules as attn_fwd).
 *   head_dim, h_q, h_kv, softmax_scale, causal, stream: as attn_fwd.
 *   workspace      device memory of at least attn_bwd_workspace_size(batch,
 *                  n_q, h_q) bytes, 16-byte aligned; contents on entry do not
 *                  matter.
 *
 * Three kernels are enqueued: rowsum(dO * O) per query row, dK and dV (a
 * workgroup per 128 keys walks the query tiles of every head of the GQA
 * group), and dQ (a workgroup per 128 query rows walks the key tiles).  None
 * uses atomics, so the results are deterministic.  batch, h_q or both n_q
 * and n_k equal to 0 is a no-op.  Host-side errors only: ATTN_ERR_NULL,
 * _SHAPE, _UNSUPPORTED, _ALIGN, _WORKSPACE; ATTN_ERR_HIP if a launch fails.
 */
int attn_bwd(int dtype,
             const void* q, const void* k, const void* v, const void* o, const void* d_o,
             const float* lse, void* dq, void* dk, void* dv,
             int batch, int n_q, int n_k, int h_q, int h_kv, int head_dim,
             const int64_t* q_stride, const int64_t* k_stride, const int64_t* v_stride,
             const int64_t* o_stride, const int64_t* do_stride, const int64_t* dq_stride,
             const int64_t* dk_stride, const int64_t* dv_stride,
             float softmax_scale, int causal,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace paged_attn_decode needs for these sizes (the
 * split-K partial results).  Returns 0 for invalid sizes.
 */
size_t paged_attn_decode_workspace_size(int num_seqs, int h_q, int h_kv, int head_dim,
                                        int max_context_len);

/*
 * paged_attn_decode -- one query token per sequence attending to its whole
 * cached context through a block table.
 *
 *   dtype               ATTN_F16 or ATTN_BF16.
 *   q                   [num_seqs][h_q][head_dim], contiguous.
 *   k_cache, v_cache    [num_blocks][h_kv][block_size][head_dim] each,
 *                       contiguous.  Logical token t of sequence s lives at
 *                       block block_table[s][t / block_size], slot
 *                       t % block_size.  The same block id may appear in
 *                       several rows (shared prefixes); blocks are only read.
 *   block_table         device [num_seqs][max_blocks_per_seq] int32; only the
 *                       first ceil(context_lens[s] / block_size) entries of a
 *                       row are read, and each must be in [0, num_blocks).
 *   context_lens        device [num_seqs] int32, each in [0, max_context_len];
 *                       the query attends to all context_lens[s] tokens (the
 *                       length includes the current token).  0 gives o = 0
 *                       and lse = -inf.
 *   o                   [num_seqs][h_q][head_dim], contiguous (written).
 *   lse                 optional [num_seqs][h_q] fp32 (written); NULL to skip.
 *   head_dim            64 or 128.   block_size: 16.
 *   h_q / h_kv          a group of at most 16 query heads per KV head.
 *   max_context_len     upper bound of context_lens, host-side; fixes the
 *                       grid and the workspace size.
 *   max_blocks_per_seq  >= ceil(max_context_len / block_size).
 *   workspace           device memory of at least
 *                       paged_attn_decode_workspace_size(num_seqs, h_q, h_kv,
 *                       head_dim, max_context_len) bytes, 16-byte aligned,
 *                       owned by the caller; its contents on entry do not
 *                       matter and are garbage on exit.
 *   stream              hipStream_t or NULL.
 *
 * Two kernels are enqueued.  The split kernel cuts the list of all
 * (sequence, KV head, block) triples into equal ranges, one per persistent
 * wave; a (sequence, KV head) pair finished inside one range is written
 * there, a pair cut by range boundaries leaves partial results in the
 * workspace, and the combine kernel merges those by their log-sum-exp (and
 * writes the empty-context outputs).  Results do not depend on which
 * physical blocks hold the data: the same logical sequences give bit-identical
 * outputs under any block table.  num_seqs == 0 is a no-op.
 * K and V are read with the non-temporal cache hint (each byte once, streamed
 * past the caches): a block that several rows of the table share is fetched
 * from memory again for each.  Batches whose sequences share prefix blocks
 * are served better by paged_attn_decode_shared, which reads them once.
 */
int paged_attn_decode(int dtype,
                      const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* context_lens,
                      void* o, float* lse,
                      int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                      int max_blocks_per_seq, int max_context_len, int num_blocks,
                      float softmax_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, meaning and results as
 * paged_attn_decode (the same kernels, bit for bit), without the workspace:
 * the split-K partials go to a scratch array of ATTN_DECODE_SCRATCH_BYTES
 * that the library holds in device memory, one per GPU, from the library's
 * first use on that GPU until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's scratch address once.
 *
 * Limits and sharing.  Sizes whose paged_attn_decode_workspace_size exceeds
 * ATTN_DECODE_SCRATCH_BYTES are rejected with ATTN_ERR_WORKSPACE before
 * anything is launched.  Every call on one GPU uses that GPU's one scratch
 * array: calls that may overlap on the same GPU (different streams, or
 * threads without ordering) race and give undefined results.  Calls ordered
 * on one stream are safe; the scratch needs no clearing between them (its
 * contents on entry do not matter, as for the workspace).  The ATTN_VALIDATE
 * mode is not applied here (it copies to pageable host memory).
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)40 << 20)
int paged_attn_decode_noalloc(int dtype,
                              const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens,
                              void* o, float* lse,
                              int num_seqs, int h_q, int h_kv, int head_dim, int block_size,
                              int max_blocks_per_seq, int max_context_len, int num_blocks,
                              float softmax_scale, void* stream);

/*
 * Bytes of device workspace paged_attn_decode_shared needs for these sizes
 * (the partials of both parts and a little per-sequence metadata).  Returns 0
 * for invalid sizes.
 */
size_t paged_attn_decode_shared_workspace_size(int num_seqs, int num_groups, int max_group_size,
                                               int h_q, int h_kv, int head_dim,
                                               int max_context_len, int max_prefix_len);

/*
 * paged_attn_decode_shared -- paged_attn_decode for sequences that share a
 * prefix: the parallel-sampling and beam-search case of the tutorial
 * "Chapter 3 Advanced principles: performance model and numerical
 * stability" (section 3.0), where several sequences hold the same leading
 * block ids.  It computes what paged_attn_decode computes, for the same
 * arguments, but reads each shared prefix block once per group instead of
 * once per sequence.
 *
 * Arguments as for paged_attn_decode, plus:
 *   group_starts        device [num_groups + 1] int32, non-decreasing, with
 *                       group_starts[0] == 0 and group_starts[num_groups] ==
 *                       num_seqs: group g is sequences group_starts[g] ..
 *                       group_starts[g + 1] - 1 (a group may be empty; an
 *                       unshared sequence is a group of one with prefix 0).
 *   prefix_lens         device [num_groups] int32, tokens of the group's
 *                       common prefix, 0 <= prefix_lens[g] <= max_prefix_len
 *                       and <= the context length of every member.  The
 *                       first prefix_lens[g] / block_size table entries of
 *                       every member of group g must equal those of the
 *                       group's first member (the same physical blocks:
 *                       that is what "shared" means); the prefix kernel reads
 *                       them from the first member's row.  Only the prefix's
 *                       whole blocks are read once per group; a partial last
 *                       block is read per sequence like the rest.
 *   num_groups          >= 1 (when num_seqs > 0).
 *   max_group_size      host-side bound of the group sizes and
 *   max_prefix_len      of prefix_lens (at most max_context_len), which size
 *                       the prefix work and the workspace.  Members and
 *                       prefix blocks past these bounds are left to the
 *                       per-sequence pass: a bound below the actual value
 *                       costs speed, not correctness.
 *   workspace           at least paged_attn_decode_shared_workspace_size(
 *                       num_seqs, num_groups, max_group_size, h_q, h_kv,
 *                       head_dim, max_context_len, max_prefix_len) bytes,
 *                       16-byte aligned; contents on entry do not matter.
 *
 * Three kernels are enqueued.  The prefix kernel gives each group's queries
 * that read one KV head (members x query heads, in tiles of 32) one pass
 * over the group's prefix blocks, in chunks, on the matrix cores, and leaves
 * one partial result per chunk and query.  The split kernel of
 * paged_attn_decode then runs over each sequence's remaining blocks, and the
 * combine kernel merges all partials of a (sequence, query head) by their
 * log-sum-exp.  The result equals paged_attn_decode's up to the order of
 * floating-point accumulation, and does not depend on which physical blocks
 * hold the data.  If the sharing contract is broken (different ids in a
 * member's prefix) the member's output uses the first member's prefix
 * blocks.  Host-side errors as for paged_attn_decode.
 */
int paged_attn_decode_shared(int dtype,
                             const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* context_lens,
                             const int32_t* group_starts, const int32_t* prefix_lens,
                             void* o, float* lse,
                             int num_seqs, int num_groups, int max_group_size,
                             int h_q, int h_kv, int head_dim, int block_size,
                             int max_blocks_per_seq, int max_context_len, int max_prefix_len,
                             int num_blocks, float softmax_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged KV cache maintenance.  The cache layout is paged_attn_decode's:
 * k_cache and v_cache are [num_blocks][h_kv][block_size][head_dim] (block_size
 * 16, head_dim 64 or 128, bf16 or fp16), and logical token t of a sequence
 * lives at slot block_table[t / block_size] * block_size + t % block_size (the
 * tutorial "Chapter 3 Advanced principles: performance model and numerical
 * stability", section 3.0: fixed-size blocks, per-sequence block tables,
 * blocks shared by forked sequences and copied before a shared block is
 * written).
 */

/*
 * attn_fwd_paged -- prefill over a paged KV cache (chunked prefill): the n_q
 * query rows of sequence b are the last n_q tokens of its context, whose
 * K and V (already written, e.g. by paged_kv_write) are read through its
 * block table.  Query row i sees keys j <= i + (context_lens[b] - n_q) when
 * causal, all context_lens[b] keys otherwise; rows that see no key get o = 0
 * and lse = -inf.  The result is attn_fwd's on the sequence's logical K/V.
 *
 *   q, o           [batch][n_q][h_q][head_dim] addressed by q_stride /
 *                  o_stride (host arrays of 3, as attn_fwd).
 *   k_cache, v_cache, block_table, block_size, num_blocks: as
 *                  paged_attn_decode; context_lens device [batch], each in
 *                  [0, max_context_len].
 *   lse            optional [batch][h_q][n_q] fp32 (written).
 *   dtype ATTN_F16 or ATTN_BF16; head_dim 64 or 128; the same kernel as
 *   attn_fwd with K/V tile rows taken block by block.  Asynchronous.
 */
int attn_fwd_paged(int dtype, const void* q, const int64_t* q_stride,
                   const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* context_lens,
                   void* o, const int64_t* o_stride, float* lse,
                   int batch, int n_q, int h_q, int h_kv, int head_dim, int block_size,
                   int max_blocks_per_seq, int max_context_len, int num_blocks,
                   float softmax_scale, int causal, void* stream);

/*
 * paged_kv_write -- write the K and V rows of n_tokens new tokens into their
 * slots: for token i, k_cache[slot / block_size][h][slot % block_size][:] =
 * k_new[i][h][:] for every KV head h, and the same for V.
 *
 *   k_new, v_new    device, token i head h at x_new + i * x_stride[0] +
 *                   h * x_stride[1] (elements; head_dim contiguous), so a
 *                   [batch][seq][h_kv][d] prefill tensor can be passed as a
 *                   view.  x_stride: host arrays of 2.
 *   slot_mapping    device [n_tokens] int32; a slot outside [0, num_blocks *
 *                   block_size) (for instance -1 for padding) is skipped.
 *   Two tokens must not name the same slot (the order of their writes is
 *   not defined).  Asynchronous; host-side errors as for paged_attn_decode.
 */
int paged_kv_write(int dtype, const void* k_new, const void* v_new,
                   const int64_t* k_stride, const int64_t* v_stride,
                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                   int n_tokens, int h_kv, int head_dim, int block_size, int num_blocks,
                   void* stream);

/*
 * paged_kv_copy_blocks -- copy whole blocks (every KV head of K and of V):
 * block dst[i] becomes a copy of block src[i].  src, dst: device [n_pairs]
 * int32; pairs naming a block outside [0, num_blocks) are skipped.  The
 * destinations must be distinct and must not be sources of other pairs (the
 * block manager's copy-on-write copies satisfy this).  Asynchronous.
 */
int paged_kv_copy_blocks(int dtype, void* k_cache, void* v_cache,
                         const int32_t* src, const int32_t* dst, int n_pairs,
                         int h_kv, int head_dim, int block_size, int num_blocks, void* stream);

/*
 * Block manager (host only; no device memory, no GPU calls).  It does the
 * bookkeeping of a paged KV cache of num_blocks blocks: it hands out slots
 * for new tokens, counts references per block, and, when a sequence appends
 * to a partially filled last block that another sequence also holds, moves
 * the sequence to a fresh block and reports the copy (source, destination)
 * that the caller must run (paged_kv_copy_blocks) before writing the new
 * tokens (paged_kv_write).  Full blocks stay shared.  A forked sequence
 * shares all of its parent's blocks.  Free blocks are reused last-freed first,
 * so the same sequence of calls gives the same block ids.  A handle is not
 * thread-safe: one thread at a time per handle.  Errors: ATTN_ERR_NULL,
 * ATTN_ERR_SHAPE (bad size, unknown or duplicate sequence id),
 * ATTN_ERR_NO_BLOCKS (not enough free blocks; the call changes nothing).
 */
typedef struct attn_block_manager attn_block_manager;

/* A manager of num_blocks blocks of block_size tokens, all free, into *out. */
int attn_bm_create(int num_blocks, int block_size, attn_block_manager** out);
void attn_bm_destroy(attn_block_manager* m);
/* Free blocks; -1 for a NULL manager. */
int attn_bm_num_free(const attn_block_manager* m);
/* References to block (sequences holding it); -1 if out of range. */
int attn_bm_ref_count(const attn_block_manager* m, int block);
/* Tokens of a sequence; -1 if unknown. */
int64_t attn_bm_length(const attn_block_manager* m, int64_t seq_id);
/* A new, empty sequence. */
int attn_bm_add_sequence(attn_block_manager* m, int64_t seq_id);
/* A new sequence child holding parent's tokens and sharing its blocks. */
int attn_bm_fork(attn_block_manager* m, int64_t parent, int64_t child);
/*
 * Append n_tokens tokens to seq_id: slots[i] (host, n_tokens) receives the
 * slot of the i-th new token; copy_src[0] / copy_dst[0] (host, room for one
 * pair) and *n_copies (0 or 1) receive the copy-on-write copy to run first.
 */
int attn_bm_append(attn_block_manager* m, int64_t seq_id, int n_tokens, int32_t* slots,
                   int32_t* copy_src, int32_t* copy_dst, int* n_copies);
/* Release a sequence; blocks no longer held by any sequence become free. */
int attn_bm_free_sequence(attn_block_manager* m, int64_t seq_id);
/*
 * Block table rows (host [n][max_blocks] int32, -1 padded) and context
 * lengths (host [n]) of n sequences, in paged_attn_decode's format.
 */
int attn_bm_block_table(const attn_block_manager* m, const int64_t* seq_ids, int n,
                        int max_blocks, int32_t* table, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
