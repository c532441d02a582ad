// Host-side range check of the device metadata a paged call reads: block
// table entries, context lengths and the shared-prefix groups.  The kernels
// trust these values (reading them costs no launch-time work), so an
// out-of-range block id or a context longer than the table is undefined
// behaviour on the device.  This check runs on host copies: directly through
// attn_validate_paged_tables, or inside paged_attn_decode,
// paged_attn_decode_shared and attn_fwd_paged when the environment variable
// ATTN_VALIDATE is set to a value other than "0" (a test mode: the call then
// copies the arrays to the host and waits for the copy).
//
// What is checked follows the contract of the tutorial "Chapter 3 Advanced
// principles: performance model and numerical stability", section 3.0: a
// sequence's logical block t / block_size lives in the physical block its
// table row names, and sequences that share a prefix name the same physical
// blocks for it.
#include <cstdint>
#include <string>

#include "../../include/attn.h"

namespace attn {
int set_error(int code, const std::string& msg);   // attn_api.hip
}

namespace {

int bad(const std::string& msg) {
  return attn::set_error(ATTN_ERR_SHAPE, "attn_validate_paged_tables: " + msg);
}

std::string at2(int64_t s, int64_t j) {
  return "[" + std::to_string(s) + "][" + std::to_string(j) + "]";
}

}  // namespace

extern "C" int attn_validate_paged_tables(const int32_t* block_table,
                                          const int32_t* context_lens, int num_seqs,
                                          int max_blocks_per_seq, int max_context_len,
                                          int num_blocks, int block_size,
                                          const int32_t* group_starts,
                                          const int32_t* prefix_lens, int num_groups) {
  try {
    attn::set_error(ATTN_OK, "");
    if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || num_blocks < 0 ||
        block_size <= 0 || num_groups < 0)
      return bad("sizes must be non-negative and block_size positive");
    if (num_seqs == 0) return ATTN_OK;
    if (context_lens == nullptr) return attn::set_error(ATTN_ERR_NULL,
        "attn_validate_paged_tables: context_lens must not be NULL");
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t ctx = context_lens[s];
      if (ctx < 0 || ctx > max_context_len)
        return bad("context_lens[" + std::to_string(s) + "] = " + std::to_string(ctx) +
                   " outside [0, max_context_len = " + std::to_string(max_context_len) + "]");
      const int64_t nb = (ctx + block_size - 1) / block_size;
      if (nb > max_blocks_per_seq)
        return bad("context_lens[" + std::to_string(s) + "] = " + std::to_string(ctx) +
                   " needs " + std::to_string(nb) + " table entries, the row has " +
                   std::to_string(max_blocks_per_seq));
      if (nb > 0 && block_table == nullptr)
        return attn::set_error(ATTN_ERR_NULL,
                               "attn_validate_paged_tables: block_table must not be NULL");
      for (int64_t j = 0; j < nb; ++j) {
        const int32_t id = block_table[(int64_t)s * max_blocks_per_seq + j];
        if (id < 0 || id >= num_blocks)
          return bad("block_table" + at2(s, j) + " = " + std::to_string(id) +
                     " outside [0, num_blocks = " + std::to_string(num_blocks) + ")");
      }
    }
    if (group_starts == nullptr && prefix_lens == nullptr) return ATTN_OK;
    if (group_starts == nullptr || prefix_lens == nullptr)
      return attn::set_error(ATTN_ERR_NULL,
                             "attn_validate_paged_tables: group_starts and prefix_lens go together");
    if (num_groups == 0) return bad("every sequence must be in a group (num_groups is 0)");
    if (group_starts[0] != 0) return bad("group_starts[0] must be 0");
    if (group_starts[num_groups] != num_seqs)
      return bad("group_starts[num_groups] = " + std::to_string(group_starts[num_groups]) +
                 " must equal num_seqs = " + std::to_string(num_seqs));
    // the whole list first: the member loop below indexes with it
    for (int g = 0; g < num_groups; ++g)
      if (group_starts[g + 1] < group_starts[g])
        return bad("group_starts must be non-decreasing (group " + std::to_string(g) + ")");
    for (int g = 0; g < num_groups; ++g) {
      const int gs = group_starts[g], ge = group_starts[g + 1];
      const int64_t plen = prefix_lens[g];
      if (plen < 0)
        return bad("prefix_lens[" + std::to_string(g) + "] = " + std::to_string(plen) +
                   " is negative");
      for (int m = gs; m < ge; ++m) {
        if (plen > context_lens[m])
          return bad("prefix_lens[" + std::to_string(g) + "] = " + std::to_string(plen) +
                     " exceeds context_lens[" + std::to_string(m) + "] = " +
                     std::to_string(context_lens[m]));
        // the prefix's whole blocks are the shared ones: every member names
        // the first member's physical blocks for them
        for (int64_t j = 0; j < plen / block_size; ++j) {
          const int32_t a = block_table[(int64_t)gs * max_blocks_per_seq + j];
          const int32_t b = block_table[(int64_t)m * max_blocks_per_seq + j];
          if (a != b)
            return bad("block_table" + at2(m, j) + " = " + std::to_string(b) +
                       " differs from the group's first member (block_table" + at2(gs, j) +
                       " = " + std::to_string(a) + ") inside the shared prefix of group " +
                       std::to_string(g));
        }
      }
    }
    return ATTN_OK;
  } catch (...) {
    return attn::set_error(ATTN_ERR_HIP, "attn_validate_paged_tables: unexpected host exception");
  }
}
