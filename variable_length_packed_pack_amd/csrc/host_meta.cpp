// Host-side packing and ragged-grid metadata (no HIP calls).
//
// vlp_pack_sequences: "gigl.nn.packed_attention", "Data flow of a packed
//   forward", "Example" and "Constraints" (lengths >= 1, int32 cu_seqlens).
// vlp_grid_capacity / vlp_build_ragged_grid: "PyCoRa", "CoRa Metadata"
//   (grid_mapping, block_offsets); "So you wanna CUDA Graph", "Scheduling
//   without max_seqlen" (per-sequence ceiling, prefix sum, decode, G_cap).
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/vlp.h"

namespace {

// ceil(len / c) without overflow for any len in [0, INT32_MAX] and c >= 1.
inline int64_t tiles_for(int64_t len, int64_t c) { return len <= 0 ? 0 : 1 + (len - 1) / c; }

}  // namespace

extern "C" vlp_status vlp_pack_sequences(const int32_t* lengths, int32_t num_seqs,
                                         int32_t max_seq_len, int64_t* flat_index,
                                         int64_t flat_index_cap, int32_t* cu_seqlens,
                                         int64_t* num_tokens) {
  if (!lengths || !cu_seqlens || !num_tokens) return VLP_ERR_NULL;
  if (num_seqs < 1 || max_seq_len < 1) return VLP_ERR_INVALID;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t n = lengths[i];
    if (n < 1 || n > max_seq_len) return VLP_ERR_INVALID;
    total += n;
    if (total > INT32_MAX) return VLP_ERR_OVERFLOW;
  }
  // Validated: now write the boundaries.
  int32_t run = 0;
  cu_seqlens[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    run += lengths[i];
    cu_seqlens[i + 1] = run;
  }
  *num_tokens = total;
  if (!flat_index) return VLP_OK;
  if (flat_index_cap < total) return VLP_ERR_CAPACITY;
  int64_t pos = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t row = static_cast<int64_t>(i) * max_seq_len;
    for (int32_t j = 0; j < lengths[i]; ++j) flat_index[pos++] = row + j;
  }
  return VLP_OK;
}

extern "C" int64_t vlp_grid_capacity(int64_t total_tokens, int32_t num_seqs, int32_t block_m) {
  if (total_tokens < 0 || num_seqs < 0 || block_m < 1) return -1;
  const int64_t m = std::min<int64_t>(total_tokens, num_seqs);
  return m + (total_tokens - m) / block_m;
}

extern "C" vlp_status vlp_build_ragged_grid(const int32_t* cu_seqlens, int32_t num_seqs,
                                            int32_t block_m, int32_t* block_offsets,
                                            int32_t* grid_mapping, int32_t* tile_order,
                                            int64_t grid_cap, int64_t* num_blocks) {
  if (!cu_seqlens || !block_offsets || !num_blocks) return VLP_ERR_NULL;
  if (num_seqs < 1 || block_m < 1) return VLP_ERR_INVALID;
  if (cu_seqlens[0] != 0) return VLP_ERR_INVALID;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (cu_seqlens[i + 1] < cu_seqlens[i]) return VLP_ERR_INVALID;

  // Exclusive prefix of per-sequence tile counts; G < 2^31 because every
  // tile holds at least one of at most INT32_MAX tokens.
  int64_t g = 0;
  block_offsets[0] = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    g += tiles_for(static_cast<int64_t>(cu_seqlens[i + 1]) - cu_seqlens[i], block_m);
    block_offsets[i + 1] = static_cast<int32_t>(g);
  }
  *num_blocks = g;
  if ((grid_mapping || tile_order) && g > grid_cap) return VLP_ERR_CAPACITY;

  if (grid_mapping) {
    for (int32_t i = 0; i < num_seqs; ++i)
      for (int32_t f = block_offsets[i]; f < block_offsets[i + 1]; ++f) grid_mapping[f] = i;
  }
  if (tile_order) {
    // Longest sequence first; equal lengths keep their index order.
    std::vector<int32_t> order(num_seqs);
    for (int32_t i = 0; i < num_seqs; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return (cu_seqlens[a + 1] - cu_seqlens[a]) > (cu_seqlens[b + 1] - cu_seqlens[b]);
    });
    int64_t pos = 0;
    for (int32_t i : order)
      for (int32_t f = block_offsets[i + 1] - 1; f >= block_offsets[i]; --f)
        tile_order[pos++] = f;
  }
  return VLP_OK;
}
