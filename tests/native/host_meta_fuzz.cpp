// Fuzz driver for the host metadata functions of libvlp (host_meta.cpp),
// built by tests/test_host_sanitizers.py with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every buffer is sized
// exactly (std::vector), so an access one past the end is reported.
//
// Checked for random inputs (seeded; zero-length sequences, single-token
// sequences, lengths at max_seq_len, block sizes 1..300):
//   vlp_pack_sequences: cu[0] = 0, cu[i+1] - cu[i] = len_i, flat_index
//     = concat_i [i * max_seq_len + j, j < len_i] ("gigl.nn.packed_attention",
//     "Example");
//   vlp_build_ragged_grid: block_offsets is the exclusive prefix of
//     ceil(len_i / C), grid_mapping[f] is the owner of tile f, tile_order is a
//     permutation with lengths non-increasing and each sequence's tiles last
//     first ("PyCoRa", "CoRa Metadata"; "So you wanna CUDA Graph", "Scheduling
//     without max_seqlen"); G <= vlp_grid_capacity;
// and every documented error path (NULL pointers, invalid lengths, token
// totals beyond int32, capacity too small, broken cu_seqlens).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "../../include/vlp.h"

static int g_fail = 0;
#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);     \
      ++g_fail;                                                              \
    }                                                                        \
  } while (0)

static void pack_case(const std::vector<int32_t>& len, int32_t max_len) {
  const int32_t b = static_cast<int32_t>(len.size());
  std::vector<int32_t> cu(b + 1, -7);
  int64_t total = -1;
  CHECK(vlp_pack_sequences(len.data(), b, max_len, nullptr, 0, cu.data(), &total) == VLP_OK);
  int64_t want = 0;
  for (int32_t n : len) want += n;
  CHECK(total == want);
  CHECK(cu[0] == 0);
  for (int32_t i = 0; i < b; ++i) CHECK(cu[i + 1] - cu[i] == len[i]);
  std::vector<int64_t> flat(static_cast<size_t>(total));
  if (total > 0) {
    CHECK(vlp_pack_sequences(len.data(), b, max_len, flat.data(), total - 1, cu.data(), &total) ==
          VLP_ERR_CAPACITY);
  }
  CHECK(vlp_pack_sequences(len.data(), b, max_len, flat.data(), total, cu.data(), &total) == VLP_OK);
  size_t pos = 0;
  for (int32_t i = 0; i < b; ++i)
    for (int32_t j = 0; j < len[i]; ++j) CHECK(flat[pos++] == static_cast<int64_t>(i) * max_len + j);
  CHECK(pos == flat.size());
}

static void grid_case(const std::vector<int32_t>& len, int32_t block_m) {
  const int32_t b = static_cast<int32_t>(len.size());
  std::vector<int32_t> cu(b + 1, 0);
  for (int32_t i = 0; i < b; ++i) cu[i + 1] = cu[i] + len[i];
  std::vector<int32_t> bo(b + 1, -1);
  int64_t g = -1;
  CHECK(vlp_build_ragged_grid(cu.data(), b, block_m, bo.data(), nullptr, nullptr, 0, &g) == VLP_OK);
  int64_t want = 0;
  CHECK(bo[0] == 0);
  for (int32_t i = 0; i < b; ++i) {
    want += (len[i] + static_cast<int64_t>(block_m) - 1) / block_m;
    CHECK(bo[i + 1] == want);
  }
  CHECK(g == want);
  CHECK(g <= vlp_grid_capacity(cu[b], b, block_m));
  std::vector<int32_t> gm(static_cast<size_t>(g)), to(static_cast<size_t>(g));
  if (g > 0) {
    std::vector<int32_t> small(static_cast<size_t>(g));  // room for g, capacity stated as g - 1
    CHECK(vlp_build_ragged_grid(cu.data(), b, block_m, bo.data(), small.data(), nullptr, g - 1, &g) ==
          VLP_ERR_CAPACITY);
  }
  CHECK(vlp_build_ragged_grid(cu.data(), b, block_m, bo.data(), gm.data(), to.data(), g, &g) == VLP_OK);
  for (int32_t i = 0; i < b; ++i)
    for (int32_t f = bo[i]; f < bo[i + 1]; ++f) CHECK(gm[f] == i);
  std::vector<char> seen(static_cast<size_t>(g), 0);
  int32_t prev_len = INT32_MAX;
  for (int64_t s = 0; s < g; ++s) {
    const int32_t f = to[s];
    CHECK(f >= 0 && f < g);
    if (f < 0 || f >= g) continue;
    CHECK(!seen[f]);
    seen[f] = 1;
    const int32_t owner = gm[f];
    CHECK(len[owner] <= prev_len);  // longest sequences first
    prev_len = len[owner];
    if (s > 0 && gm[to[s - 1]] == owner) CHECK(to[s - 1] == f + 1);  // last tile first
  }
}

static void error_paths() {
  int32_t len[3] = {3, 1, 2};
  int32_t cu[4] = {0, 3, 4, 6};
  int64_t total = 0, g = 0;
  int32_t bo[4];
  CHECK(vlp_pack_sequences(nullptr, 3, 3, nullptr, 0, cu, &total) == VLP_ERR_NULL);
  CHECK(vlp_pack_sequences(len, 3, 3, nullptr, 0, nullptr, &total) == VLP_ERR_NULL);
  CHECK(vlp_pack_sequences(len, 3, 3, nullptr, 0, cu, nullptr) == VLP_ERR_NULL);
  CHECK(vlp_pack_sequences(len, 0, 3, nullptr, 0, cu, &total) == VLP_ERR_INVALID);
  CHECK(vlp_pack_sequences(len, 3, 2, nullptr, 0, cu, &total) == VLP_ERR_INVALID);  // 3 > max
  int32_t zero[2] = {1, 0};
  CHECK(vlp_pack_sequences(zero, 2, 3, nullptr, 0, cu, &total) == VLP_ERR_INVALID);
  int32_t huge[3] = {INT32_MAX, INT32_MAX, 5};
  int32_t cu3[4];
  CHECK(vlp_pack_sequences(huge, 3, INT32_MAX, nullptr, 0, cu3, &total) == VLP_ERR_OVERFLOW);
  CHECK(vlp_build_ragged_grid(nullptr, 3, 64, bo, nullptr, nullptr, 0, &g) == VLP_ERR_NULL);
  CHECK(vlp_build_ragged_grid(cu, 3, 0, bo, nullptr, nullptr, 0, &g) == VLP_ERR_INVALID);
  int32_t bad0[4] = {1, 3, 4, 6};
  CHECK(vlp_build_ragged_grid(bad0, 3, 64, bo, nullptr, nullptr, 0, &g) == VLP_ERR_INVALID);
  int32_t down[4] = {0, 3, 2, 6};
  CHECK(vlp_build_ragged_grid(down, 3, 64, bo, nullptr, nullptr, 0, &g) == VLP_ERR_INVALID);
  int32_t big_cu[3] = {0, INT32_MAX, INT32_MAX};
  int32_t bo2[3];
  CHECK(vlp_build_ragged_grid(big_cu, 2, 1, bo2, nullptr, nullptr, 0, &g) == VLP_OK && g == INT32_MAX);
  CHECK(vlp_grid_capacity(-1, 3, 64) == -1);
  CHECK(vlp_grid_capacity(10, 3, 0) == -1);
  CHECK(vlp_grid_capacity(INT32_MAX, INT32_MAX, 1) == INT32_MAX);
}

int main(int argc, char** argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 3000;
  std::mt19937_64 rng(20251203);
  error_paths();
  for (int c = 0; c < cases; ++c) {
    const int32_t b = 1 + static_cast<int32_t>(rng() % 64);
    const int32_t max_len = 1 + static_cast<int32_t>(rng() % 400);
    std::vector<int32_t> len(b);
    for (auto& n : len) {
      const uint64_t kind = rng() % 8;
      n = kind == 0 ? 1 : kind == 1 ? max_len : 1 + static_cast<int32_t>(rng() % max_len);
    }
    pack_case(len, max_len);
    const int32_t block_m = 1 + static_cast<int32_t>(rng() % 300);
    std::vector<int32_t> glen(len);
    for (auto& n : glen)
      if (rng() % 5 == 0) n = 0;  // zero-length sequences own no tiles
    grid_case(glen, block_m);
  }
  printf("host_meta fuzz: %d cases, %d failed checks\n", cases, g_fail);
  return g_fail ? 1 : 0;
}
