// Shared-prefix groups of a batch, found from its block tables.
//
// Sharing physical blocks within and across requests is the point of
// PagedAttention (vLLM abstract on the papers page "external vector
// cache"); a fork shares the leading blocks of a parent by reference counts
// (course page "Module 10. KV Caches and Efficient Inference", notebook
// section 5, share_prefix). Sequences whose tables begin with the same
// physical block therefore share a prefix: the longest run of leading block
// ids common to all of them. This file only reads tables; it decides which
// tokens the shared-prefix attention computes once per group.
#include <algorithm>
#include <cstdint>
#include <map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pkv::fail;

extern "C" int paged_kv_prefix_groups(const int32_t *block_tables, int32_t max_blocks,
                                      const int32_t *context_lens, int32_t B, int32_t nq,
                                      int32_t bs, int32_t min_members, int32_t min_tokens,
                                      int32_t *seq_prefix, int32_t *group_start,
                                      int32_t *members, int32_t *group_tokens,
                                      int32_t *n_groups, int32_t *max_members,
                                      int32_t *max_prefix) {
  if (!block_tables || !context_lens || !seq_prefix || !group_start || !members ||
      !group_tokens || !n_groups || !max_members || !max_prefix)
    return fail(PKV_EINVAL, "NULL pointer");
  if (B <= 0 || max_blocks <= 0 || nq <= 0 || bs <= 0 || bs % 16)
    return fail(PKV_EINVAL, "sizes must be positive and block_size a multiple of 16");
  if (min_members < 2) return fail(PKV_EINVAL, "a group needs at least two members");
  if (min_tokens < 16) return fail(PKV_EINVAL, "min_tokens must be at least 16");
  const int64_t max_ctx = (int64_t)max_blocks * bs;

  // candidates: sequences with a usable length, keyed by their first block
  std::map<int32_t, std::vector<int32_t>> by_first;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t L = context_lens[b];
    seq_prefix[b] = 0;
    if (L < nq || L > max_ctx) continue;
    const int32_t first = block_tables[(size_t)b * max_blocks];
    if (first < 0) continue;
    by_first[first].push_back(b);
  }

  int32_t ng = 0, nm = 0, big = 0, longest = 0;
  group_start[0] = 0;
  for (const auto &kv : by_first) {
    const std::vector<int32_t> &g = kv.second;
    if ((int32_t)g.size() < min_members) continue;
    // every query row of every member must see the whole prefix, and only
    // the members' own blocks can be shared
    int64_t cap = max_ctx;
    for (int32_t b : g) cap = std::min<int64_t>(cap, (int64_t)context_lens[b] - nq + 1);
    const int64_t cap_blocks = (cap + bs - 1) / bs;
    const int32_t *lead = block_tables + (size_t)g[0] * max_blocks;
    int64_t common = 0;
    while (common < cap_blocks) {
      const int32_t blk = lead[common];
      bool same = blk >= 0;
      for (size_t i = 1; same && i < g.size(); ++i)
        same = block_tables[(size_t)g[i] * max_blocks + common] == blk;
      if (!same) break;
      ++common;
    }
    const int64_t tokens = std::min<int64_t>(common * bs, cap) / 16 * 16;  // whole tiles
    if (tokens < min_tokens) continue;
    for (int32_t b : g) {
      members[nm++] = b;
      seq_prefix[b] = (int32_t)tokens;
    }
    group_tokens[ng] = (int32_t)tokens;
    group_start[++ng] = nm;
    big = std::max<int32_t>(big, (int32_t)g.size());
    longest = std::max<int32_t>(longest, (int32_t)tokens);
  }
  *n_groups = ng;
  *max_members = big;
  *max_prefix = longest;
  return PKV_OK;
}
