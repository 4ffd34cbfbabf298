// Host-side block allocator: pool of fixed-size physical blocks, per-sequence
// block tables, prefix sharing with reference counts, copy-on-write, release
// and truncate.
//
// Behaviour follows the page-pool simulator of the course page "Module 10. KV
// Caches and Efficient Inference" (notebook "KV cache and serving: bytes,
// pages, and ceilings", section 5 "Page pool: prefix sharing and
// copy-on-write"), with the slot mapping and block reclamation of "NeuralOps
// v1.3.4" (Paged KV Cache Engine). Design for the hot path:
//   * every operation is O(blocks it touches); per-block fills (used only by
//     the counters and the invariant check) are derived on demand instead of
//     being refreshed after every operation;
//   * sequences live in an ordered map so listings are sorted by id;
//   * errors are detected before any mutation, so a failed call leaves the
//     pool exactly as it was.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

std::string &last_error() {
  static thread_local std::string msg;
  return msg;
}

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  last_error() = buf;
  return code;
}

}  // namespace pkv

using pkv::fail;

struct SeqState {
  int32_t length = 0;
  std::vector<int32_t> blocks;
};

struct pkv_pool {
  int32_t total = 0;
  int32_t bs = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refs;
  std::map<int64_t, SeqState> seqs;

  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_stack.push_back(b);
  }
  // Blocks an append of n tokens needs, counting a private copy of a shared
  // partial last block.
  int64_t blocks_needed(const SeqState &s, int64_t n) const {
    if (n == 0) return 0;
    int64_t used = s.length % bs, room = 0, extra = 0;
    if (!s.blocks.empty() && used) {
      room = bs - used;
      if (refs[s.blocks.back()] > 1) extra = 1;
    }
    int64_t rest = std::max<int64_t>(0, n - room);
    return extra + (rest + bs - 1) / bs;
  }
  std::vector<int32_t> fills() const {
    std::vector<int32_t> f(total, 0);
    for (const auto &kv : seqs) {
      const SeqState &s = kv.second;
      for (size_t j = 0; j < s.blocks.size(); ++j) {
        int64_t here = std::min<int64_t>(bs, (int64_t)s.length - (int64_t)j * bs);
        f[s.blocks[j]] = std::max<int32_t>(f[s.blocks[j]], (int32_t)here);
      }
    }
    return f;
  }
};

static int check_pool(const pkv_pool *p) {
  return p ? PKV_OK : fail(PKV_EINVAL, "pool handle is NULL");
}

// Append without argument checks (callers check); returns status.
static int do_alloc(pkv_pool *p, int64_t id, int32_t n, int32_t *slots,
                    pkv_cow_t *cow, int32_t *n_cow) {
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)id);
  SeqState &s = it->second;
  if ((int64_t)s.length + n > INT32_MAX)
    return fail(PKV_EINVAL, "sequence %lld would exceed INT32_MAX tokens", (long long)id);
  int64_t need = p->blocks_needed(s, n);
  if (need > (int64_t)p->free_stack.size())
    return fail(PKV_ENOMEM, "need %lld free blocks, %zu remain", (long long)need,
                p->free_stack.size());
  *n_cow = 0;
  if (n == 0) return PKV_OK;
  const int32_t bs = p->bs;
  int32_t used = s.length % bs;
  int32_t k = 0;
  if (!s.blocks.empty() && used) {
    int32_t last = s.blocks.back();
    if (p->refs[last] > 1) {
      p->refs[last] -= 1;
      int32_t fresh = p->take();
      s.blocks.back() = fresh;
      cow[0].src = last;
      cow[0].dst = fresh;
      *n_cow = 1;
    }
    int32_t take = std::min(n, bs - used);
    const int32_t base = s.blocks.back() * bs + used;
    for (int32_t j = 0; j < take; ++j) slots[k++] = base + j;
    s.length += take;
  }
  while (k < n) {
    int32_t take = std::min(n - k, bs);
    int32_t b = p->take();
    s.blocks.push_back(b);
    for (int32_t j = 0; j < take; ++j) slots[k++] = b * bs + j;
    s.length += take;
  }
  return PKV_OK;
}

extern "C" {

const char *paged_kv_last_error(void) { return pkv::last_error().c_str(); }

int paged_kv_pool_create(int32_t total_blocks, int32_t block_size,
                         const int32_t *initial_free_stack, pkv_pool **out) {
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  if (total_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "total_blocks and block_size must be positive");
  if ((int64_t)total_blocks * block_size > INT32_MAX)
    return fail(PKV_EINVAL, "total_blocks * block_size exceeds INT32_MAX slots");
  std::vector<int32_t> stack(total_blocks);
  if (initial_free_stack) {
    std::vector<char> seen(total_blocks, 0);
    for (int32_t i = 0; i < total_blocks; ++i) {
      int32_t b = initial_free_stack[i];
      if (b < 0 || b >= total_blocks || seen[b])
        return fail(PKV_EINVAL, "initial free stack is not a permutation of 0..N-1");
      seen[b] = 1;
      stack[i] = b;
    }
  } else {
    for (int32_t i = 0; i < total_blocks; ++i) stack[i] = total_blocks - 1 - i;
  }
  pkv_pool *p = new pkv_pool;
  p->total = total_blocks;
  p->bs = block_size;
  p->free_stack = std::move(stack);
  p->refs.assign(total_blocks, 0);
  *out = p;
  return PKV_OK;
}

void paged_kv_pool_destroy(pkv_pool *pool) { delete pool; }

int paged_kv_seq_create(pkv_pool *p, int64_t id) {
  if (int rc = check_pool(p)) return rc;
  if (p->seqs.count(id)) return fail(PKV_EEXIST, "sequence %lld already exists", (long long)id);
  p->seqs.emplace(id, SeqState{});
  return PKV_OK;
}

int paged_kv_alloc(pkv_pool *p, int64_t id, int32_t n, int32_t *slots,
                   pkv_cow_t *cow, int32_t *n_cow) {
  if (int rc = check_pool(p)) return rc;
  if (n < 0) return fail(PKV_EINVAL, "n_tokens must be >= 0");
  if ((n > 0 && !slots) || !cow || !n_cow)
    return fail(PKV_EINVAL, "slot_mapping_out, cow_out and n_cow_out are required");
  return do_alloc(p, id, n, slots, cow, n_cow);
}

int paged_kv_alloc_batch(pkv_pool *p, const int64_t *ids, const int32_t *ns,
                         int32_t n_seqs, int32_t *slots, pkv_cow_t *cow,
                         int32_t *n_cow, int32_t *n_done) {
  if (int rc = check_pool(p)) return rc;
  if (n_seqs < 0) return fail(PKV_EINVAL, "n_seqs must be >= 0");
  if (!n_cow || !n_done || (n_seqs > 0 && (!ids || !ns || !cow)))
    return fail(PKV_EINVAL, "NULL argument");
  int64_t total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (ns[i] < 0) return fail(PKV_EINVAL, "n_tokens[%d] < 0", i);
    total += ns[i];
  }
  if (total > 0 && !slots) return fail(PKV_EINVAL, "slot_mapping_out is NULL");
  *n_cow = 0;
  *n_done = 0;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t c = 0;
    int rc = do_alloc(p, ids[i], ns[i], slots + off, cow + *n_cow, &c);
    if (rc) return rc;
    off += ns[i];
    *n_cow += c;
    *n_done = i + 1;
  }
  return PKV_OK;
}

int paged_kv_fork(pkv_pool *p, int64_t parent, int64_t child, int32_t prefix) {
  if (int rc = check_pool(p)) return rc;
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)parent);
  if (prefix < 0) return fail(PKV_EINVAL, "prefix_tokens must be >= 0");
  if (prefix > it->second.length)
    return fail(PKV_EINVAL, "prefix_tokens %d exceeds parent length %d", prefix,
                it->second.length);
  if (p->seqs.count(child))
    return fail(PKV_EEXIST, "target sequence %lld already exists", (long long)child);
  SeqState s;
  s.length = prefix;
  int32_t count = (prefix + p->bs - 1) / p->bs;
  s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + count);
  for (int32_t b : s.blocks) p->refs[b] += 1;
  p->seqs.emplace(child, std::move(s));
  return PKV_OK;
}

int paged_kv_free(pkv_pool *p, int64_t id) {
  if (int rc = check_pool(p)) return rc;
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)id);
  for (int32_t b : it->second.blocks) p->drop(b);
  p->seqs.erase(it);
  return PKV_OK;
}

int paged_kv_truncate(pkv_pool *p, int64_t id, int32_t new_length) {
  if (int rc = check_pool(p)) return rc;
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)id);
  SeqState &s = it->second;
  if (new_length < 0 || new_length > s.length)
    return fail(PKV_EINVAL, "new_length %d outside [0, %d]", new_length, s.length);
  size_t keep = (size_t)((new_length + p->bs - 1) / p->bs);
  for (size_t j = keep; j < s.blocks.size(); ++j) p->drop(s.blocks[j]);
  s.blocks.resize(keep);
  s.length = new_length;
  return PKV_OK;
}

int paged_kv_seq_length(const pkv_pool *p, int64_t id, int32_t *len) {
  if (int rc = check_pool(p)) return rc;
  if (!len) return fail(PKV_EINVAL, "len is NULL");
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)id);
  *len = it->second.length;
  return PKV_OK;
}

int paged_kv_seq_ids(const pkv_pool *p, int64_t *ids, int32_t cap, int32_t *n_out) {
  if (int rc = check_pool(p)) return rc;
  if (!n_out) return fail(PKV_EINVAL, "n_out is NULL");
  *n_out = (int32_t)p->seqs.size();
  if (!ids) return PKV_OK;  // count only
  if (cap < *n_out) return fail(PKV_EINVAL, "capacity %d < %d sequences", cap, *n_out);
  int32_t i = 0;
  for (const auto &kv : p->seqs) ids[i++] = kv.first;
  return PKV_OK;
}

int paged_kv_page_table(const pkv_pool *p, int64_t id, int32_t *out, int32_t cap,
                        int32_t *n_out) {
  if (int rc = check_pool(p)) return rc;
  if (!n_out) return fail(PKV_EINVAL, "n_out is NULL");
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "unknown sequence %lld", (long long)id);
  const auto &bl = it->second.blocks;
  *n_out = (int32_t)bl.size();
  if ((size_t)cap < bl.size() || (cap > 0 && !out))
    return fail(PKV_EINVAL, "capacity %d < %zu blocks", cap, bl.size());
  std::copy(bl.begin(), bl.end(), out);
  return PKV_OK;
}

int paged_kv_free_stack(const pkv_pool *p, int32_t *out, int32_t cap, int32_t *n_out) {
  if (int rc = check_pool(p)) return rc;
  if (!n_out) return fail(PKV_EINVAL, "n_out is NULL");
  *n_out = (int32_t)p->free_stack.size();
  if ((size_t)cap < p->free_stack.size() || (cap > 0 && !out))
    return fail(PKV_EINVAL, "capacity %d < %zu free blocks", cap, p->free_stack.size());
  std::copy(p->free_stack.begin(), p->free_stack.end(), out);
  return PKV_OK;
}

int paged_kv_block_tables(const pkv_pool *p, const int64_t *ids, int32_t n,
                          int32_t max_blocks, int32_t *tables, int32_t *lens) {
  if (int rc = check_pool(p)) return rc;
  if (n < 0 || max_blocks <= 0) return fail(PKV_EINVAL, "n_seqs < 0 or max_blocks <= 0");
  if (n > 0 && (!ids || !tables || !lens)) return fail(PKV_EINVAL, "NULL argument");
  // check everything first so a failure writes nothing
  std::vector<const SeqState *> rows(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(ids[i]);
    if (it == p->seqs.end())
      return fail(PKV_ENOENT, "unknown sequence %lld", (long long)ids[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return fail(PKV_EINVAL, "sequence %lld has %zu blocks > max_blocks %d",
                  (long long)ids[i], it->second.blocks.size(), max_blocks);
    rows[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t *row = tables + (size_t)i * max_blocks;
    const auto &bl = rows[i]->blocks;
    std::copy(bl.begin(), bl.end(), row);
    std::fill(row + bl.size(), row + max_blocks, -1);
    lens[i] = rows[i]->length;
  }
  return PKV_OK;
}

int paged_kv_stats(const pkv_pool *p, pkv_stats_t *st) {
  if (int rc = check_pool(p)) return rc;
  if (!st) return fail(PKV_EINVAL, "out is NULL");
  std::vector<int32_t> f = p->fills();
  int64_t payload = 0, logical = 0;
  for (int32_t b = 0; b < p->total; ++b)
    if (p->refs[b]) payload += f[b];
  for (const auto &kv : p->seqs) logical += kv.second.length;
  st->free_blocks = (int64_t)p->free_stack.size();
  st->allocated_blocks = p->total - st->free_blocks;
  st->physical_capacity_tokens = st->allocated_blocks * p->bs;
  st->physical_payload_tokens = payload;
  st->logical_tokens = logical;
  st->internal_waste_tokens = st->physical_capacity_tokens - payload;
  st->sharing_savings_tokens = logical - payload;
  return PKV_OK;
}

int paged_kv_validate(const pkv_pool *p) {
  if (int rc = check_pool(p)) return rc;
  const int32_t n = p->total;
  std::vector<char> on_free(n, 0);
  for (int32_t b : p->free_stack) {
    if (b < 0 || b >= n) return fail(PKV_ECORRUPT, "free stack holds invalid id %d", b);
    if (on_free[b]) return fail(PKV_ECORRUPT, "free stack holds %d twice", b);
    on_free[b] = 1;
  }
  std::vector<int64_t> expect(n, 0);
  int64_t logical = 0;
  for (const auto &kv : p->seqs) {
    const SeqState &s = kv.second;
    if (s.length < 0) return fail(PKV_ECORRUPT, "negative length");
    if ((int64_t)s.blocks.size() != ((int64_t)s.length + p->bs - 1) / p->bs)
      return fail(PKV_ECORRUPT, "table length does not match length of %lld",
                  (long long)kv.first);
    std::vector<int32_t> sorted(s.blocks);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return fail(PKV_ECORRUPT, "sequence %lld names a block twice", (long long)kv.first);
    for (int32_t b : s.blocks) {
      if (b < 0 || b >= n) return fail(PKV_ECORRUPT, "table holds invalid id %d", b);
      expect[b] += 1;
    }
    logical += s.length;
  }
  std::vector<int32_t> f = p->fills();
  int64_t payload = 0;
  for (int32_t b = 0; b < n; ++b) {
    if (p->refs[b] != expect[b])
      return fail(PKV_ECORRUPT, "block %d: ref %d but %lld table entries", b, p->refs[b],
                  (long long)expect[b]);
    if (p->refs[b] == 0) {
      if (!on_free[b] || f[b] != 0)
        return fail(PKV_ECORRUPT, "unreferenced block %d is not clean and free", b);
    } else {
      if (on_free[b]) return fail(PKV_ECORRUPT, "referenced block %d is free", b);
      if (f[b] < 1 || f[b] > p->bs) return fail(PKV_ECORRUPT, "block %d fill %d", b, f[b]);
      payload += f[b];
    }
  }
  if (logical < payload) return fail(PKV_ECORRUPT, "payload exceeds logical tokens");
  return PKV_OK;
}

}  // extern "C"
