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
#include <unordered_map>
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
  std::vector<int32_t> blocks;  // exactly ceil(length / bs) ids
};

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct pkv_pool {
  int32_t total = 0;
  int32_t bs = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refs;        // table entries naming each block
  std::map<int64_t, SeqState> seqs;

  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refs[b] = 1;
    return b;
  }
  // One reference less for each id, in order; blocks nobody names any more
  // go on top of the free stack in that order.
  void unref(const int32_t *b, size_t n) {
    for (size_t i = 0; i < n; ++i) refs[b[i]] -= 1;
    for (size_t i = 0; i < n; ++i)
      if (refs[b[i]] == 0) free_stack.push_back(b[i]);
  }
  // Table entries a sequence of `len` tokens gains by growing by n.
  int64_t grow(int64_t len, int64_t n) const { return ceil_div(len + n, bs) - ceil_div(len, bs); }
  // A write of n > 0 tokens into a partial last block that `tail_refs`
  // tables name must first move the sequence to a private copy.
  bool copy_first(int64_t len, int64_t n, int32_t tail_refs) const {
    return n > 0 && len % bs != 0 && tail_refs > 1;
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

// Grow a sequence by n tokens; the caller has checked that the free stack
// holds what this takes. The private copy (if any) is taken first, then the
// new table entries in order; each new token's slot follows from the table.
static void apply_alloc(pkv_pool *p, SeqState &s, int32_t n, int32_t *slots, pkv_cow_t *cow,
                        int32_t *n_cow) {
  *n_cow = 0;
  if (!s.blocks.empty() && p->copy_first(s.length, n, p->refs[s.blocks.back()])) {
    const int32_t shared = s.blocks.back();
    p->refs[shared] -= 1;  // another table still names it
    s.blocks.back() = p->take();
    cow[0].src = shared;
    cow[0].dst = s.blocks.back();
    *n_cow = 1;
  }
  for (int64_t g = p->grow(s.length, n); g > 0; --g) s.blocks.push_back(p->take());
  const int32_t bs = p->bs;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t t = s.length + k;
    slots[k] = s.blocks[t / bs] * bs + t % bs;
  }
  s.length += n;
}

// Preflight of appends of ns[i] tokens to ids[i], i < n, in order, as
// separate appends would see the pool: unknown ids, the int32 length limit
// and the free blocks all of them take together (new entries, plus a copy
// when a member writes into a partial last block still named by another
// table; a copy made earlier in the batch lowers that block's count, and a
// sequence whose append went through owns its last block). Changes nothing.
static int preflight(const pkv_pool *p, const int64_t *ids, const int32_t *ns, int32_t n,
                     std::vector<SeqState *> *rows) {
  std::unordered_map<int64_t, int64_t> len;      // lengths as the batch leaves them
  std::unordered_map<int64_t, char> owns_tail;   // a nonzero append happened
  std::unordered_map<int32_t, int32_t> copied;   // copies made off each shared block
  int64_t need = 0;
  rows->assign(n, nullptr);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(ids[i]);
    if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)ids[i]);
    SeqState *s = const_cast<SeqState *>(&it->second);
    (*rows)[i] = s;
    auto lit = len.find(ids[i]);
    const int64_t L = lit == len.end() ? s->length : lit->second;
    if (L + ns[i] > INT32_MAX)
      return fail(PKV_EINVAL, "sequence %lld would pass INT32_MAX tokens", (long long)ids[i]);
    need += p->grow(L, ns[i]);
    if (!owns_tail[ids[i]] && !s->blocks.empty()) {
      const int32_t tail = s->blocks.back();
      if (p->copy_first(L, ns[i], p->refs[tail] - copied[tail])) {
        need += 1;
        copied[tail] += 1;
      }
    }
    if (ns[i] > 0) owns_tail[ids[i]] = 1;
    len[ids[i]] = L + ns[i];
  }
  if (need > (int64_t)p->free_stack.size())
    return fail(PKV_ENOMEM, "append wants %lld blocks; the pool has %zu", (long long)need,
                p->free_stack.size());
  return PKV_OK;
}

// The invariants of the page pool's validate. Fills are derived from the
// tables once those are known to name only ids inside the pool; `fill_in`
// (when not NULL) stands in for them, so a checker can hand in fills that
// disagree with the tables.
static int check_invariants(const pkv_pool *p, const std::vector<int32_t> *fill_in) {
  const int32_t n = p->total;
  std::vector<char> on_stack(n, 0);
  for (int32_t b : p->free_stack) {
    if (b < 0 || b >= n) return fail(PKV_ECORRUPT, "free stack names id %d outside the pool", b);
    if (on_stack[b]) return fail(PKV_ECORRUPT, "free stack names block %d twice", b);
    on_stack[b] = 1;
  }
  std::vector<int64_t> named(n, 0);
  int64_t logical = 0;
  for (const auto &kv : p->seqs) {
    const SeqState &s = kv.second;
    const long long id = (long long)kv.first;
    if (s.length < 0) return fail(PKV_ECORRUPT, "sequence %lld has a negative length", id);
    if ((int64_t)s.blocks.size() != ceil_div(s.length, p->bs))
      return fail(PKV_ECORRUPT, "sequence %lld: table size disagrees with its length", id);
    std::vector<int32_t> sorted(s.blocks);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return fail(PKV_ECORRUPT, "sequence %lld names one block twice", id);
    for (int32_t b : s.blocks) {
      if (b < 0 || b >= n) return fail(PKV_ECORRUPT, "sequence %lld names id %d outside the pool", id, b);
      named[b] += 1;
    }
    logical += s.length;
  }
  const std::vector<int32_t> fill = fill_in ? *fill_in : p->fills();
  int64_t payload = 0;
  for (int32_t b = 0; b < n; ++b) {
    if (p->refs[b] != named[b])
      return fail(PKV_ECORRUPT, "block %d: count %d but %lld names", b, p->refs[b],
                  (long long)named[b]);
    if (named[b] && on_stack[b]) return fail(PKV_ECORRUPT, "block %d is named and also free", b);
    if (!named[b] && !on_stack[b]) return fail(PKV_ECORRUPT, "block %d is neither named nor free", b);
    if (named[b]) {
      if (fill[b] < 1 || fill[b] > p->bs) return fail(PKV_ECORRUPT, "block %d holds %d tokens", b, fill[b]);
      payload += fill[b];
    }
  }
  if (payload > logical) return fail(PKV_ECORRUPT, "more tokens stored than the sequences hold");
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
  if (p->seqs.count(id)) return fail(PKV_EEXIST, "id %lld is taken", (long long)id);
  p->seqs.emplace(id, SeqState{});
  return PKV_OK;
}

int paged_kv_alloc(pkv_pool *p, int64_t id, int32_t n, int32_t *slots,
                   pkv_cow_t *cow, int32_t *n_cow) {
  if (int rc = check_pool(p)) return rc;
  if (n < 0) return fail(PKV_EINVAL, "an append needs n_tokens >= 0");
  if ((n > 0 && !slots) || !cow || !n_cow)
    return fail(PKV_EINVAL, "slot_mapping_out, cow_out and n_cow_out are required");
  std::vector<SeqState *> row;
  if (int rc = preflight(p, &id, &n, 1, &row)) return rc;
  apply_alloc(p, *row[0], n, slots, cow, n_cow);
  return PKV_OK;
}

int paged_kv_alloc_batch(pkv_pool *p, const int64_t *ids, const int32_t *ns,
                         int32_t n_seqs, int32_t *slots, pkv_cow_t *cow,
                         int32_t *n_cow, int32_t *n_done) {
  if (int rc = check_pool(p)) return rc;
  if (n_seqs < 0) return fail(PKV_EINVAL, "n_seqs must be >= 0");
  if (!n_cow || !n_done || (n_seqs > 0 && (!ids || !ns || !cow)))
    return fail(PKV_EINVAL, "NULL argument");
  *n_cow = 0;
  *n_done = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (ns[i] < 0) return fail(PKV_EINVAL, "n_tokens[%d] < 0", i);
    total += ns[i];
  }
  if (total > 0 && !slots) return fail(PKV_EINVAL, "slot_mapping_out is NULL");
  std::vector<SeqState *> rows;
  if (int rc = preflight(p, ids, ns, n_seqs, &rows)) return rc;
  int64_t off = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t c = 0;
    apply_alloc(p, *rows[i], ns[i], slots + off, cow + *n_cow, &c);
    off += ns[i];
    *n_cow += c;
  }
  *n_done = n_seqs;
  return PKV_OK;
}

int paged_kv_fork(pkv_pool *p, int64_t parent, int64_t child, int32_t prefix) {
  if (int rc = check_pool(p)) return rc;
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)parent);
  if (prefix < 0) return fail(PKV_EINVAL, "prefix_tokens must be >= 0");
  if (prefix > it->second.length)
    return fail(PKV_EINVAL, "prefix of %d tokens is longer than the parent (%d)", prefix,
                it->second.length);
  if (p->seqs.count(child))
    return fail(PKV_EEXIST, "fork target %lld is taken", (long long)child);
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
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)id);
  p->unref(it->second.blocks.data(), it->second.blocks.size());
  p->seqs.erase(it);
  return PKV_OK;
}

int paged_kv_truncate(pkv_pool *p, int64_t id, int32_t new_length) {
  if (int rc = check_pool(p)) return rc;
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)id);
  SeqState &s = it->second;
  if (new_length < 0 || new_length > s.length)
    return fail(PKV_EINVAL, "a new length must lie in [0, %d], not %d", s.length, new_length);
  const size_t keep = (size_t)ceil_div(new_length, p->bs);
  std::vector<int32_t> dropped(s.blocks.begin() + keep, s.blocks.end());
  s.blocks.resize(keep);
  p->unref(dropped.data(), dropped.size());
  s.length = new_length;
  return PKV_OK;
}

int paged_kv_seq_length(const pkv_pool *p, int64_t id, int32_t *len) {
  if (int rc = check_pool(p)) return rc;
  if (!len) return fail(PKV_EINVAL, "len is NULL");
  auto it = p->seqs.find(id);
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)id);
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
  if (it == p->seqs.end()) return fail(PKV_ENOENT, "no sequence with id %lld", (long long)id);
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
      return fail(PKV_ENOENT, "no sequence with id %lld", (long long)ids[i]);
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
  return check_invariants(p, nullptr);
}

}  // extern "C"
