// The host allocator and the prefix-group finder compiled for the CPU under
// AddressSanitizer and UndefinedBehaviorSanitizer (built with g++ by
// tests/test_pool_sanitized.py; no GPU code is involved).
//
//   pool_check corrupt  break one invariant of a valid pool at a time and
//                       expect paged_kv_validate to answer PKV_ECORRUPT with
//                       that rule's message (the rules of the page pool's
//                       validate: course page "Module 10. KV Caches and
//                       Efficient Inference", notebook section 5; refusing
//                       broken states: section 9, negative tests)
//   pool_check ops      replay operations read from stdin, printing what
//                       each returns and the pool after it
//   pool_check groups   read batches of tables from stdin, print the groups
//
// The source files are included so that the checker can reach the pool's
// internal state to corrupt it.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pool.cpp"
#include "groups.cpp"

namespace {

int failures = 0;

// A valid pool with 4-slot blocks: a (6 tokens), b forked from a's 6 tokens
// (both blocks shared), c (9 tokens); 3 of 10 blocks free.
pkv_pool *valid_pool() {
  pkv_pool *p = nullptr;
  if (paged_kv_pool_create(10, 4, nullptr, &p)) std::abort();
  int32_t slots[16], nc;
  pkv_cow_t cow[1];
  if (paged_kv_seq_create(p, 1) || paged_kv_alloc(p, 1, 6, slots, cow, &nc) ||
      paged_kv_fork(p, 1, 2, 6) || paged_kv_seq_create(p, 3) ||
      paged_kv_alloc(p, 3, 9, slots, cow, &nc) || paged_kv_validate(p))
    std::abort();
  return p;
}

void expect_corrupt(const char *rule, const std::function<void(pkv_pool *)> &corrupt,
                    const std::vector<int32_t> *fill = nullptr) {
  pkv_pool *p = valid_pool();
  corrupt(p);
  const int rc = fill ? check_invariants(p, fill) : paged_kv_validate(p);
  const std::string msg = paged_kv_last_error();
  const bool ok = rc == PKV_ECORRUPT && msg.find(rule) != std::string::npos;
  std::printf("%s rule '%s': rc %d, \"%s\"\n", ok ? "ok" : "FAIL", rule, rc, msg.c_str());
  if (!ok) ++failures;
  paged_kv_pool_destroy(p);
}

int corrupt_mode() {
  // the valid pool itself passes
  {
    pkv_pool *p = valid_pool();
    if (paged_kv_validate(p) != PKV_OK) ++failures;
    paged_kv_pool_destroy(p);
  }
  expect_corrupt("outside the pool", [](pkv_pool *p) { p->free_stack.push_back(p->total + 3); });
  expect_corrupt("twice", [](pkv_pool *p) { p->free_stack.push_back(p->free_stack[0]); });
  expect_corrupt("negative length", [](pkv_pool *p) {
    p->seqs[9].length = -3;  // no entries: ceil(-3 / 4) rounds to 0
  });
  expect_corrupt("table size disagrees", [](pkv_pool *p) { p->seqs[3].length = 13; });
  expect_corrupt("names one block twice", [](pkv_pool *p) {
    std::vector<int32_t> &t = p->seqs[3].blocks;
    const int32_t second = t[1];
    t[1] = t[0];
    p->refs[t[0]] += 1;
    p->refs[second] -= 1;
    p->free_stack.push_back(second);
  });
  expect_corrupt("names id 11 outside the pool", [](pkv_pool *p) {
    std::vector<int32_t> &t = p->seqs[3].blocks;
    const int32_t old = t[2];
    t[2] = p->total + 1;
    p->refs[old] -= 1;
    p->free_stack.push_back(old);
  });
  expect_corrupt("count 2 but 1 names", [](pkv_pool *p) { p->refs[p->seqs[3].blocks[0]] += 1; });
  expect_corrupt("named and also free",
                 [](pkv_pool *p) { p->free_stack.push_back(p->seqs[3].blocks[1]); });
  expect_corrupt("neither named nor free", [](pkv_pool *p) { p->free_stack.pop_back(); });
  // fills that disagree with the tables (a pool keeping fill counters)
  {
    pkv_pool *p = valid_pool();
    std::vector<int32_t> fill = p->fills();
    const int32_t last = p->seqs[3].blocks[2];
    paged_kv_pool_destroy(p);
    for (int32_t bad : {0, 5}) {
      std::vector<int32_t> f = fill;
      f[last] = bad;
      const std::string rule = "holds " + std::to_string(bad) + " tokens";
      expect_corrupt(rule.c_str(), [](pkv_pool *) {}, &f);
    }
    // a alone (6 tokens in 2 blocks) with both fills stored as 4
    std::vector<int32_t> f(10, 0);
    pkv_pool *q = valid_pool();
    for (int32_t b : q->seqs[1].blocks) f[b] = 4;
    paged_kv_pool_destroy(q);
    expect_corrupt("more tokens stored", [](pkv_pool *p) {
      if (paged_kv_free(p, 2) || paged_kv_free(p, 3)) std::abort();
    }, &f);
  }
  std::printf("%d failures\n", failures);
  return failures ? 1 : 0;
}

void print_pool(const pkv_pool *p) {
  std::printf("free");
  for (int32_t b : p->free_stack) std::printf(" %d", b);
  std::printf("\n");
  for (const auto &kv : p->seqs) {
    std::printf("seq %lld %d", (long long)kv.first, kv.second.length);
    for (int32_t b : kv.second.blocks) std::printf(" %d", b);
    std::printf("\n");
  }
  pkv_stats_t st;
  if (paged_kv_stats(p, &st)) std::abort();
  std::printf("stats %lld %lld %lld %lld %lld %lld %lld\n", (long long)st.allocated_blocks,
              (long long)st.free_blocks, (long long)st.physical_capacity_tokens,
              (long long)st.physical_payload_tokens, (long long)st.logical_tokens,
              (long long)st.internal_waste_tokens, (long long)st.sharing_savings_tokens);
}

// Lines: "pool N BS [perm...]" first, then
//   create ID | alloc ID N | batch K ID N ID N ... | fork P C PREFIX |
//   free ID | trunc ID N
// After each operation: "rc R", the slots and pairs it returned, the pool.
int ops_mode() {
  std::string line;
  pkv_pool *p = nullptr;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op.empty()) continue;
    int rc = 0;
    std::vector<int32_t> slots;
    std::vector<pkv_cow_t> cow;
    if (op == "pool") {
      int32_t n, bs;
      in >> n >> bs;
      std::vector<int32_t> perm;
      for (int32_t b; in >> b;) perm.push_back(b);
      rc = paged_kv_pool_create(n, bs, perm.empty() ? nullptr : perm.data(), &p);
    } else if (op == "create") {
      long long id;
      in >> id;
      rc = paged_kv_seq_create(p, id);
    } else if (op == "alloc") {
      long long id;
      int32_t n, nc = 0;
      in >> id >> n;
      slots.assign(n > 0 ? n : 1, -7);
      cow.assign(1, pkv_cow_t{-7, -7});
      rc = paged_kv_alloc(p, id, n, slots.data(), cow.data(), &nc);
      slots.resize(rc ? 0 : n);
      cow.resize(rc ? 0 : nc);
    } else if (op == "batch") {
      int32_t k;
      in >> k;
      std::vector<int64_t> ids(k);
      std::vector<int32_t> ns(k);
      int64_t total = 0;
      for (int32_t i = 0; i < k; ++i) {
        long long id;
        in >> id >> ns[i];
        ids[i] = id;
        total += ns[i] > 0 ? ns[i] : 0;
      }
      int32_t nc = 0, done = 0;
      slots.assign(total > 0 ? total : 1, -7);
      cow.assign(k > 0 ? k : 1, pkv_cow_t{-7, -7});
      rc = paged_kv_alloc_batch(p, ids.data(), ns.data(), k, slots.data(), cow.data(), &nc,
                                &done);
      slots.resize(rc ? 0 : total);
      cow.resize(rc ? 0 : nc);
    } else if (op == "fork") {
      long long a, c;
      int32_t n;
      in >> a >> c >> n;
      rc = paged_kv_fork(p, a, c, n);
    } else if (op == "free") {
      long long id;
      in >> id;
      rc = paged_kv_free(p, id);
    } else if (op == "trunc") {
      long long id;
      int32_t n;
      in >> id >> n;
      rc = paged_kv_truncate(p, id, n);
    } else {
      std::fprintf(stderr, "unknown op %s\n", op.c_str());
      return 2;
    }
    std::printf("rc %d\nslots", rc);
    for (int32_t s : slots) std::printf(" %d", s);
    std::printf("\npairs");
    for (const auto &c : cow) std::printf(" %d:%d", c.src, c.dst);
    std::printf("\n");
    if (p) {
      if (paged_kv_validate(p) != PKV_OK) {
        std::printf("invalid %s\n", paged_kv_last_error());
        return 1;
      }
      print_pool(p);
    }
  }
  paged_kv_pool_destroy(p);
  return 0;
}

// Each case: "B MAXB NQ BS MIN_MEMBERS MIN_TOKENS", then B*MAXB table
// entries, then B lengths. Output: the groups as "group TOKENS m1 m2 ...".
int groups_mode() {
  int32_t B, maxb, nq, bs, mm, mt;
  while (std::cin >> B >> maxb >> nq >> bs >> mm >> mt) {
    std::vector<int32_t> tables((size_t)B * maxb), lens(B);
    for (auto &t : tables) std::cin >> t;
    for (auto &l : lens) std::cin >> l;
    std::vector<int32_t> seq_prefix(B), start(B + 1), members(B), tokens(B);
    int32_t ng = 0, mmax = 0, pmax = 0;
    int rc = paged_kv_prefix_groups(tables.data(), maxb, lens.data(), B, nq, bs, mm, mt,
                                    seq_prefix.data(), start.data(), members.data(),
                                    tokens.data(), &ng, &mmax, &pmax);
    std::printf("rc %d groups %d\n", rc, rc ? 0 : ng);
    for (int32_t g = 0; !rc && g < ng; ++g) {
      std::printf("group %d", tokens[g]);
      for (int32_t i = start[g]; i < start[g + 1]; ++i) std::printf(" %d", members[i]);
      std::printf("\n");
    }
  }
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  const std::string mode = argc > 1 ? argv[1] : "";
  if (mode == "corrupt") return corrupt_mode();
  if (mode == "ops") return ops_mode();
  if (mode == "groups") return groups_mode();
  std::fprintf(stderr, "usage: pool_check corrupt|ops|groups\n");
  return 2;
}
