// Seeded random operation stream over the host half of librkv (radix tree +
// FIFO allocator), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_radix_sanitized.py.  After every operation it checks, from
// the canonical dump and the free list alone: every slot of the pool is owned
// exactly once (tree, free list or the driver), labels are non-empty, sibling
// first tokens are distinct and ascending, locks are non-negative, and the
// statistics agree with the dump.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "rkv.h"

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

static void verify(rkv_tree* t, int64_t P, const std::vector<int32_t>& held) {
  int64_t n = 0;
  CHECK(rkv_radix_serialize(t, nullptr, 0, &n) == RKV_OK);
  std::vector<int64_t> d((size_t)n);
  CHECK(rkv_radix_serialize(t, d.data(), n, &n) == RKV_OK);
  int64_t fl = 0;
  CHECK(rkv_free_list(t, nullptr, 0, &fl) == RKV_OK);
  std::vector<int32_t> fifo((size_t)fl + 1);
  CHECK(rkv_free_list(t, fifo.data(), fl, &fl) == RKV_OK);
  std::vector<int> seen((size_t)P, 0);
  int64_t cached = 0, nodes = 0, locked = 0;
  std::vector<std::pair<int64_t, int64_t>> last_first;  // (parent, first token) in dump order
  for (size_t i = 0; i < d.size();) {
    const int64_t id = d[i], parent = d[i + 1], lock = d[i + 3], len = d[i + 4];
    CHECK(lock >= 0);
    if (id != 0) {
      CHECK(len > 0);
      ++nodes;
      cached += len;
      if (lock > 0) locked += len;
      last_first.push_back({parent, d[i + 5]});
    }
    for (int64_t k = 0; k < len; ++k) {
      const int64_t s = d[i + 5 + len + k];
      CHECK(s >= 0 && s < P);
      ++seen[(size_t)s];
    }
    i += 5 + 2 * (size_t)len;
  }
  // siblings: same parent appear in ascending first-token order, distinct
  for (size_t a = 0; a < last_first.size(); ++a)
    for (size_t b = a + 1; b < last_first.size(); ++b)
      if (last_first[a].first == last_first[b].first) CHECK(last_first[a].second != last_first[b].second);
  for (int64_t k = 0; k < fl; ++k) ++seen[(size_t)fifo[(size_t)k]];
  for (int32_t s : held) ++seen[(size_t)s];
  for (int64_t s = 0; s < P; ++s) CHECK(seen[(size_t)s] == 1);
  int64_t st[8];
  CHECK(rkv_stats(t, st) == RKV_OK);
  CHECK(st[0] == cached && st[1] == fl && st[3] == locked && st[2] == cached - locked && st[4] == nodes);
}

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int ops = argc > 2 ? std::atoi(argv[2]) : 20000;
  const int64_t P = 64;
  std::mt19937_64 rng(seed);
  rkv_tree* t = nullptr;
  CHECK(rkv_tree_create(&t, P, nullptr) == RKV_OK);
  std::vector<int32_t> held;
  std::vector<int64_t> locked_nodes;
  const int vocab = 2 + (int)(seed % 3);
  for (int op = 0; op < ops; ++op) {
    const int kind = (int)(rng() % 100);
    const int L = 1 + (int)(rng() % 14);
    std::vector<int32_t> tok((size_t)L);
    for (auto& x : tok) x = (int32_t)(rng() % (uint64_t)vocab);
    if (kind < 25) {
      std::vector<int32_t> out((size_t)L);
      int64_t m = 0, node = 0, peeked = -1;
      CHECK(rkv_radix_peek(t, tok.data(), L, &peeked) == RKV_OK);
      CHECK(rkv_radix_match(t, tok.data(), L, out.data(), &m, &node) == RKV_OK);
      CHECK(m >= 0 && m <= L);
      CHECK(peeked == m);   // the read-only walk finds what the match finds
      if (node != 0 && (rng() & 1)) {
        CHECK(rkv_radix_lock(t, node) == RKV_OK);
        locked_nodes.push_back(node);
      }
    } else if (kind < 55) {
      std::vector<int32_t> sl((size_t)L);
      int rc = rkv_alloc(t, L, sl.data());
      if (rc == RKV_ENOSPC) {
        int64_t fl = 0, freed = 0;
        CHECK(rkv_free_list(t, nullptr, 0, &fl) == RKV_OK);
        rc = rkv_radix_evict(t, L - fl, &freed);
        CHECK(rc == RKV_OK || rc == RKV_EBUSY);
        rc = rkv_alloc(t, L, sl.data());
      }
      if (rc == RKV_OK) {
        int64_t m = 0;
        CHECK(rkv_radix_insert(t, tok.data(), sl.data(), L, &m) == RKV_OK);
      } else {
        CHECK(rc == RKV_ENOSPC);
      }
    } else if (kind < 65) {
      if (!locked_nodes.empty()) {
        const size_t k = (size_t)(rng() % locked_nodes.size());
        CHECK(rkv_radix_unlock(t, locked_nodes[k]) == RKV_OK);
        locked_nodes.erase(locked_nodes.begin() + (long)k);
      }
    } else if (kind < 75) {
      int64_t freed = 0;
      const int rc = rkv_radix_evict(t, 1 + (int64_t)(rng() % 8), &freed);
      CHECK(rc == RKV_OK || rc == RKV_EBUSY);
    } else if (kind < 82) {
      const int n = (int)(rng() % 5);
      std::vector<int32_t> sl((size_t)n + 1);
      if (rkv_alloc(t, n, sl.data()) == RKV_OK) held.insert(held.end(), sl.begin(), sl.begin() + n);
    } else if (kind < 88) {
      if (!held.empty()) {
        const size_t k = (size_t)(rng() % held.size());
        CHECK(rkv_free(t, &held[k], 1) == RKV_OK);
        held.erase(held.begin() + (long)k);
      }
    } else {
      // a small batch through prepare / commit
      const int B = 1 + (int)(rng() % 3);
      std::vector<int32_t> flat;
      std::vector<int64_t> indptr(1, 0);
      int64_t ld = 1;
      for (int r = 0; r < B; ++r) {
        const int Lr = 1 + (int)(rng() % 12);
        for (int k = 0; k < Lr; ++k) flat.push_back((int32_t)(rng() % (uint64_t)vocab));
        indptr.push_back((int64_t)flat.size());
        if (Lr > ld) ld = Lr;
      }
      std::vector<int32_t> r2t((size_t)(B * ld)), pl((size_t)B), sl((size_t)B), qo((size_t)B + 1),
          ns(flat.size());
      std::vector<int64_t> nodes((size_t)B);
      // the schedule's reusable prefixes are what prepare then matches
      std::vector<int32_t> order((size_t)B);
      std::vector<int64_t> reuse((size_t)B);
      CHECK(rkv_schedule(t, B, flat.data(), indptr.data(), order.data(), reuse.data()) == RKV_OK);
      const int rc = rkv_batch_prepare(t, B, flat.data(), indptr.data(), r2t.data(), ld, pl.data(), sl.data(),
                                       qo.data(), ns.data(), (int64_t)flat.size(), nodes.data());
      CHECK(rc == RKV_OK || rc == RKV_EBUSY);
      if (rc == RKV_OK) {
        for (int r = 0; r < B; ++r) CHECK(pl[(size_t)r] < sl[(size_t)r] && pl[(size_t)r] == reuse[(size_t)r]);
        CHECK(rkv_batch_commit(t, B, flat.data(), indptr.data(), r2t.data(), ld, nodes.data()) == RKV_OK);
      }
    }
    verify(t, P, held);
  }
  // bad arguments never change state
  CHECK(rkv_radix_unlock(t, 1 << 30) == RKV_EINVAL);
  CHECK(rkv_free(t, nullptr, 1) == RKV_EINVAL);
  verify(t, P, held);
  rkv_tree_destroy(t);
  std::printf("fuzz ok seed=%llu ops=%d\n", (unsigned long long)seed, ops);
  return 0;
}
