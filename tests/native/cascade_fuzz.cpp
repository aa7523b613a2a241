// Seeded random tables through rkv_cascade_plan, built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every plan is checked against what its
// definition fixes:
//   - perm is a permutation; rec_indptr is non-decreasing from 0;
//   - every job's members share slots over the job's keys, none of them up to
//     its own query key, with at most max_members members and seg_chunk keys;
//   - every request's keys 0 .. L-1 are covered exactly once by its jobs and
//     its tail; its shared records are exactly 0 .. n - ntail - 1;
//   - with min_keys = 1 and unbounded chunks and groups, the keys read are the
//     distinct prefixes of the truncated rows (an explicit trie) plus one
//     query key per request;
//   - a too-small capacity gives RKV_ENOSPC with the size and no other write,
//     and bad arguments give RKV_EINVAL.
// Usage: cascade_fuzz <seed> <rounds>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "rkv.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);       \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

struct Table {
  int32_t B = 0;
  int64_t ld = 1;
  std::vector<int32_t> r2t, L;
};

static Table make_table(std::mt19937_64& g) {
  Table t;
  t.B = (int32_t)(g() % 40);
  std::vector<std::vector<int32_t>> rows;
  int32_t fresh = 7;
  for (int32_t i = 0; i < t.B; ++i) {
    std::vector<int32_t> row;
    const unsigned pick = (unsigned)(g() % 10);
    if (!rows.empty() && pick == 0) {
      row = rows[g() % rows.size()];
    } else if (!rows.empty() && pick < 8) {
      const auto& base = rows[g() % rows.size()];
      row.assign(base.begin(), base.begin() + (long)(g() % (base.size() + 1)));
      const int add = (int)(g() % 40) + (row.empty() ? 1 : 0);
      for (int k = 0; k < add; ++k) row.push_back(fresh++);
    } else {
      const int n = 1 + (int)(g() % 90);
      for (int k = 0; k < n; ++k) row.push_back(fresh++);
    }
    rows.push_back(row);
  }
  for (auto& r : rows) t.ld = std::max<int64_t>(t.ld, (int64_t)r.size() + (int64_t)(g() % 3));
  t.r2t.assign((size_t)t.B * t.ld, -1);
  for (int32_t i = 0; i < t.B; ++i) {
    for (size_t k = 0; k < rows[i].size(); ++k) t.r2t[(size_t)i * t.ld + k] = rows[i][k];
    t.L.push_back((int32_t)rows[i].size());
  }
  return t;
}

static int64_t distinct_prefixes(const Table& t) {
  std::vector<std::map<int32_t, int32_t>> trie(1);
  for (int32_t r = 0; r < t.B; ++r) {
    int32_t node = 0;
    for (int32_t k = 0; k + 1 < t.L[r]; ++k) {
      const int32_t s = t.r2t[(size_t)r * t.ld + k];
      auto it = trie[node].find(s);
      if (it == trie[node].end()) {
        trie.emplace_back();
        const int32_t nn = (int32_t)trie.size() - 1;
        trie[node][s] = nn;
        node = nn;
      } else {
        node = it->second;
      }
    }
  }
  return (int64_t)trie.size() - 1;
}

static void check_plan(const Table& t, int32_t sc, int32_t tc, int32_t mk, int32_t mm, const std::vector<int32_t>& perm,
                       const std::vector<int32_t>& rec, const std::vector<int32_t>& tb, const std::vector<int32_t>& jobs,
                       int64_t n_jobs, int32_t tail_splits) {
  const int32_t B = t.B;
  std::vector<int32_t> seen(B, 0);
  for (int32_t i = 0; i < B; ++i) {
    CHECK(perm[i] >= 0 && perm[i] < B);
    CHECK(!seen[perm[i]]);
    seen[perm[i]] = 1;
  }
  CHECK(rec[0] == 0);
  for (int32_t r = 0; r < B; ++r) CHECK(rec[r + 1] >= rec[r] + 1);
  std::vector<std::vector<int32_t>> cover(B);
  std::vector<std::set<int32_t>> recs(B);
  for (int32_t r = 0; r < B; ++r) cover[r].assign(t.L[r], 0);
  for (int64_t j = 0; j < n_jobs; ++j) {
    const int32_t kb = jobs[5 * j], ke = jobs[5 * j + 1], first = jobs[5 * j + 2], count = jobs[5 * j + 3],
                  ro = jobs[5 * j + 4];
    CHECK(0 <= kb && kb < ke && ke - kb <= sc);
    CHECK(1 <= count && count <= mm && first >= 0 && first + count <= B);
    const int32_t rep = perm[first];
    for (int32_t m = first; m < first + count; ++m) {
      const int32_t r = perm[m];
      CHECK(ke <= t.L[r] - 1);
      for (int32_t k = kb; k < ke; ++k) {
        CHECK(t.r2t[(size_t)r * t.ld + k] == t.r2t[(size_t)rep * t.ld + k]);
        cover[r][k] += 1;
      }
      CHECK(recs[r].insert(ro).second);
    }
  }
  int32_t max_tail = 0;
  for (int32_t r = 0; r < B; ++r) {
    CHECK(tb[r] >= 0 && tb[r] <= t.L[r] - 1);
    const int32_t nt = (t.L[r] - tb[r] + tc - 1) / tc;
    max_tail = std::max(max_tail, nt);
    const int32_t n = rec[r + 1] - rec[r];
    CHECK(n >= nt);
    CHECK((int32_t)recs[r].size() == n - nt);
    int32_t want = 0;
    for (int32_t x : recs[r]) CHECK(x == want++);
    for (int32_t k = tb[r]; k < t.L[r]; ++k) cover[r][k] += 1;
    for (int32_t k = 0; k < t.L[r]; ++k) CHECK(cover[r][k] == 1);
    if (mk > 1) CHECK(tb[r] == 0 || tb[r] >= mk);
  }
  CHECK(tail_splits == max_tail);
  if (mk == 1 && sc >= (int32_t)t.ld && mm >= B) {
    int64_t keys = 0;
    for (int64_t j = 0; j < n_jobs; ++j) keys += jobs[5 * j + 1] - jobs[5 * j];
    for (int32_t r = 0; r < B; ++r) keys += t.L[r] - tb[r];
    CHECK(keys == distinct_prefixes(t) + B);
  }
}

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 500;
  std::mt19937_64 g(seed);
  for (int it = 0; it < rounds; ++it) {
    const Table t = make_table(g);
    const int32_t B = t.B;
    int32_t sc, tc, mk, mm;
    if (it % 3 == 0) {
      sc = (int32_t)t.ld + 1; tc = 1 + (int32_t)(g() % 100); mk = 1; mm = B + 1;
    } else {
      sc = 1 + (int32_t)(g() % 50); tc = 1 + (int32_t)(g() % 50); mk = 1 + (int32_t)(g() % 12);
      mm = 1 + (int32_t)(g() % 8);
    }
    std::vector<int32_t> perm(B + 1, -7), rec(B + 1, -7), tb(B + 1, -7);
    int64_t n_jobs = -1;
    int32_t ts = -1;
    // sizing: capacity 0 -> ENOSPC (when there are jobs) and nothing written
    const int rc0 = rkv_cascade_plan(B ? t.r2t.data() : nullptr, t.ld, B ? t.L.data() : nullptr, B, sc, tc, mk, mm,
                                     perm.data(), rec.data(), tb.data(), nullptr, 0, &n_jobs, &ts);
    CHECK(rc0 == RKV_OK || rc0 == RKV_ENOSPC);
    if (rc0 == RKV_ENOSPC) {
      CHECK(n_jobs > 0 && rec[0] == -7 && perm[0] == -7 && ts == -1);
    } else {
      CHECK(n_jobs == 0);
    }
    std::vector<int32_t> jobs((size_t)std::max<int64_t>(n_jobs, 1) * 5, -7);
    const int rc = rkv_cascade_plan(B ? t.r2t.data() : nullptr, t.ld, B ? t.L.data() : nullptr, B, sc, tc, mk, mm,
                                    perm.data(), rec.data(), tb.data(), jobs.data(), n_jobs, &n_jobs, &ts);
    CHECK(rc == RKV_OK);
    check_plan(t, sc, tc, mk, mm, perm, rec, tb, jobs, n_jobs, ts);
    // bad arguments
    if (B > 0) {
      std::vector<int32_t> badL = t.L;
      badL[g() % B] = (g() & 1) ? 0 : (int32_t)t.ld + 1;
      CHECK(rkv_cascade_plan(t.r2t.data(), t.ld, badL.data(), B, sc, tc, mk, mm, perm.data(), rec.data(), tb.data(),
                             jobs.data(), n_jobs, &n_jobs, &ts) == RKV_EINVAL);
    }
    CHECK(rkv_cascade_plan(t.r2t.data(), t.ld, t.L.data(), B, 0, tc, mk, mm, perm.data(), rec.data(), tb.data(),
                           jobs.data(), n_jobs, &n_jobs, &ts) == RKV_EINVAL);
  }
  std::printf("fuzz ok: %d tables\n", rounds);
  return 0;
}
