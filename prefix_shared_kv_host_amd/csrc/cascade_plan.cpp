// Host planner for prefix-shared decode.
//
// RadixAttention stores a shared prompt prefix once in the KV pool, so every
// request under a radix node gathers the same slots for that node's keys
// (unite.ai, "SGLang: Efficient Execution of Structured Language Model
// Programs", section "Introduccion a SGLang", RadixAttention bullet).  A
// decode batch can therefore read each shared run of slots once for all of
// its requests and merge that partial softmax state with each request's
// private remainder.  The pages stop at reusing the cache; the cascade is an
// extension built on the split identity that decode already uses.
//
// The plan is derived from the index table alone (no tree needed): rows are
// truncated to L_r - 1 keys (the query's own key stays private) and sorted
// lexicographically; in that order the requests that share a prefix of
// length d form contiguous blocks, and the blocks nest into the prefix tree
// of the batch.  With lcp[i] = common prefix of sorted rows i-1 and i, the
// block [lo, hi] (hi > lo) shares exactly d = min(lcp[lo+1..hi]) keys and
// splits into children at every i with lcp[i] == d.  A depth-first walk over
// the blocks emits one segment per block whose new keys (counted from the
// last emitted ancestor) reach min_keys, cuts it into jobs, and gives every
// request its record list.

#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <string>
#include <vector>

#include "rkv.h"
#include "rkv_internal.h"

namespace {

// First position where a[0..n) and b[0..n) differ (n if none): 64-byte
// blocks by memcmp, then element by element inside the first differing block.
inline int32_t mismatch_at(const int32_t* a, const int32_t* b, int32_t n) {
  int32_t i = 0;
  while (i + 16 <= n && std::memcmp(a + i, b + i, 64) == 0) i += 16;
  while (i < n && a[i] == b[i]) ++i;
  return i;
}

struct Frame {
  int32_t lo, hi;        // block of sorted positions
  int32_t eff;           // end of the last emitted segment above
  int32_t rec;           // shared records of every member so far
};

}  // namespace

extern "C" int rkv_cascade_plan(const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens, int32_t B,
                                int32_t seg_chunk, int32_t tail_chunk, int32_t min_keys, int32_t max_members,
                                int32_t* perm, int32_t* rec_indptr, int32_t* tail_begin, int32_t* jobs,
                                int64_t jobs_cap, int64_t* out_n_jobs, int32_t* out_tail_splits) {
  rkv::clear_error();
  if (B < 0 || seg_chunk < 1 || tail_chunk < 1 || min_keys < 1 || max_members < 1 || jobs_cap < 0)
    return rkv::fail(RKV_EINVAL, "rkv_cascade_plan: bad sizes");
  if (!out_n_jobs || !out_tail_splits || !rec_indptr || (jobs_cap > 0 && !jobs))
    return rkv::fail(RKV_EINVAL, "rkv_cascade_plan: NULL pointer");
  if (B > 0 && (!req_to_token || !seq_lens || !perm || !tail_begin))
    return rkv::fail(RKV_EINVAL, "rkv_cascade_plan: NULL pointer");
  for (int32_t r = 0; r < B; ++r)
    if (seq_lens[r] < 1 || seq_lens[r] > ld)
      return rkv::fail(RKV_EINVAL, "rkv_cascade_plan: seq_lens[" + std::to_string(r) + "] outside [1, ld]");

  auto row = [&](int32_t r) { return req_to_token + (int64_t)r * ld; };
  auto len = [&](int32_t r) { return seq_lens[r] - 1; };

  std::vector<int32_t> order(B);
  for (int32_t r = 0; r < B; ++r) order[r] = r;
  // lexicographic order of the truncated rows as int32 sequences
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    const int32_t n = std::min(len(a), len(b));
    const int32_t i = mismatch_at(row(a), row(b), n);
    return i < n ? row(a)[i] < row(b)[i] : len(a) < len(b);
  });
  std::vector<int32_t> lcp(B > 0 ? B : 1, 0);
  for (int32_t i = 1; i < B; ++i) {
    const int32_t a = order[i - 1], b = order[i];
    const int32_t n = std::min(len(a), len(b));
    lcp[i] = mismatch_at(row(a), row(b), n);
  }

  std::vector<int32_t> job;                 // 5 values per job
  std::vector<int32_t> shared(B, 0), tail(B, 0);
  std::vector<Frame> stack;
  if (B > 0) stack.push_back({0, B - 1, 0, 0});
  std::vector<int32_t> cuts;
  while (!stack.empty()) {
    const Frame f = stack.back();
    stack.pop_back();
    if (f.lo == f.hi) {
      tail[order[f.lo]] = f.eff;
      shared[order[f.lo]] = f.rec;
      continue;
    }
    int32_t d = INT32_MAX;
    for (int32_t i = f.lo + 1; i <= f.hi; ++i) d = std::min(d, lcp[i]);
    int32_t eff = f.eff, rec = f.rec;
    if ((int64_t)d - f.eff >= min_keys) {
      const int32_t count = f.hi - f.lo + 1;
      const int32_t nch = (d - f.eff + seg_chunk - 1) / seg_chunk;
      for (int32_t c = 0; c < nch; ++c) {
        const int32_t b0 = f.eff + c * seg_chunk;
        const int32_t b1 = std::min(d, b0 + seg_chunk);
        for (int32_t g0 = 0; g0 < count; g0 += max_members)
          job.insert(job.end(), {b0, b1, f.lo + g0, std::min(max_members, count - g0), f.rec + c});
      }
      eff = d;
      rec = f.rec + nch;
    }
    // children: cut at every lcp == d; pushed last-first so the walk is a preorder
    cuts.clear();
    cuts.push_back(f.lo);
    for (int32_t i = f.lo + 1; i <= f.hi; ++i)
      if (lcp[i] == d) cuts.push_back(i);
    cuts.push_back(f.hi + 1);
    for (size_t k = cuts.size() - 1; k-- > 0;) stack.push_back({cuts[k], cuts[k + 1] - 1, eff, rec});
  }

  const int64_t n_jobs = (int64_t)job.size() / 5;
  *out_n_jobs = n_jobs;
  if (n_jobs > jobs_cap)
    return rkv::fail(RKV_ENOSPC, "rkv_cascade_plan: " + std::to_string(n_jobs) + " jobs, capacity " +
                                     std::to_string(jobs_cap));
  int64_t total = 0;
  int32_t max_tail = 0;
  rec_indptr[0] = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int32_t nt = (seq_lens[r] - tail[r] + tail_chunk - 1) / tail_chunk;
    max_tail = std::max(max_tail, nt);
    total += (int64_t)shared[r] + nt;
    if (total > INT32_MAX) return rkv::fail(RKV_EINVAL, "rkv_cascade_plan: more than 2^31-1 records");
  }
  total = 0;
  for (int32_t r = 0; r < B; ++r) {
    perm[r] = order[r];
    tail_begin[r] = tail[r];
    total += shared[r] + (seq_lens[r] - tail[r] + tail_chunk - 1) / tail_chunk;
    rec_indptr[r + 1] = (int32_t)total;
  }
  std::copy(job.begin(), job.end(), jobs);
  *out_tail_splits = max_tail;
  return RKV_OK;
}
