// Host radix tree over token sequences + FIFO token-slot allocator.
//
// RadixAttention keeps the KV cache as an LRU cache inside a radix tree and
// uses the tree for matching, insertion and eviction (unite.ai, "SGLang:
// Efficient Execution of Structured Language Model Programs", section
// "Introduccion a SGLang", RadixAttention bullet).  Edges carry token
// sequences; a new prompt reuses the KV of its longest cached prefix (Step 3
// of the walkthrough in section "SGLang: Modelo de programacion y
// metodologia"); nodes are split so sequences share their common part (Steps
// 4 and 7); whole least-recently-used nodes are evicted under a memory limit
// (Steps 5, 8 and 9).  The exact observable rules (tick, split ids, duplicate
// slots, eviction order, FIFO order) are spelled out in include/rkv.h.
//
// Data structures, chosen for the host hot loop (match/insert are O(length)
// token compares plus O(depth) child lookups):
//   - children: a flat vector of (first token, node) pairs kept sorted, found
//     by binary search; sorted order is also the canonical dump order;
//   - LRU candidates: an ordered set of (last_access, id) holding exactly the
//     non-root leaves with lock 0, so eviction pops its minimum;
//   - FIFO: a ring buffer of pool_slots int32 entries;
//   - owner: one byte per slot (free, held by the caller, in the tree), so
//     insert, commit and free can reject a slot the caller does not hold
//     before they change anything (a foreign slot pushed to the FIFO would
//     otherwise overrun the ring or hand one slot out twice).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <set>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "rkv.h"
#include "rkv_internal.h"

namespace {

// Length of the common prefix of a[0..n) and b[0..n), from position `from`
// on (the first `from` entries are known equal): 64-byte blocks by memcmp,
// then element by element inside the first block that differs.
inline int64_t common_from(const int32_t* a, const int32_t* b, int64_t from, int64_t n) {
  int64_t k = from;
  while (k + 16 <= n && std::memcmp(a + k, b + k, 64) == 0) k += 16;
  while (k < n && a[k] == b[k]) ++k;
  return k;
}

struct Node {
  int64_t id = 0;
  std::vector<int32_t> label;
  std::vector<int32_t> slots;
  Node* parent = nullptr;
  std::vector<std::pair<int32_t, Node*>> kids;  // sorted by first token
  int64_t last_access = 0;
  int64_t lock = 0;
  bool in_lru = false;
};

}  // namespace

struct rkv_tree {
  int64_t pool = 0;
  // FIFO ring
  std::vector<int32_t> ring;
  int64_t head = 0, count = 0;
  // who holds each slot; kPending marks a caller slot already seen while a
  // call checks its arguments (a repeat is then caught) and is undone before
  // the call returns
  enum : uint8_t { kFree = 0, kCaller = 1, kTree = 2, kPending = 3 };
  std::vector<uint8_t> owner;
  // tree
  Node root;
  std::unordered_map<int64_t, std::unique_ptr<Node>> nodes;  // non-root nodes by id
  std::set<std::pair<int64_t, int64_t>> lru;                   // (last_access, id)
  int64_t next_id = 1;
  int64_t tick = 0;
  // stats
  int64_t cached = 0, locked_tokens = 0, matched_total = 0, prompt_total = 0, evicted_total = 0;
  // scratch
  std::vector<Node*> path;

  // ---------------------------------------------------------------- FIFO
  void push(int32_t s) {
    int64_t i = head + count;
    if (i >= pool) i -= pool;
    ring[i] = s;
    owner[(size_t)s] = kFree;
    ++count;
  }
  // pops n slots (n <= count) in FIFO order into each of the non-null
  // outputs: one or two contiguous runs of the ring
  void pop_n(int64_t n, int32_t* out_a, int32_t* out_b) {
    while (n > 0) {
      const int64_t run = std::min<int64_t>(n, pool - head);
      for (int64_t i = 0; i < run; ++i) owner[(size_t)ring[(size_t)(head + i)]] = kCaller;
      if (out_a) std::memcpy(out_a, ring.data() + head, sizeof(int32_t) * (size_t)run);
      if (out_b) std::memcpy(out_b, ring.data() + head, sizeof(int32_t) * (size_t)run);
      if (out_a) out_a += run;
      if (out_b) out_b += run;
      head += run;
      if (head == pool) head = 0;
      count -= run;
      n -= run;
    }
  }

  // ---------------------------------------------------------------- LRU set
  bool candidate(const Node* n) const { return n != &root && n->kids.empty() && n->lock == 0; }
  void lru_refresh(Node* n) {
    bool want = candidate(n);
    if (n->in_lru && !want) {
      lru.erase({n->last_access, n->id});
      n->in_lru = false;
    } else if (!n->in_lru && want) {
      lru.insert({n->last_access, n->id});
      n->in_lru = true;
    }
  }
  void touch(Node* n, int64_t t) {
    if (n->in_lru) {
      lru.erase({n->last_access, n->id});
      n->last_access = t;
      lru.insert({n->last_access, n->id});
    } else {
      n->last_access = t;
    }
  }

  // ---------------------------------------------------------------- children
  static std::vector<std::pair<int32_t, Node*>>::iterator find_kid(Node* n, int32_t tok) {
    auto it = std::lower_bound(n->kids.begin(), n->kids.end(), tok,
                               [](const std::pair<int32_t, Node*>& a, int32_t b) { return a.first < b; });
    return it;
  }
  Node* child(Node* n, int32_t tok) {
    auto it = find_kid(n, tok);
    return (it != n->kids.end() && it->first == tok) ? it->second : nullptr;
  }
  void add_kid(Node* n, Node* c) {
    bool was_leaf = n->kids.empty();
    auto it = find_kid(n, c->label[0]);
    n->kids.insert(it, {c->label[0], c});
    if (was_leaf) lru_refresh(n);
  }
  void remove_kid(Node* n, Node* c) {
    auto it = find_kid(n, c->label[0]);
    n->kids.erase(it);
    if (n->kids.empty()) lru_refresh(n);
  }

  Node* make_node() {
    auto up = std::make_unique<Node>();
    up->id = next_id++;
    Node* raw = up.get();
    nodes.emplace(raw->id, std::move(up));
    return raw;
  }

  // Cut x's edge after k tokens; the new upper node takes x's place.
  Node* split(Node* x, int64_t k) {
    Node* up = make_node();
    Node* parent = x->parent;
    up->label.assign(x->label.begin(), x->label.begin() + k);
    up->slots.assign(x->slots.begin(), x->slots.begin() + k);
    up->parent = parent;
    up->last_access = x->last_access;
    up->lock = x->lock;
    auto it = find_kid(parent, x->label[0]);
    it->second = up;  // same first token, same position
    x->label.erase(x->label.begin(), x->label.begin() + k);
    x->slots.erase(x->slots.begin(), x->slots.begin() + k);
    x->parent = up;
    up->kids.push_back({x->label[0], x});
    // up is not a leaf; x keeps its leaf status, so the LRU set is unchanged
    return up;
  }

  // Descend along tok, splitting where it ends or diverges inside an edge.
  // Fills `path` (root first) and appends matched slots to *slots if given.
  Node* walk(const int32_t* tok, int64_t n, int64_t* matched, int32_t* slots) {
    path.clear();
    path.push_back(&root);
    Node* node = &root;
    int64_t m = 0;
    while (m < n) {
      Node* c = child(node, tok[m]);
      if (!c) break;
      const int64_t lab = (int64_t)c->label.size();
      const int64_t lim = std::min<int64_t>(lab, n - m);
      const int64_t k = common_from(c->label.data(), tok + m, 1, lim);
      if (k < lab) c = split(c, k);
      if (slots) std::memcpy(slots + m, c->slots.data(), sizeof(int32_t) * (size_t)k);
      m += k;
      node = c;
      path.push_back(c);
    }
    *matched = m;
    return node;
  }

  // Length of the longest cached prefix of tok[0..n), with no side effect:
  // no split, no tick, no lock (the walk stops inside an edge instead of
  // cutting it).
  int64_t peek(const int32_t* tok, int64_t n) const {
    const Node* node = &root;
    int64_t m = 0;
    while (m < n) {
      auto it = std::lower_bound(node->kids.begin(), node->kids.end(), tok[m],
                                 [](const std::pair<int32_t, Node*>& a, int32_t b) { return a.first < b; });
      if (it == node->kids.end() || it->first != tok[m]) break;
      const Node* c = it->second;
      const int64_t lab = (int64_t)c->label.size();
      const int64_t lim = std::min<int64_t>(lab, n - m);
      const int64_t k = common_from(c->label.data(), tok + m, 1, lim);
      m += k;
      if (k < lab) break;
      node = c;
    }
    return m;
  }

  // peek that also copies the cached slots of the matched positions
  int64_t peek_slots(const int32_t* tok, int64_t n, int32_t* slots) const {
    const Node* node = &root;
    int64_t m = 0;
    while (m < n) {
      auto it = std::lower_bound(node->kids.begin(), node->kids.end(), tok[m],
                                 [](const std::pair<int32_t, Node*>& a, int32_t b) { return a.first < b; });
      if (it == node->kids.end() || it->first != tok[m]) break;
      const Node* c = it->second;
      const int64_t lab = (int64_t)c->label.size();
      const int64_t lim = std::min<int64_t>(lab, n - m);
      const int64_t k = common_from(c->label.data(), tok + m, 1, lim);
      std::memcpy(slots + m, c->slots.data(), sizeof(int32_t) * (size_t)k);
      m += k;
      if (k < lab) break;
      node = c;
    }
    return m;
  }

  // Argument check of an insert of tok[0..n) with slots sl[0..n), read-only
  // on the tree: every position either holds the tree's own slot for it or a
  // slot the caller holds, and no caller slot appears twice (across all the
  // calls made before the matching unmark_pending()).  Such an insert only
  // pushes caller slots, each once, so the FIFO never exceeds the pool.  The
  // same holds when earlier inserts of one batch grow the matched part: the
  // extra positions then hold caller slots that are pushed.
  bool owned_ok(const int32_t* tok, const int32_t* sl, int64_t n) {
    tmp_slots.resize((size_t)std::max<int64_t>(n, 1));
    const int64_t m = peek_slots(tok, n, tmp_slots.data());
    for (int64_t i = 0; i < n; ++i) {
      if (i < m && sl[i] == tmp_slots[(size_t)i]) continue;
      uint8_t& o = owner[(size_t)sl[i]];
      if (o != kCaller) return false;
      o = kPending;
      pending.push_back(sl[i]);
    }
    return true;
  }
  void unmark_pending() {
    for (int32_t s : pending) owner[(size_t)s] = kCaller;
    pending.clear();
  }
  std::vector<int32_t> pending;

  int64_t do_match(const int32_t* tok, int64_t n, int32_t* slots, int64_t* node_id) {
    ++tick;
    int64_t m = 0;
    Node* stop = walk(tok, n, &m, slots);
    for (Node* p : path) touch(p, tick);
    *node_id = (m > 0) ? stop->id : 0;
    return m;
  }

  void lock_path(Node* n, int64_t delta) {
    for (Node* p = n; p != &root; p = p->parent) {
      const int64_t before = p->lock;
      p->lock += delta;
      if (before == 0 && p->lock > 0) locked_tokens += (int64_t)p->label.size();
      if (before > 0 && p->lock == 0) locked_tokens -= (int64_t)p->label.size();
      lru_refresh(p);
    }
  }

  Node* find(int64_t id) {
    if (id == 0) return &root;
    auto it = nodes.find(id);
    return it == nodes.end() ? nullptr : it->second.get();
  }

  int64_t do_insert(const int32_t* tok, const int32_t* sl, int64_t n) {
    ++tick;
    int64_t m = 0;
    tmp_slots.resize((size_t)std::max<int64_t>(n, 1));
    Node* stop = walk(tok, n, &m, tmp_slots.data());
    for (int64_t i = 0; i < m; ++i)
      if (sl[i] != tmp_slots[(size_t)i]) push(sl[i]);
    if (m < n) {
      Node* leaf = make_node();
      leaf->label.assign(tok + m, tok + n);
      leaf->slots.assign(sl + m, sl + n);
      for (int64_t i = m; i < n; ++i) owner[(size_t)sl[i]] = kTree;
      leaf->parent = stop;
      leaf->last_access = tick;
      add_kid(stop, leaf);
      cached += n - m;
      lru_refresh(leaf);
    }
    for (Node* p : path) touch(p, tick);
    return m;
  }
  std::vector<int32_t> tmp_slots;

  int do_evict(int64_t want, int64_t* freed_out) {
    int64_t freed = 0;
    while (freed < want) {
      if (lru.empty()) {
        *freed_out = freed;
        return RKV_EBUSY;
      }
      auto it = lru.begin();
      Node* v = find(it->second);
      lru.erase(it);
      v->in_lru = false;
      for (int32_t s : v->slots) push(s);
      const int64_t len = (int64_t)v->slots.size();
      freed += len;
      evicted_total += len;
      cached -= len;
      Node* parent = v->parent;
      remove_kid(parent, v);
      nodes.erase(v->id);
    }
    *freed_out = freed;
    return RKV_OK;
  }

  void dump(Node* n, std::vector<int64_t>& out) const {
    out.push_back(n->id);
    out.push_back(n->parent ? n->parent->id : -1);
    out.push_back(n->last_access);
    out.push_back(n->lock);
    out.push_back((int64_t)n->label.size());
    for (int32_t x : n->label) out.push_back(x);
    for (int32_t x : n->slots) out.push_back(x);
    for (auto& kv : n->kids) dump(kv.second, out);
  }
};

namespace {

int bad(const std::string& msg) { return rkv::fail(RKV_EINVAL, msg); }

bool slot_ok(const rkv_tree* t, int32_t s) { return s >= 0 && (int64_t)s < t->pool; }

}  // namespace

extern "C" {

int rkv_tree_create(rkv_tree** out, int64_t pool_slots, const int32_t* initial_free) {
  rkv::clear_error();
  if (!out) return bad("rkv_tree_create: out is NULL");
  *out = nullptr;
  if (pool_slots < 1 || pool_slots > INT32_MAX) return bad("rkv_tree_create: pool_slots out of range");
  rkv_tree* t = new (std::nothrow) rkv_tree();
  if (!t) return rkv::fail(RKV_ENOSPC, "rkv_tree_create: out of host memory");
  try {
    t->pool = pool_slots;
    t->ring.resize((size_t)pool_slots);
    t->owner.assign((size_t)pool_slots, rkv_tree::kFree);
    if (initial_free) {
      std::vector<uint8_t> seen((size_t)pool_slots, 0);
      for (int64_t i = 0; i < pool_slots; ++i) {
        const int32_t s = initial_free[i];
        if (!slot_ok(t, s) || seen[(size_t)s]) {
          delete t;
          return bad("rkv_tree_create: initial_free is not a permutation of [0, pool_slots)");
        }
        seen[(size_t)s] = 1;
        t->ring[(size_t)i] = s;
      }
    } else {
      for (int64_t i = 0; i < pool_slots; ++i) t->ring[(size_t)i] = (int32_t)i;
    }
    t->count = pool_slots;
  } catch (const std::bad_alloc&) {
    delete t;
    return rkv::fail(RKV_ENOSPC, "rkv_tree_create: out of host memory");
  }
  *out = t;
  return RKV_OK;
}

void rkv_tree_destroy(rkv_tree* t) { delete t; }

int rkv_radix_match(rkv_tree* t, const int32_t* tok, int64_t n, int32_t* out_slots,
                    int64_t* out_len, int64_t* out_node) {
  rkv::clear_error();
  if (!t || !out_len || !out_node || n < 0 || (n > 0 && (!tok || !out_slots)))
    return bad("rkv_radix_match: bad argument");
  *out_len = t->do_match(tok, n, out_slots, out_node);
  return RKV_OK;
}

int rkv_radix_peek(const rkv_tree* t, const int32_t* tok, int64_t n, int64_t* out_len) {
  rkv::clear_error();
  if (!t || !out_len || n < 0 || (n > 0 && !tok)) return bad("rkv_radix_peek: bad argument");
  *out_len = t->peek(tok, n);
  return RKV_OK;
}

int rkv_schedule(const rkv_tree* t, int32_t Q, const int32_t* tok, const int64_t* tok_indptr,
                 int32_t* order, int64_t* matched) {
  rkv::clear_error();
  if (!t || Q < 0) return bad("rkv_schedule: bad argument");
  if (Q == 0) return RKV_OK;
  if (!tok_indptr || !order || !matched) return bad("rkv_schedule: NULL pointer");
  for (int32_t q = 0; q < Q; ++q) {
    const int64_t L = tok_indptr[q + 1] - tok_indptr[q];
    if (L < 0 || tok_indptr[q] < 0) return bad("rkv_schedule: tok_indptr must be non-decreasing from 0");
    if (L > 0 && !tok) return bad("rkv_schedule: tok is NULL");
    // the cached part a batch would reuse: prepare caps the match at L - 1
    matched[q] = L > 0 ? t->peek(tok + tok_indptr[q], L - 1) : 0;
    order[q] = q;
  }
  std::stable_sort(order, order + Q, [&](int32_t x, int32_t y) { return matched[x] > matched[y]; });
  return RKV_OK;
}

int rkv_radix_lock(rkv_tree* t, int64_t node) {
  rkv::clear_error();
  if (!t) return bad("rkv_radix_lock: tree is NULL");
  Node* n = t->find(node);
  if (!n) return bad("rkv_radix_lock: no such node");
  t->lock_path(n, +1);
  return RKV_OK;
}

int rkv_radix_unlock(rkv_tree* t, int64_t node) {
  rkv::clear_error();
  if (!t) return bad("rkv_radix_unlock: tree is NULL");
  Node* n = t->find(node);
  if (!n) return bad("rkv_radix_unlock: no such node");
  for (Node* p = n; p != &t->root; p = p->parent)
    if (p->lock <= 0) return bad("rkv_radix_unlock: lock count would go negative");
  t->lock_path(n, -1);
  return RKV_OK;
}

int rkv_radix_insert(rkv_tree* t, const int32_t* tok, const int32_t* slots, int64_t n,
                     int64_t* out_cached) {
  rkv::clear_error();
  if (!t || !out_cached || n < 0 || (n > 0 && (!tok || !slots)))
    return bad("rkv_radix_insert: bad argument");
  for (int64_t i = 0; i < n; ++i)
    if (!slot_ok(t, slots[i])) return bad("rkv_radix_insert: slot out of range");
  const bool ok = t->owned_ok(tok, slots, n);
  t->unmark_pending();
  if (!ok) return bad("rkv_radix_insert: a slot is neither the tree's own for its position nor held by the caller, or it repeats");
  *out_cached = t->do_insert(tok, slots, n);
  return RKV_OK;
}

int rkv_radix_evict(rkv_tree* t, int64_t want, int64_t* out_freed) {
  rkv::clear_error();
  if (!t || !out_freed || want < 0) return bad("rkv_radix_evict: bad argument");
  int rc = t->do_evict(want, out_freed);
  if (rc == RKV_EBUSY) rkv::fail(RKV_EBUSY, "rkv_radix_evict: every remaining leaf is locked");
  return rc;
}

int rkv_alloc(rkv_tree* t, int64_t n, int32_t* out) {
  rkv::clear_error();
  if (!t || n < 0 || (n > 0 && !out)) return bad("rkv_alloc: bad argument");
  if (t->count < n) return rkv::fail(RKV_ENOSPC, "rkv_alloc: not enough free slots");
  t->pop_n(n, out, nullptr);
  return RKV_OK;
}

int rkv_free(rkv_tree* t, const int32_t* slots, int64_t n) {
  rkv::clear_error();
  if (!t || n < 0 || (n > 0 && !slots)) return bad("rkv_free: bad argument");
  if (t->count + n > t->pool) return bad("rkv_free: more slots than the pool holds");
  for (int64_t i = 0; i < n; ++i)
    if (!slot_ok(t, slots[i])) return bad("rkv_free: slot out of range");
  bool held = true;
  for (int64_t i = 0; i < n && held; ++i) {
    uint8_t& o = t->owner[(size_t)slots[i]];
    if (o != rkv_tree::kCaller) held = false;
    else {
      o = rkv_tree::kPending;
      t->pending.push_back(slots[i]);
    }
  }
  t->unmark_pending();
  if (!held) return bad("rkv_free: a slot is not held by the caller, or it repeats");
  for (int64_t i = 0; i < n; ++i) t->push(slots[i]);
  return RKV_OK;
}

int rkv_stats(rkv_tree* t, int64_t out[8]) {
  rkv::clear_error();
  if (!t || !out) return bad("rkv_stats: bad argument");
  out[0] = t->cached;
  out[1] = t->count;
  out[2] = t->cached - t->locked_tokens;
  out[3] = t->locked_tokens;
  out[4] = (int64_t)t->nodes.size();
  out[5] = t->matched_total;
  out[6] = t->prompt_total;
  out[7] = t->evicted_total;
  return RKV_OK;
}

int rkv_radix_serialize(rkv_tree* t, int64_t* buf, int64_t cap, int64_t* len) {
  rkv::clear_error();
  if (!t || !len || cap < 0 || (cap > 0 && !buf)) return bad("rkv_radix_serialize: bad argument");
  std::vector<int64_t> out;
  t->dump(&t->root, out);
  *len = (int64_t)out.size();
  const int64_t w = std::min<int64_t>(cap, (int64_t)out.size());
  if (w > 0) std::memcpy(buf, out.data(), sizeof(int64_t) * (size_t)w);
  return RKV_OK;
}

int rkv_free_list(rkv_tree* t, int32_t* buf, int64_t cap, int64_t* len) {
  rkv::clear_error();
  if (!t || !len || cap < 0 || (cap > 0 && !buf)) return bad("rkv_free_list: bad argument");
  *len = t->count;
  const int64_t w = std::min<int64_t>(cap, t->count);
  for (int64_t i = 0; i < w; ++i) buf[i] = t->ring[(size_t)((t->head + i) % t->pool)];
  return RKV_OK;
}

int rkv_batch_prepare(rkv_tree* t, int32_t B, const int32_t* tok, const int64_t* tok_indptr,
                      int32_t* req_to_token, int64_t ld, int32_t* prefix_lens, int32_t* seq_lens,
                      int32_t* qo_indptr, int32_t* new_slots, int64_t new_cap,
                      int64_t* out_nodes) {
  rkv::clear_error();
  if (!t || B < 0) return bad("rkv_batch_prepare: bad argument");
  if (B == 0) {
    if (qo_indptr) qo_indptr[0] = 0;
    return RKV_OK;
  }
  if (!tok || !tok_indptr || !req_to_token || !prefix_lens || !seq_lens || !qo_indptr ||
      !out_nodes || ld < 1 || new_cap < 0)
    return bad("rkv_batch_prepare: bad argument");
  int64_t total_len = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
    if (tok_indptr[r] < 0 || L < 1 || L > ld || L > INT32_MAX)
      return bad("rkv_batch_prepare: every length must be in [1, ld]");
    total_len += L;
  }
  if (new_cap < total_len) return bad("rkv_batch_prepare: new_cap must be >= the sum of lengths");

  for (int32_t r = 0; r < B; ++r) {
    const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
    int32_t* row = req_to_token + (int64_t)r * ld;
    int64_t node = 0;
    const int64_t p = t->do_match(tok + tok_indptr[r], L - 1, row, &node);
    prefix_lens[r] = (int32_t)p;
    seq_lens[r] = (int32_t)L;
    out_nodes[r] = node;
    t->lock_path(t->find(node), +1);
  }
  int64_t T = 0;
  qo_indptr[0] = 0;
  for (int32_t r = 0; r < B; ++r) {
    T += (int64_t)seq_lens[r] - prefix_lens[r];
    qo_indptr[r + 1] = (int32_t)T;
  }
  if (t->count < T) {
    int64_t freed = 0;
    if (t->do_evict(T - t->count, &freed) != RKV_OK) {
      for (int32_t r = 0; r < B; ++r) t->lock_path(t->find(out_nodes[r]), -1);
      return rkv::fail(RKV_EBUSY, "rkv_batch_prepare: eviction cannot free enough slots");
    }
  }
  int64_t pos = 0;
  for (int32_t r = 0; r < B; ++r) {
    int32_t* row = req_to_token + (int64_t)r * ld;
    const int64_t n = (int64_t)seq_lens[r] - prefix_lens[r];
    t->pop_n(n, row + prefix_lens[r], new_slots + pos);
    pos += n;
    std::fill(row + seq_lens[r], row + ld, -1);
    t->matched_total += prefix_lens[r];
    t->prompt_total += seq_lens[r];
  }
  return RKV_OK;
}

int rkv_batch_commit(rkv_tree* t, int32_t B, const int32_t* tok, const int64_t* tok_indptr,
                     const int32_t* req_to_token, int64_t ld, const int64_t* nodes) {
  rkv::clear_error();
  if (!t || B < 0) return bad("rkv_batch_commit: bad argument");
  if (B == 0) return RKV_OK;
  if (!tok || !tok_indptr || !req_to_token || !nodes || ld < 1)
    return bad("rkv_batch_commit: bad argument");
  // every check comes before the first insert, so EINVAL changes nothing
  std::unordered_map<Node*, int64_t> unlocks;   // node -> unlocks this batch makes on it
  for (int32_t r = 0; r < B; ++r) {
    const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
    if (tok_indptr[r] < 0 || L < 1 || L > ld) return bad("rkv_batch_commit: every length must be in [1, ld]");
    const int32_t* row = req_to_token + (int64_t)r * ld;
    for (int64_t i = 0; i < L; ++i)
      if (!slot_ok(t, row[i])) return bad("rkv_batch_commit: slot out of range");
    Node* n = t->find(nodes[r]);
    if (!n) return bad("rkv_batch_commit: no such node");
    for (Node* p = n; p != &t->root; p = p->parent) ++unlocks[p];
  }
  // a split during the inserts gives the new upper node the lower one's
  // lock count, which covers the unlocks still to come through it
  for (const auto& kv : unlocks)
    if (kv.first->lock < kv.second) return bad("rkv_batch_commit: node is not locked");
  bool ok = true;
  for (int32_t r = 0; r < B && ok; ++r) {
    const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
    ok = t->owned_ok(tok + tok_indptr[r], req_to_token + (int64_t)r * ld, L);
  }
  t->unmark_pending();
  if (!ok)
    return bad("rkv_batch_commit: a slot is neither the tree's own for its position nor held by the caller, "
               "or it repeats within the batch");
  for (int32_t r = 0; r < B; ++r) {
    const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
    t->do_insert(tok + tok_indptr[r], req_to_token + (int64_t)r * ld, L);
    t->lock_path(t->find(nodes[r]), -1);
  }
  return RKV_OK;
}

int rkv_batch_append(rkv_tree* t, int32_t B, int32_t* req_to_token, int64_t ld, int32_t* seq_lens,
                     int32_t* new_slots) {
  rkv::clear_error();
  if (!t || B < 0) return bad("rkv_batch_append: bad argument");
  if (B == 0) return RKV_OK;
  if (!req_to_token || !seq_lens || !new_slots || ld < 2) return bad("rkv_batch_append: bad argument");
  for (int32_t r = 0; r < B; ++r)
    if (seq_lens[r] < 1 || (int64_t)seq_lens[r] >= ld)
      return bad("rkv_batch_append: every length must be in [1, ld - 1]");
  if (t->count < B) {
    int64_t freed = 0;
    if (t->do_evict(B - t->count, &freed) != RKV_OK)
      return rkv::fail(RKV_EBUSY, "rkv_batch_append: eviction cannot free enough slots");
  }
  t->pop_n(B, new_slots, nullptr);
  for (int32_t r = 0; r < B; ++r) {
    req_to_token[(int64_t)r * ld + seq_lens[r]] = new_slots[r];
    ++seq_lens[r];
  }
  return RKV_OK;
}

}  // extern "C"
