/*
 * rkv.h - C ABI of librkv: RadixAttention's prefix-shared KV cache on one
 * AMD MI355X (gfx950).
 *
 * What the library does.  Requests that share a prompt prefix read the same
 * cached K/V instead of recomputing it.  The KV cache is an LRU cache held in
 * a radix tree over token sequences, with matching, insertion and eviction as
 * its operations (unite.ai, "SGLang: Efficient Execution of Structured
 * Language Model Programs", section "Introduccion a SGLang", RadixAttention
 * bullet; the nine-step walkthrough in section "SGLang: Modelo de
 * programacion y metodologia").  The K/V rows live in one token-slot pool;
 * the tree hands out per-request index tables (req_to_token) that the GPU
 * kernels use to gather those rows.
 *
 * Two halves:
 *   host   - radix tree + FIFO slot allocator (C++; not thread-safe per
 *            handle: drive one tree from one scheduler thread);
 *   device - kv_scatter, attn_extend, attn_decode: hand-written HIP kernels
 *            for gfx950, asynchronous on the caller's stream.
 *
 * Conventions for every call:
 *   - Return value: RKV_OK (0) or a negative RKV_E* code.  No exception ever
 *     crosses the ABI.  rkv_last_error() gives a thread-local message for the
 *     last failure on the calling thread.
 *   - Arguments are checked before any state changes; a call that returns
 *     RKV_EINVAL has changed nothing (batch_prepare documents one exception).
 *   - Counts and lengths are int64_t unless noted; slot ids are int32_t in
 *     [0, pool_slots).
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RKV_OK = 0,
  RKV_EINVAL = -1,   /* bad argument (null, negative, out of range, shape)   */
  RKV_ENOSPC = -2,   /* not enough free slots                               */
  RKV_EBUSY = -3,    /* eviction ran out of unlocked leaves                 */
  RKV_EHIP = -4,     /* a HIP runtime call or kernel launch failed          */
  RKV_ENOTSUP = -5   /* valid but unsupported shape or dtype                */
};

enum { RKV_F32 = 0, RKV_BF16 = 1 };

typedef struct rkv_tree rkv_tree;

/* Message for the last failing call on this thread ("" if none).  The pointer
 * stays valid until the next rkv_* call on the same thread.  (Library
 * plumbing; it implements no passage of the pages.) */
const char* rkv_last_error(void);

/* Library version string, e.g. "rkv 0.1 gfx950".  (Library plumbing.) */
const char* rkv_version(void);

/* ------------------------------------------------------------------------
 * Host: radix tree + slot allocator.
 *
 * State (the "contract" both this library and its test oracle follow):
 *   node: id (root = 0, then a counter from 1 that never reuses ids), label
 *   (tokens of the edge into the node), slots (one per label token), parent,
 *   children keyed by first label token, last_access (tick), lock (count).
 *   A global tick is incremented once at the start of every match and every
 *   insert, and of nothing else.  The allocator is a FIFO of slot ids.
 *
 * Slot ownership.  Every slot is at any time in exactly one place: free (in
 * the FIFO), held by the caller (popped by rkv_alloc, rkv_batch_prepare or
 * rkv_batch_append and not yet inserted or freed), or in the tree.  The
 * library tracks this per slot (one byte each).  rkv_radix_insert,
 * rkv_batch_commit and rkv_free accept only slots the caller holds, or, for
 * an insert, the tree's own slot at its own position; anything else, or a
 * caller slot given twice, is RKV_EINVAL with nothing changed.
 * ------------------------------------------------------------------------ */

/* Creates a tree with an empty cache over a pool of `pool_slots` slots
 * (1 <= pool_slots <= 2^31-1): the walkthrough's starting point, an empty
 * radix tree (unite.ai, "SGLang: Efficient Execution of Structured Language
 * Model Programs", section "SGLang: Modelo de programacion y metodologia",
 * Step 1), over a KV memory of fixed size whose limit later
 * forces eviction (Step 5).  `initial_free`, if not NULL, gives the
 * initial FIFO order and must be a permutation of [0, pool_slots) (EINVAL
 * otherwise); NULL means 0, 1, ..., pool_slots-1.  *out receives the handle,
 * owned by the caller until rkv_tree_destroy. */
int rkv_tree_create(rkv_tree** out, int64_t pool_slots, const int32_t* initial_free);

/* Frees the tree and everything it owns (the counterpart of
 * rkv_tree_create).  NULL is a no-op. */
void rkv_tree_destroy(rkv_tree* t);

/* Longest cached prefix of tok[0..n) (the page's "matching", Step 3 of the
 * walkthrough: a new prompt finds its prefix and reuses its KV).  Walks from
 * the root; where the query ends or diverges inside an edge, that edge is
 * split (rkv contract: the new upper node gets a fresh id and copies the lower
 * node's last_access and lock; the lower node keeps its id).  Every node on
 * the path from the root to the stop node gets last_access = tick.
 * Outputs: *out_len = matched length m, out_slots[0..m) = the cached slots in
 * sequence order (out_slots must have room for n), *out_node = stop node id
 * (0 when m = 0).  Slots stay owned by the tree and stay valid only while the
 * stop node is locked. */
int rkv_radix_match(rkv_tree* t, const int32_t* tok, int64_t n, int32_t* out_slots,
                    int64_t* out_len, int64_t* out_node);

/* Length of the longest cached prefix of tok[0..n), with no side effect on
 * the tree: no split, no LRU stamp, no lock (a read-only rkv_radix_match, for
 * schedulers that rank waiting requests).  *out_len = that length. */
int rkv_radix_peek(const rkv_tree* t, const int32_t* tok, int64_t n, int64_t* out_len);

/* Cache-aware order of a waiting queue (unite.ai, "SGLang: Efficient
 * Execution of Structured Language Model Programs", section "SGLang:
 * Evaluacion y resultados": cache-aware scheduling keeps hit rates close to
 * the optimum).  Request q is tok[tok_indptr[q] .. tok_indptr[q+1]) (int64
 * offsets, Q+1 of them).  matched[q] = the prefix a batch would reuse now:
 * rkv_radix_peek of its first L_q - 1 tokens (0 for an empty request).
 * order[0..Q) = queue positions by matched descending, ties in queue order
 * (stable).  Read-only on the tree.  Q = 0 is a no-op. */
int rkv_schedule(const rkv_tree* t, int32_t Q, const int32_t* tok, const int64_t* tok_indptr,
                 int32_t* order, int64_t* matched);

/* Radix keys for an image (or any non-text input) that occupies n_tokens
 * positions of a request (the article's section "Resultados en modelos
 * multimodales": the image's hash is the radix key, so requests with the
 * same image reuse its tokens' KV).  *out_hash (nullable) = 64-bit FNV-1a of
 * bytes[0..len); keys[i] = -1 - (splitmix64(hash + (i+1) * 0x9e3779b97f4a7c15)
 * >> 33) for i < n_tokens (splitmix64 = its output finalizer), each in
 * [-2^31, -1], so they never equal a text token id (>= 0).  Put them in the
 * request's token sequence where the image's tokens sit; every tree call
 * then treats them like tokens.  EINVAL on negative sizes or NULL buffers. */
int rkv_image_keys(const uint8_t* bytes, int64_t len, int64_t n_tokens, int32_t* keys, uint64_t* out_hash);

/* The pages evict only nodes that the request being served does not need
 * (unite.ai, "SGLang: Efficient Execution of Structured Language Model
 * Programs", section "SGLang: Modelo de programacion y metodologia", Steps 5,
 * 8 and 9: the continuing session's path survives, the least
 * recently used other nodes go); they do not say how.  Reading taken: a
 * reference count per node on the matched path of every request in flight.
 * lock: +1 on the lock count of `node` and every ancestor up to, not
 * including, the root; locked nodes are never evicted.  unlock: -1 on the
 * same nodes; EINVAL (and no change) if any count would go negative or the
 * node does not exist.  Node 0 (the root) is a no-op for both. */
int rkv_radix_lock(rkv_tree* t, int64_t node);
int rkv_radix_unlock(rkv_tree* t, int64_t node);

/* Inserts tok[0..n) with the caller's slots[0..n) (unite.ai, "SGLang:
 * Efficient Execution of Structured Language Model Programs", section "SGLang:
 * Modelo de programacion y metodologia", Steps 2-3: a
 * finished sequence enters the tree; the uncached rest becomes a new node).
 * Walks and splits as match does.  The tree takes ownership of all n slots:
 * for the m positions already cached the tree keeps its own slots and
 * appends each caller slot that differs from the tree's to the FIFO tail, in
 * increasing position; if m < n the rest becomes a new leaf (fresh id) under
 * the stop node.  Every node on the path, the new leaf included, gets
 * last_access = tick.  *out_cached = m.  Slots must be in [0, pool_slots),
 * and each must be the tree's own slot for its position or a slot the
 * caller holds, given once (see Slot ownership above); otherwise RKV_EINVAL
 * and nothing changes, checked by a read-only walk before the insert. */
int rkv_radix_insert(rkv_tree* t, const int32_t* tok, const int32_t* slots, int64_t n,
                     int64_t* out_cached);

/* LRU eviction (unite.ai, "SGLang: Efficient Execution of Structured Language
 * Model Programs", section "SGLang: Modelo de programacion y metodologia",
 * Steps 5, 8, 9: whole nodes, least recently
 * used first, under a memory limit; the RadixAttention bullet of section
 * "Introduccion a SGLang" names eviction as one of the tree's operations).
 * While fewer than `want` tokens are freed: pick the unlocked non-root leaf
 * with the smallest (last_access, id), append
 * its slots to the FIFO tail in label order, detach it.  Whole leaves only,
 * so *out_freed may exceed want.  Returns RKV_EBUSY if no candidate is left
 * before `want` is reached; what was freed stays freed. */
int rkv_radix_evict(rkv_tree* t, int64_t want, int64_t* out_freed);

/* Slot allocation: the walkthrough closes by noting that RadixAttention
 * allocates and evicts nodes dynamically as requests arrive (unite.ai,
 * "SGLang: Efficient Execution of Structured Language Model Programs", section
 * "SGLang: Modelo de programacion y metodologia", the paragraph after
 * Step 9); the pages do not say how KV memory is handed out.  Reading taken:
 * one pool of token slots with a FIFO free list.
 * Pops n slots from the FIFO head into out[0..n).  RKV_ENOSPC, with no
 * change, if fewer than n are free (no implicit eviction).  The caller owns
 * the slots until it passes them to rkv_radix_insert or rkv_free. */
int rkv_alloc(rkv_tree* t, int64_t n, int32_t* out);

/* Appends slots[0..n) to the FIFO tail in the given order (the
 * counterpart of rkv_alloc).  EINVAL, with no change, if a slot is out of
 * range, not held by the caller, or given twice. */
int rkv_free(rkv_tree* t, const int32_t* slots, int64_t n);

/* out[8] = {cached tokens, free slots, evictable tokens (in nodes with lock
 * 0), locked tokens, nodes (non-root), matched tokens over all prepared
 * requests, prompt tokens over all prepared requests, evicted tokens}.
 * Cache hit rate = out[5] / out[6], the quantity the article reports
 * without a formula (unite.ai, "SGLang: Efficient Execution of Structured
 * Language Model Programs", section "SGLang: Evaluacion y resultados": hit
 * rates of 50-99 %; section "Despliegue en produccion"). */
int rkv_stats(rkv_tree* t, int64_t out[8]);

/* Canonical dump, for tests that compare two trees bit for bit (no passage:
 * inspection only): DFS from the root, children in ascending first-token
 * order; per node the int64 values (id, parent id (-1 for the root),
 * last_access, lock, len, label[len], slots[len]).  Writes at most cap
 * values; *len receives the full length (call with cap 0 to size). */
int rkv_radix_serialize(rkv_tree* t, int64_t* buf, int64_t cap, int64_t* len);

/* FIFO contents head to tail; same sizing convention as serialize
 * (inspection only, like serialize). */
int rkv_free_list(rkv_tree* t, int32_t* buf, int64_t cap, int64_t* len);

/* The serving step before attention (unite.ai, "SGLang: Efficient Execution of
 * Structured Language Model Programs", section "SGLang: Modelo de programacion
 * y metodologia": Step 3, a new prompt finds its
 * cached prefix and reuses its KV; Step 7, a batch of requests sharing
 * few-shot examples; Steps 5, 8 and 9, nodes evicted to make room).
 * Prepares one batch of B requests whose token ids are
 * tok[tok_indptr[r] .. tok_indptr[r+1]) (lengths L_r >= 1, L_r <= ld).
 * For r = 0..B-1 in order: match the first L_r - 1 tokens (so every request
 * computes at least its last token), lock the stop node.  Then with
 * T = sum(L_r - p_r): if fewer than T slots are free, evict the difference;
 * on RKV_EBUSY unlock this batch's nodes and return RKV_EBUSY (the matches,
 * splits, ticks and evictions already done remain).  Then pop T slots and
 * give them to the requests in order, positions ascending.
 * Outputs (host buffers owned by the caller):
 *   req_to_token [B, ld] row-major: cached slots then new slots, -1 after L_r
 *   prefix_lens[B] = p_r, seq_lens[B] = L_r, qo_indptr[B+1] = prefix sums of
 *   n_r = L_r - p_r, new_slots[T] (new_cap must be >= sum L_r),
 *   out_nodes[B] = locked stop nodes (hand them to rkv_batch_commit).
 * B = 0 is a no-op. */
int rkv_batch_prepare(rkv_tree* t, int32_t B, const int32_t* tok, const int64_t* tok_indptr,
                      int32_t* req_to_token, int64_t ld, int32_t* prefix_lens,
                      int32_t* seq_lens, int32_t* qo_indptr, int32_t* new_slots,
                      int64_t new_cap, int64_t* out_nodes);

/* The serving step after attention (unite.ai, "SGLang: Efficient Execution of
 * Structured Language Model Programs", section "SGLang: Modelo de programacion
 * y metodologia", Steps 2, 3 and 7: the finished
 * sequences enter the tree, new parts as new nodes, shared parts split off).
 * Commits a prepared batch: for r = 0..B-1, insert the full sequence with
 * slots req_to_token[r, 0..L_r), then unlock nodes[r].  Every argument is
 * checked before the first insert, so RKV_EINVAL changes nothing: lengths
 * in [1, ld], slots in range, nodes that exist, lock counts that cover
 * every unlock the batch makes on each node (a node named by k requests
 * needs a count >= k), and slots as rkv_radix_insert requires them, with no
 * caller slot in two requests.  The sequences must be the ones the table
 * rows describe: after rkv_batch_append, the grown sequences. */
int rkv_batch_commit(rkv_tree* t, int32_t B, const int32_t* tok, const int64_t* tok_indptr,
                     const int32_t* req_to_token, int64_t ld, const int64_t* nodes);

/* Decode continuation of a prepared batch that is not yet committed (its
 * nodes still locked): one more position per request, without matching the
 * history again.  The pages' walkthrough (unite.ai, "SGLang: Efficient
 * Execution of Structured Language Model Programs", section "SGLang: Modelo
 * de programacion y metodologia", Step 3) caches a finished turn, answer
 * included, as one new node; here the generated tokens therefore enter the
 * tree only at rkv_batch_commit, and each step needs just one new slot per
 * request.  If fewer than B slots are free, evict the difference (RKV_EBUSY
 * if that fails: no slot popped, no table entry written; leaves evicted on
 * the way stay evicted).  Then pop B slots in FIFO order and for r = 0..B-1:
 * req_to_token[r, seq_lens[r]] = new_slots[r], seq_lens[r] += 1.
 * req_to_token [B, ld] and seq_lens [B] are the caller's host tables from
 * rkv_batch_prepare (updated in place); every seq_lens[r] must be in
 * [1, ld - 1] (else RKV_EINVAL, nothing changed).  new_slots [B] is written.
 * Commit later with the extended token sequences.  B = 0 is a no-op. */
int rkv_batch_append(rkv_tree* t, int32_t B, int32_t* req_to_token, int64_t ld, int32_t* seq_lens,
                     int32_t* new_slots);

/* ------------------------------------------------------------------------
 * Device: every pointer below is a device pointer owned by the caller, 16-byte
 * aligned, tensors contiguous.  Calls are asynchronous on `stream` (a
 * hipStream_t; NULL = the null stream); the library allocates nothing on
 * these paths except a 4-byte error flag per device the first time RKV_DEBUG
 * is set, and never synchronizes except in that debug mode.
 *
 * Layouts: pools k_pool, v_pool are [pool_slots, Hkv, D] (one slot = Hkv*D
 * contiguous elements); q and o are [rows, Hq, D]; req_to_token is int32
 * [B, ld] row-major.  dtype is RKV_F32 or RKV_BF16 for q, pools and o alike.
 * Supported: D in {64, 128}, Hq % Hkv == 0, Hq / Hkv <= 16; anything else is
 * RKV_ENOTSUP.  No kernel reads or writes outside the pool whatever the
 * tables hold: a gathered entry outside [0, pool_slots) reads as zeros in
 * the decode kernels and the f32 extend, is clamped to slot pool_slots - 1 in
 * the bf16 extend (the output of such a row is meaningless either way), and
 * is skipped by scatter.  With the environment variable RKV_DEBUG=1 such an
 * entry makes the call return RKV_EINVAL after a stream synchronization.
 * ------------------------------------------------------------------------ */

/* Writes the new tokens' K/V into their pool slots, where later requests
 * that share the prefix read them instead of recomputing them (unite.ai,
 * "SGLang: Efficient Execution of Structured Language Model Programs", section
 * "Introduccion a SGLang", RadixAttention bullet: a request's KV
 * cache is kept after processing so other calls can reuse it).
 * k_pool[slots[i]] = k_new[i] and v_pool[slots[i]] = v_new[i] for
 * i in [0, T); k_new, v_new are [T, Hkv, D].  A plain copy: bit-exact, every
 * other pool row untouched.  Slots must be distinct (duplicates race).  T = 0
 * is a no-op. */
int rkv_kv_scatter(const void* k_new, const void* v_new, const int32_t* slots, int64_t T,
                   void* k_pool, void* v_pool, int64_t pool_slots, int32_t hkv, int32_t d,
                   int32_t dtype, void* stream);

/* Device side of rkv_batch_append, for a req_to_token / seq_lens pair kept
 * on the device across decode steps (only the B new slot ids cross PCIe per
 * step): for r in [0, B), req_to_token[r, seq_lens[r]] = new_slots[r] and
 * seq_lens[r] += 1.  All three are int32 device arrays (4-byte alignment
 * suffices).  A row whose seq_lens[r] is outside [0, ld) is left as it is
 * (with RKV_DEBUG=1 the call then returns RKV_EINVAL).  B = 0 is a no-op. */
int rkv_table_append(int32_t* req_to_token, int64_t ld, int32_t* seq_lens, const int32_t* new_slots,
                     int32_t B, void* stream);

/* Extend (prefill over a cached prefix): the attention of a prompt whose
 * prefix was found in the tree; only its new tokens are computed, and they
 * attend to the reused cached KV plus their own (unite.ai, "SGLang: Efficient
 * Execution of Structured Language Model Programs", section "SGLang: Modelo de
 * programacion y metodologia", Step 3; the
 * extend primitive in that section's list adds text to a prompt).  The
 * attention itself is plain causal softmax attention; the pages give no
 * formula for it.  Request r has p_r = prefix_lens[r]
 * cached tokens and n_r = qo_indptr[r+1] - qo_indptr[r] new ones, whose
 * queries are q rows qo_indptr[r] .. qo_indptr[r+1].  New row j sits at
 * position c = p_r + j and attends causally to keys 0..c of its own request:
 *   o[row, h] = sum_t softmax_t(sm_scale * q[row, h] . K_t) V_t,
 *   K_t = k_pool[req_to_token[r, t], h / (Hq/Hkv)],  V_t likewise,
 *   lse[row, h] = natural-log log-sum-exp of the scaled scores (fp32;
 *   `lse` may be NULL).
 * qo_indptr[0] must be 0, total_new must equal qo_indptr[B] (the number of
 * q rows) and max_new must be >= every n_r; together they size the grid (a
 * smaller max_new leaves rows of the longer requests unwritten).  When
 * total_new == B * max_new every request has max_new new tokens, and the
 * bf16 path takes request r's rows to start at r * max_new without reading
 * qo_indptr.  The new tokens' K/V must already be in
 * the pool (rkv_kv_scatter). bf16: QK^T and PV on bf16 MFMA with fp32
 * accumulation, fp32 online
 * softmax, softmax weights rounded to bf16 for PV, o rounded to bf16 (RNE).
 * The row sums that normalize o (and give lse) are sums of those same
 * rounded weights: each is within a factor 1 +- 2^-8 of its exact value, so
 * bf16 lse is within -ln(1 - 2^-8) (plus fp32 rounding) of the exact value.
 * f32: fp32 arithmetic throughout.  B = 0 or total_new = 0 is a no-op.
 * req_order (nullable, int32 [B], device): a permutation of the requests in
 * which the bf16 path hands out work (each request's row tiles still in
 * ascending order); it changes only the schedule (every output is
 * bit-identical to NULL's).
 * Longest first shortens ragged batches, whose launch otherwise ends on a
 * long request started late.  An entry outside [0, B) is skipped; a
 * repeated or missing request leaves rows written twice or not at all.  The
 * f32 path ignores it. */
int rkv_attn_extend(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                    const int32_t* req_to_token, int64_t ld, const int32_t* qo_indptr,
                    const int32_t* prefix_lens, const int32_t* req_order, int32_t B,
                    int64_t total_new, int32_t max_new,
                    int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t dtype,
                    int64_t pool_slots, void* stream);

/* Bytes of device workspace rkv_attn_decode needs for these sizes
 * (num_splits as passed to rkv_attn_decode); sizing for the call below.
 * 0 on bad arguments. */
size_t rkv_attn_decode_workspace_bytes(int32_t B, int32_t hq, int32_t d, int32_t max_seq_len,
                                       int32_t num_splits);

/* Single-token decode: the attention step of generation, one new token
 * per request (unite.ai, "SGLang: Efficient Execution of Structured Language
 * Model Programs", section "SGLang: Modelo de programacion y metodologia", the
 * gen primitive; section "Introduccion a
 * SGLang" notes that decoding proceeds one token at a time), reading every
 * key of the request's context through its table, cached prefix included.
 * q, o are [B, Hq, D]; request r's query is its last
 * position L_r - 1 (L_r = seq_lens[r] >= 1, its own K/V already scattered)
 * and attends to all L_r keys req_to_token[r, 0..L_r) (same formula as
 * extend).  Split-KV: the keys of a request are cut into S_r contiguous
 * chunks, each reduced to a partial (max, sum, acc) in fp32, then merged by
 * log-sum-exp rescaling.  S_r depends only on L_r and num_splits (0 =
 * ceil(L_r / 768) chunks of equal length, rounded up to 64 keys; N > 0 = at
 * most N chunks), never on the rest of
 * the batch, so a request's output bits do not depend on its batch.  Every
 * seq_lens[r] must be <= max_seq_len and <= ld.  `workspace` (ws_bytes >=
 * rkv_attn_decode_workspace_bytes) holds the partials.
 * Arithmetic: fp32 FMA on the vector units; for bf16 with Hq/Hkv >= 4 the
 * query heads of a kv head go through bf16 MFMA together (scores and PV in
 * fp32 accumulation, weights rounded to bf16 for PV, row sums of those
 * rounded weights, so lse is within ln(1 + 2^-8) of the exact value). */
int rkv_attn_decode(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                    const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                    int32_t B, int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d,
                    float sm_scale, int32_t dtype, int32_t num_splits, void* workspace,
                    size_t ws_bytes, int64_t pool_slots, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as rkv_attn_decode (same arguments minus the workspace, same
 * kernels, bit-identical results), with the split partials in a scratch
 * array that the library holds, one per GPU it runs on, for the life of the
 * process: 32 MiB (33554432 bytes).  A call whose
 * rkv_attn_decode_workspace_bytes(B, hq, d, max_seq_len, num_splits) exceeds
 * that returns RKV_EINVAL and launches nothing.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on a
 * device takes the array's device address (hipGetSymbolAddress).  Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller.
 * Under RKV_DEBUG=1 out-of-range slots are reported through a flag held the
 * same way. */
int rkv_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                            const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                            int32_t B, int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d,
                            float sm_scale, int32_t dtype, int32_t num_splits, int64_t pool_slots,
                            void* stream);

/* ------------------------------------------------------------------------
 * Prefix-shared ("cascade") decode.  Requests under one radix node gather the
 * same slots for that node's keys (the page's RadixAttention bullet, section
 * "Introduccion a SGLang": a shared prefix is cached once and reused).  This
 * extension reads each such shared run once per decode batch for all of its
 * requests and merges the partial softmax state with each request's private
 * remainder, by the same log-sum-exp rule as split-KV decode.  The result is
 * the decode attention defined above; only the rounding order differs.
 * ------------------------------------------------------------------------ */

/* Host planner.  From the host copy of a decode batch's table
 * (req_to_token [B, ld], seq_lens[B], 1 <= L_r <= ld) it finds the runs of
 * keys that several requests share with identical slots:
 *   - row r is considered over its first L_r - 1 keys (the query key is
 *     private); perm[0..B) = requests sorted by that row (slot ids compared
 *     as int32 sequences, a proper prefix first), ties by request id;
 *   - every maximal block of requests sharing a prefix deeper than their
 *     parent block's gives a segment [start, depth), where start is the end
 *     of the last emitted segment above it; a segment shorter than min_keys
 *     is not emitted and its keys fall to the segments (or tails) below;
 *   - segments are cut into seg_chunk-key chunks and into member groups of
 *     at most max_members (consecutive in perm).  jobs[5*i ..] =
 *     {key_begin, key_end, first, count, rec_off}: the requests
 *     perm[first .. first+count) share slots over [key_begin, key_end) of
 *     their rows; each gets that chunk's partial in its record rec_off;
 *   - tail_begin[r]: first key of r's private tail (always < L_r); the tail
 *     is cut into tail_chunk-key splits;
 *   - records of r: its shared chunks in path order, then its tail splits;
 *     rec_indptr[B+1] = their prefix sums (rec_indptr[B] = n_records);
 *     *out_tail_splits = the most tail splits of any request.
 * Jobs are in a preorder of the prefix tree.  jobs_cap counts jobs (5 int32
 * each); with fewer than needed the call returns RKV_ENOSPC, sets
 * *out_n_jobs to the number needed and writes nothing else (call with
 * jobs_cap 0 and jobs NULL to size).  EINVAL on bad sizes or NULL pointers.
 * O(sum L_r log B) time. */
int rkv_cascade_plan(const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens, int32_t B,
                     int32_t seg_chunk, int32_t tail_chunk, int32_t min_keys, int32_t max_members,
                     int32_t* perm, int32_t* rec_indptr, int32_t* tail_begin, int32_t* jobs,
                     int64_t jobs_cap, int64_t* out_n_jobs, int32_t* out_tail_splits);

/* Bytes of device workspace rkv_attn_decode_cascade needs: n_records
 * records of Hq rows of (d + 4) fp32 (sizing for the call below).  0 on bad
 * arguments. */
size_t rkv_attn_decode_cascade_workspace_bytes(int64_t n_records, int32_t hq, int32_t d);

/* Decode (same inputs, outputs and formula as rkv_attn_decode) following a
 * plan from rkv_cascade_plan built on the same req_to_token and seq_lens,
 * with the same max_members and tail_chunk; perm, rec_indptr, tail_begin
 * and jobs are that plan's arrays copied to the device, n_jobs, tail_splits
 * and n_records (= rec_indptr[B]) its host values.  Phase 1 runs one wave
 * per (kv head, job): the job's keys are gathered once, from the row of
 * request perm[first], for the count * (Hq/Hkv) query columns of its
 * members (bf16 MFMA; max_members * Hq/Hkv columns at most 32 for d = 128
 * and 64 for d = 64, ENOTSUP otherwise), and one wave or workgroup per
 * (request, tail split) covers the private keys; phase 2 merges each request's
 * records.  bf16
 * only (ENOTSUP otherwise); arithmetic as in rkv_attn_decode's MFMA path.
 * The plan's values are checked in the kernels before they index anything:
 * a job or request that does not fit is skipped, and with RKV_DEBUG=1 the
 * call returns RKV_EINVAL.  Workspace: rkv_attn_decode_cascade_workspace_bytes
 * (may be NULL when n_jobs == 0 and n_records == B: every request then has
 * one partial).
 * tail_order (nullable, int32 [B], device): a permutation of the requests
 * in which the tail splits are handed out (the shared jobs keep the plan's
 * order); it changes only the schedule (every output is bit-identical to
 * NULL's).  Requests whose tail splits are longest first let the launch end
 * on short items.  An entry outside [0, B) is skipped; a repeated or missing
 * request leaves its tails computed twice or not at all (its output then
 * merges stale workspace). */
int rkv_attn_decode_cascade(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                            const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens, int32_t B,
                            int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                            int32_t dtype, const int32_t* perm, const int32_t* rec_indptr,
                            const int32_t* tail_begin, const int32_t* jobs, int64_t n_jobs,
                            const int32_t* tail_order, int32_t max_members, int32_t tail_chunk,
                            int32_t tail_splits, int64_t n_records, void* workspace, size_t ws_bytes,
                            int64_t pool_slots, void* stream);

/* ------------------------------------------------------------------------
 * Sampling penalties over the running requests (the sampling page,
 * sglang-zh.llamafactory.cn, "sampling_params": the Penalties block defines
 * frequency_penalty, presence_penalty, repetition_penalty and
 * min_new_tokens; its section on the performance implications of penalties
 * puts them on the GPU for the whole batch, with state of size vocab x
 * running requests).  Formulas (the page gives intent and ranges only):
 *   for every token of the prompt or the output: x = x > 0 ? x / r : x * r;
 *   for every token of the output: x = x - f * count - p;
 *   while out_len < min_new_tokens: x = -inf for the request's stop ids
 *   (its EOS and stop_token_ids), after the two steps above.
 * fp32 arithmetic (x / r correctly rounded, then one fma for -f*count and
 * one subtraction); bf16 logits are read exactly and written rounded to
 * nearest even.
 *
 * State, per request slot (device memory owned by the caller; slots index
 * rows, so requests can come and go):
 *   counts [n_slots, vocab] int32: bits 0..30 = times the token occurs in
 *     the output so far (saturating), bit 31 = it occurs in the prompt;
 *   seen [n_slots, cap] int32 and seen_len [n_slots]: the distinct tokens of
 *     prompt and output, each once, in unspecified order; cap must be at
 *     least the request's distinct prompt tokens plus its output length;
 *   out_len [n_slots]: output tokens so far.
 * Rows, token ids and stop ids are range-checked in the kernels: an entry out
 * of range (or a full seen list) is skipped, and with RKV_DEBUG=1 the call
 * returns RKV_EINVAL after a stream synchronization.
 * ------------------------------------------------------------------------ */

/* Admits n requests: for request i, slot rows[i] is reset (counts row zero,
 * out_len 0) and its prompt prompt_ids[prompt_indptr[i] ..
 * prompt_indptr[i+1]) (device int32, n+1 offsets) is marked in bit 31 and
 * listed in seen.  rows must be distinct.  n = 0 is a no-op. */
int rkv_penalty_admit(int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len, int32_t n_slots,
                      int32_t vocab, int32_t cap, int32_t n, const int32_t* rows, const int32_t* prompt_indptr,
                      const int32_t* prompt_ids, void* stream);

/* Records one output token per running request: for b in [0, B), tokens[b]
 * is appended to slot rows[b] (count + 1, listed in seen if new, out_len +
 * 1).  rows must be distinct.  Call it after sampling, before the next
 * apply.  B = 0 is a no-op. */
int rkv_penalty_accumulate(int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len, int32_t n_slots,
                           int32_t vocab, int32_t cap, int32_t B, const int32_t* rows, const int32_t* tokens,
                           void* stream);

/* Applies the penalties in place to logits [B, ld] (row b belongs to slot
 * rows[b]; dtype RKV_F32 or RKV_BF16; ld >= vocab; only the first vocab
 * entries of a row are read or written).  Per batch entry b (device
 * arrays): freq[b], pres[b], rep[b] (float), min_new[b] (int32), stop ids
 * stop_ids[stop_indptr[b] .. stop_indptr[b+1]) (stop_ids may be NULL when
 * every list is empty).  new_tokens (nullable, [B]): when given, each
 * request's previous output token is first recorded exactly as
 * rkv_penalty_accumulate does, in the same launch (one launch per decode
 * step).  Only the logits of listed tokens and, while masking, the stop ids
 * are touched: O(prompt + output) entries per request, not O(vocab).
 * rows must be distinct.  B = 0 is a no-op. */
int rkv_penalty_apply(void* logits, int64_t ld, int32_t dtype, int32_t B, const int32_t* rows, int32_t* counts,
                      int32_t* seen, int32_t* seen_len, int32_t* out_len, int32_t n_slots, int32_t vocab,
                      int32_t cap, const float* freq, const float* pres, const float* rep, const int32_t* min_new,
                      const int32_t* stop_indptr, const int32_t* stop_ids, const int32_t* new_tokens,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
