// Split-KV single-token decode attention over the token-slot pool.
//
// Decoding one token per request (the page's `gen` primitive run step by step;
// unite.ai, "SGLang: Efficient Execution of Structured Language Model
// Programs", section "SGLang: Modelo de programacion y metodologia") reads the
// whole cached K/V of every request once: about 1 flop per byte for plain
// multi-head attention, 8 for 8-way grouped heads.  The kernel is therefore
// bound by HBM bandwidth and is built to keep many 16-byte gathers in flight:
//
//   phase 1  one workgroup (4 waves) per (split, request, kv head [, head
//            group]).  A row of K (or V) for one kv head is D elements =
//            LPR lanes x 16 bytes, so one wave instruction gathers RPW = 64/LPR
//            whole rows from arbitrary slots, and every wave keeps U rows of K
//            and U rows of V per lane in flight.  Scores are reduced across the
//            LPR lanes of a row with DPP row operations; each row group keeps
//            an fp32 online-softmax state (m, l, acc) per query head; groups
//            are merged with cross-lane exchanges and then across waves in LDS.
//            A request whose keys fit in one split writes o and lse directly;
//            otherwise the split's (m, l, acc) goes to the workspace.
//   phase 2  one wave per (request, q head) merges the S_r partials by
//            log-sum-exp rescaling.
//
// S_r depends only on L_r (and the caller's num_splits), never on the rest of
// the batch, so a request's output bits do not depend on its batch; by
// default a request gets ceil(L_r / 768) splits of equal length.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <string>
#include <type_traits>

#include "device.h"
#include "rkv.h"
#include "rkv_internal.h"

namespace {

constexpr int kChunk = 768;     // keys per split under the default rule (measured: 512-768 best on MHA, 768 on 64/8 GQA)
constexpr int kMaxG = 8;        // query heads handled per workgroup

struct DecodeArgs {
  const void* q;
  const void* kp;
  const void* vp;
  void* o;
  float* lse;
  const int32_t* r2t;
  int64_t ld;
  const int32_t* seq_lens;
  int32_t B, hq, hkv, G, hg;      // hg = head groups of <= kMaxG per kv head
  int32_t max_seq_len;            // every length is clamped to it (<= ld)
  int32_t hb;                     // kv heads per workgroup (a slot's contiguous run)
  int32_t splits;                 // grid extent over splits
  int32_t num_splits;             // 0 = fixed chunk rule
  float scale_log2e;              // sm_scale * log2(e)
  int64_t pool_slots;
  float* ws;                      // [B, hq, splits, D + 4]: acc[D], max, sum, pad
  int* err;
  // prefix-shared plan (all null for plain decode): the partials of request
  // r are records rec_indptr[r] .. rec_indptr[r+1] of ws, laid out
  // [record, hq, D + 4]; its private keys tail_begin[r] .. L_r are cut into
  // tail_chunk-key splits that fill the last records of that range
  const int32_t* rec_indptr;
  const int32_t* tail_begin;
  int32_t n_records;
  int32_t tail_chunk;
  // optional order of the requests' tail splits (null: batch order): the
  // tail item at request position i works on request tail_order[i]
  const int32_t* tail_order;
};

// Prefix-shared jobs: keys [key_begin, key_end) of request perm[first]'s row
// are common to the `count` requests perm[first .. first+count); each of them
// gets that range's partial in its record rec_indptr[r] + rec_off.
struct SharedJobs {
  const int32_t* jobs;            // [n_jobs, 5]: key_begin, key_end, first, count, rec_off
  const int32_t* perm;            // [B]
  int32_t n_jobs;
  int32_t max_members;
};

// 16-byte K/V loads.  STREAM = non-temporal: measured on this chip, random
// 256-byte to 4-KB row gathers reach ~6.7 TB/s with the hint and ~6.1 TB/s
// without (a 4-GiB read: 7.0 vs 6.3 TB/s).  The hint pays only for rows that
// no other request of the launch reads and that each instruction reads
// whole: the private tails of a prefix-shared plan (c3 tails: 1227 -> 1128
// us).  Plain decode keeps normal loads, because siblings there re-read
// shared rows from L2/MALL (c3: 1288 -> 1417 us with the hint), and so do
// the matrix-core K loads, which read half cache lines per instruction.  The
// matrix-core V tiles (whole rows per DMA instruction) stream for the tails
// of large prefix-shared launches.  For the shared runs the hint gains 2 %
// on back-to-back decode launches but loses 1-3 % when the decode follows an
// extend step (c3), so they keep normal loads.
typedef unsigned int kv_u32x4 __attribute__((ext_vector_type(4)));
// cache-policy operand of an LDS-DMA load that marks it non-temporal
constexpr int kNonTemporal = 2;
template <bool STREAM>
__device__ __forceinline__ uint4 load_kv(const char* p) {
  if constexpr (STREAM) {
    const kv_u32x4 w = __builtin_nontemporal_load((const kv_u32x4*)p);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return *(const uint4*)p;
  }
}

// Keys per split of a request of L keys.  num_splits > 0: at most that many
// splits.  0: ceil(L / kChunk) splits, the count of kChunk-key chunks, but
// of equal length (rounded up to 64 keys, so never above kChunk, and the
// count stays the same): a short last split per request would leave the
// launch's last round to full-length items.  Either way the split depends
// only on L.
__host__ __device__ inline int split_chunk(int L, int num_splits) {
  int n = num_splits > 0 ? num_splits : (L + kChunk - 1) / kChunk;
  if (n < 1) n = 1;
  const int c = (L + n - 1) / n;
  return c < 64 ? 64 : ((c + 63) / 64) * 64;
}

// Keys [k_begin, k_end) of split s of request r (of length L), and where its
// partial goes: rec < 0 means the split is the request's only partial and
// writes o and lse itself; otherwise the partial goes to workspace record
// `rec` (plain layout: split index; prefix-shared layout: record index).
// Returns false when the split is empty, or when a prefix-shared plan does
// not fit the request (flag raised in debug mode; nothing is written).
__device__ __forceinline__ bool split_span(const DecodeArgs& a, int r, int s, int L, int& k_begin, int& k_end,
                                           int& rec, int& nsplit) {
  if (!a.rec_indptr) {
    const int chunk = split_chunk(L, a.num_splits);
    nsplit = (L + chunk - 1) / chunk;
    if (s >= nsplit) return false;
    k_begin = s * chunk;
    k_end = min(L, k_begin + chunk);
    rec = nsplit == 1 ? -1 : s;
    return true;
  }
  const int tb = a.tail_begin[r];
  const int r0 = a.rec_indptr[r], r1 = a.rec_indptr[r + 1];
  nsplit = (L - tb + a.tail_chunk - 1) / a.tail_chunk;
  if (tb < 0 || tb >= L || r0 < 0 || r1 > a.n_records || r1 - r0 < nsplit) {
    if (s == 0 && a.err) rkv::raise_flag(a.err);
    return false;
  }
  if (s >= nsplit) return false;
  // the tail's nsplit splits of equal length (rounded up to 64 keys, never
  // above tail_chunk: every split keeps at least one key)
  const int tc = min(a.tail_chunk, ((L - tb + nsplit - 1) / nsplit + 63) / 64 * 64);
  k_begin = tb + s * tc;
  k_end = min(L, k_begin + tc);
  rec = (r1 - r0 == 1) ? -1 : r1 - nsplit + s;
  if (rec >= 0 && !a.ws) {
    if (a.err) rkv::raise_flag(a.err);
    return false;
  }
  return true;
}

// Workspace row of (request r, q head, record/split rec).
__device__ __forceinline__ float* ws_row(const DecodeArgs& a, int D, int r, int head, int rec) {
  if (a.rec_indptr) return a.ws + ((int64_t)rec * a.hq + head) * (D + 4);
  return a.ws + (((int64_t)r * a.hq + head) * a.splits + rec) * (D + 4);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static void unpack(const uint4& w, float* f) {
    f[0] = __builtin_bit_cast(float, w.x);
    f[1] = __builtin_bit_cast(float, w.y);
    f[2] = __builtin_bit_cast(float, w.z);
    f[3] = __builtin_bit_cast(float, w.w);
  }
  __device__ static float load1(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store1(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static void unpack(const uint4& w, float* f) {
    f[0] = rkv::bf16lo(w.x); f[1] = rkv::bf16hi(w.x);
    f[2] = rkv::bf16lo(w.y); f[3] = rkv::bf16hi(w.y);
    f[4] = rkv::bf16lo(w.z); f[5] = rkv::bf16hi(w.z);
    f[6] = rkv::bf16lo(w.w); f[7] = rkv::bf16hi(w.w);
  }
  __device__ static float load1(const void* p, int64_t i) { return rkv::bf16_to_f32(((const uint16_t*)p)[i]); }
  __device__ static void store1(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = rkv::f32_to_bf16(v); }
};

// Combine state b into state a (log2-domain maxima).
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float mb, float lb,
                                            const float* accb, int n) {
  const float M = fmaxf(m, mb);
  if (M == -INFINITY) return;
  const float fa = exp2f(m - M), fb = exp2f(mb - M);
  l = l * fa + lb * fb;
  for (int e = 0; e < n; ++e) acc[e] = acc[e] * fa + accb[e] * fb;
  m = M;
}

// Phase 1 on the matrix cores (bf16): query columns that read the same K/V
// rows go through v_mfma_f32_16x16x32_bf16 together as the N dimension
// (S^T = K Q^T, 16 keys x 16 query columns per block).  Two users:
//   * grouped heads (Hq/Hkv >= 4): one wave per (request, kv head, split),
//     the G query heads of the kv head are the columns (one block);
//   * prefix-shared jobs: one wave per (job, kv head); the columns are
//     (member request, q head) pairs, up to CB blocks of 16, and every block
//     reuses the same K operands and the same V tile.
// One wave walks its keys 32 at a time:
//   * the 32 K rows are copied global -> LDS as whole rows by 16-byte DMA
//     into one K stage (KLDS: the matrix-core kernels), read back as MFMA A
//     operands (ds_read_b128) by the score products, and refilled for the
//     next step as soon as those products have their operands.  Whole rows
//     per instruction halve the L1 requests per byte against the other form,
//     where each lane gathers the 16-byte pieces of its two K rows straight
//     into registers (64 bytes of a row per instruction, half a cache line):
//     measured, the L1's request handling bounded that form (64/8-head
//     decode 234 -> 219 us plain, 227 -> 214 us prefix-shared; the 8/1-head
//     share 39 -> 33 us).  The register form stays for the shared items of
//     the vector kernel's prefix-shared variant, whose LDS holds four waves'
//     V stages and no more;
//   * the 32 V rows are copied global -> LDS by 16-byte DMA (two stages) and
//     read transposed (ds_read_b64_tr_b16) as the V^T operand of O^T += V^T P^T;
//   * K rows are assigned so that a lane's S^T accumulators hold 8 consecutive
//     keys, which is its slice of the bf16 P^T operand;
//   * fp32 online softmax in the log2 domain, row sums on the MFMA.
// Bytes moved are the vector kernel's for one block; the arithmetic moves
// from VALU FMAs (8 per head per element) to the matrix cores.
namespace gqa {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define RKV_LDS __attribute__((address_space(3)))
constexpr float kRescaleThreshold = 8.0f;
// key (within a 32-key step) whose K row feeds MFMA row m of block kb
__device__ __forceinline__ int key_of(int kb, int m) { return 8 * (m >> 2) + 4 * kb + (m & 3); }
template <int CH>
__device__ __forceinline__ int swz_v(int row) {
  return CH == 16 ? ((row & 3) | (((row >> 3) & 3) << 2)) : ((row & 3) | (((row >> 3) & 1) << 2));
}

// Online-softmax state of CB column blocks; lane (column l16, group gq)
// holds o for d = db*16 + 4*gq + [0..3], the row sum in l[cb][0], and the
// running maximum (log2 domain) of its column in m[cb].
template <int D, int CB>
struct State {
  f32x4 o[CB][D / 16];
  f32x4 l[CB];
  float m[CB];
};

// Walks keys [k_begin, k_end) of row_tab for kv head g; q[cb][k] is the Q^T
// operand of block cb (columns l16, rows d = k*32 + 8*gq + [0..7]).  Blocks
// cb >= ncb (wave-uniform) are skipped.  Every gather is clamped into the
// range and into the pool.  VSTREAM: the V tiles are fetched non-temporally.
// LDS DMA issued from assembly (lane l's 16 bytes land at lds + 16*l): the
// compiler then keeps no lgkmcnt bookkeeping for it and does not drain the
// operand reads fetched ahead; every stage it fills is read only after a full
// s_waitcnt by the same wave.  The LDS address is the low half of the generic
// address (the shared aperture is 4 GiB aligned).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int D, int CB, bool VSTREAM, bool KLDS>
__device__ __forceinline__ void walk(const DecodeArgs& a, const int32_t* row_tab, int k_begin, int k_end, int g,
                                     const bf16x8 (&q)[CB][D / 32], int ncb, State<D, CB>& st, char* V0,
                                     char* V1, char* KS) {
  constexpr int ROWB = D * 2;
  constexpr int CH = D / 8;
  constexpr int KSTEPS = D / 32;
  constexpr int DBLK = D / 16;
  constexpr int STEP = 32;
  constexpr int RPI = 1024 / ROWB;          // V rows per DMA instruction
  constexpr int NDMA = STEP / RPI;          // DMA instructions per step
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, gq = lane >> 4;
  const float c = a.scale_log2e;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  const uint32_t P = (uint32_t)min(a.pool_slots, (int64_t)0x7fffffff);
  const uint32_t slot_bytes = (uint32_t)a.hkv * ROWB;
  const char* kg = (const char*)a.kp + (uint64_t)g * ROWB + (KLDS ? 0 : gq * 16);
  const char* vg = (const char*)a.vp + (uint64_t)g * ROWB;
  // lane (lane & 31) loads the slot of key base + (lane & 31).  Its range
  // check (checked) is taken where the slots are used, one step later: a
  // test right after the load would wait for every gather still in flight.
  auto fetch = [&](int base) -> int32_t { return row_tab[min(base + (lane & 31), k_end - 1)]; };
  auto checked = [&](int32_t slot) -> int32_t {
    if ((uint32_t)slot >= P) {
      if (a.err) rkv::raise_flag(a.err);
      slot = 0;
    }
    return slot;
  };
  // K operands of one step (register form); refilled for the next step as
  // soon as the score products have read them
  uint4 kreg[2][KSTEPS];
  auto load_k = [&](int32_t slots) {
    if constexpr (KLDS) {
      // whole 256-byte rows into the K stage: LDS row R = 16*kb + m holds
      // the key feeding MFMA row m of block kb, its 16-byte chunks XORed
      // with the row so that a 16-row operand read is conflict-free
      const int drow = lane / CH, dch = lane % CH;
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const int R = j * RPI + drow;
        const int32_t sl = __shfl(slots, key_of(R >> 4, R & 15));
        dma16(kg + (uint64_t)(uint32_t)sl * slot_bytes + ((dch ^ (R & (CH - 1))) << 4), KS + j * 1024);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int32_t sl = __shfl(slots, key_of(kb, l16));
        const char* rowp = kg + (uint64_t)(uint32_t)sl * slot_bytes;
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) kreg[kb][k] = load_kv<false>(rowp + k * 64);
      }
    }
  };
  auto k_op = [&](int kb, int k) -> bf16x8 {
    if constexpr (KLDS) {
      const int R = kb * 16 + l16;
      return __builtin_bit_cast(bf16x8, *(const uint4*)(KS + R * ROWB + (((4 * k + gq) ^ (R & (CH - 1))) << 4)));
    } else {
      return __builtin_bit_cast(bf16x8, kreg[kb][k]);
    }
  };
  auto dma_v = [&](int32_t slots, char* dst) {
    const int drow = lane / CH, dch = lane % CH;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int R = j * RPI + drow;
      const int32_t sl = __shfl(slots, R);
      const int lch = dch ^ swz_v<CH>(R);
      __builtin_amdgcn_global_load_lds((const void*)(vg + (uint64_t)(uint32_t)sl * slot_bytes + lch * 16),
                                       (RKV_LDS void*)(dst + j * 1024), 16, 0, VSTREAM ? kNonTemporal : 0);
    }
  };
  // K(k_begin) in the K stage (or registers) and V(k_begin) in stage V0; the
  // slots of each next step are fetched a step ahead
  {
    const int32_t s0 = checked(fetch(k_begin));
    load_k(s0);
    dma_v(s0, V0);
  }
  int32_t nslot = 0;
  if (k_begin + STEP < k_end) nslot = fetch(k_begin + STEP);
  // One 32-key step on the K operands (K stage or kreg) and the V tile in
  // `cur`; with LOAD it issues the next step's gathers (K once the score
  // products have read theirs, V into `nxt`).  The stages are fixed at compile
  // time, and the loads happen unconditionally inside a step, so that
  // nothing waits for a gather it does not read:
  //   - with a run-time LDS stage index the compiler cannot tell the
  //     transposed reads from the DMA still in flight and waits for all of it
  //     before them;
  //   - a conditional load into registers becomes a copy at the join, which
  //     waits for the load.
  // Either puts one full memory latency into every step.
  auto step = [&](int base, char* cur, char* nxt, auto load_tag) {
    constexpr bool LOAD = decltype(load_tag)::value;
    // the scheduler may not pull this step's products above the wait (it
    // would then wait in the previous step for these gathers)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);          // K operands, this step's V tile and the next slots are in
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sacc[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (cb >= ncb) break;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
          sacc[cb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_op(kb, k), q[cb][k], sacc[cb][kb], 0, 0, 0);
      }
    }
    if constexpr (LOAD) {
      nslot = checked(nslot);
      load_k(nslot);
      dma_v(nslot, nxt);
      if (base + 2 * STEP < k_end) nslot = fetch(base + 2 * STEP);
    }
    // lane (column l16, group gq) holds keys base + 8*gq + 4*kb + i
    const int lim = k_end - 1 - base;
    bf16x8 pb[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if (cb >= ncb) break;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (8 * gq + 4 * kb + i > lim) sacc[cb][kb][i] = -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(sacc[cb][0][0], sacc[cb][0][1]), fmaxf(sacc[cb][0][2], sacc[cb][0][3])),
                       fmaxf(fmaxf(sacc[cb][1][0], sacc[cb][1][1]), fmaxf(sacc[cb][1][2], sacc[cb][1][3])));
      mx = rkv::max_xor16(mx);
      mx = rkv::max_xor32(mx);
      const float mt = mx * c;
      if (__builtin_amdgcn_ballot_w64(mt > st.m[cb] + kRescaleThreshold)) {
        const float mn = fmaxf(st.m[cb], mt);
        const float alpha = __builtin_amdgcn_exp2f(st.m[cb] - mn);
        st.m[cb] = mn;
        st.l[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) st.o[cb][db] *= alpha;
      }
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kb = e >> 1, i = 2 * (e & 1);
        wv[e] = rkv::pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sacc[cb][kb][i], c, -st.m[cb])),
                                 __builtin_amdgcn_exp2f(fmaf(sacc[cb][kb][i + 1], c, -st.m[cb])));
      }
      pb[cb] = __builtin_bit_cast(bf16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
      st.l[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[cb], st.l[cb], 0, 0, 0);
    }
    // PV: one V^T operand of this tile at a time, reused by every block
    const char* vs = cur;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      v4i16 part[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = gq * 8 + hh * 4 + (l16 >> 2);
        const int d = db * 16 + 4 * (l16 & 3);
        const char* ptr = vs + row * ROWB + (((d >> 3) ^ swz_v<CH>(row)) << 4) + ((d & 7) << 1);
        part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RKV_LDS v4i16*)ptr);
      }
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, make_uint4(__builtin_bit_cast(uint2, part[0]).x, __builtin_bit_cast(uint2, part[0]).y,
                             __builtin_bit_cast(uint2, part[1]).x, __builtin_bit_cast(uint2, part[1]).y));
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (cb >= ncb) break;
        st.o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[cb], st.o[cb][db], 0, 0, 0);
      }
    }
  };
  using Load = std::true_type;
  using Last = std::false_type;
  int base = k_begin;
  for (; base + 2 * STEP < k_end; base += 2 * STEP) {   // both steps have a successor
    step(base, V0, V1, Load{});
    step(base + STEP, V1, V0, Load{});
  }
  if (base + STEP < k_end) {
    step(base, V0, V1, Load{});
    step(base + STEP, V1, V0, Last{});
  } else {
    step(base, V0, V1, Last{});
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Loads the Q^T operand of one column (zeros when the column is unused).
template <int D>
__device__ __forceinline__ void load_q(const void* qbase, int64_t row, bool valid, bf16x8 (&out)[D / 32]) {
  const uint16_t* qp = (const uint16_t*)qbase + row * D + ((threadIdx.x & 63) >> 4) * 8;
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *(const uint4*)(qp + k * 32);
    out[k] = __builtin_bit_cast(bf16x8, v);
  }
}

// Writes one column's unnormalised partial (o, max, sum) to a workspace row.
template <int D>
__device__ __forceinline__ void store_partial(float* dst, const f32x4 (&o)[D / 16], float m, float l) {
  const int gq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *(f32x4*)(dst + db * 16 + 4 * gq) = o[db];
  if (gq == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}
}  // namespace gqa

template <int D, bool VSTREAM>
__device__ __forceinline__ void gqa_item(const DecodeArgs& a, int64_t w, char* V0, char* V1, char* KS) {
  using namespace gqa;
  const int s = (int)(w % a.splits);
  int64_t rest = w / a.splits;
  int r = (int)(rest % a.B);
  const int g = (int)(rest / a.B);
  if (g >= a.hkv) return;
  if (a.tail_order) {
    r = a.tail_order[r];
    if ((unsigned)r >= (unsigned)a.B) return;
  }
  const int L = min(a.seq_lens[r], a.max_seq_len);
  int k_begin, k_end, rec, nsplit;
  if (!split_span(a, r, s, L, k_begin, k_end, rec, nsplit)) return;

  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, gq = lane >> 4;
  const bool hvalid = l16 < a.G;
  const int head = g * a.G + (hvalid ? l16 : 0);
  bf16x8 qreg[1][D / 32];
  load_q<D>(a.q, (int64_t)r * a.hq + head, hvalid, qreg[0]);
  State<D, 1> st;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) st.o[0][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.l[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m[0] = -INFINITY;
  walk<D, 1, VSTREAM, true>(a, a.r2t + (int64_t)r * a.ld, k_begin, k_end, g, qreg, 1, st, V0, V1, KS);
  if (!hvalid) return;
  const float lsum = st.l[0][0];
  if (rec < 0) {
    const float inv = 1.f / lsum;
    uint16_t* orow = (uint16_t*)a.o + ((int64_t)r * a.hq + head) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *(uint2*)(orow + db * 16 + 4 * gq) = make_uint2(rkv::pack_bf16x2(st.o[0][db][0] * inv, st.o[0][db][1] * inv),
                                                      rkv::pack_bf16x2(st.o[0][db][2] * inv, st.o[0][db][3] * inv));
    if (a.lse && gq == 0) a.lse[(int64_t)r * a.hq + head] = (st.m[0] + log2f(lsum)) * 0.69314718055994531f;
  } else {
    store_partial<D>(ws_row(a, D, r, head, rec), st.o[0], st.m[0], lsum);
  }
}

// Prefix-shared phase 1: one wave per (kv head, job), kv head outermost so
// that the member groups of one chunk (consecutive jobs, same K/V) run side
// by side on one XCD.  Column c = cb*16 + l16 is member c / G of the job and
// q head g*G + c % G.  The plan's values are checked against the batch
// before use; a job that does not fit is skipped (flag raised in debug mode).
template <int D, int CB, bool KLDS>
__device__ __forceinline__ void shared_item(const DecodeArgs& a, const SharedJobs& j, int64_t w, char* V0,
                                            char* V1, char* KS) {
  using namespace gqa;
  const int job = (int)(w % j.n_jobs);
  const int g = (int)(w / j.n_jobs);
  if (g >= a.hkv) return;
  const int32_t* jp = j.jobs + (int64_t)job * 5;
  const int kb = jp[0], ke = jp[1], first = jp[2], count = jp[3], rec_off = jp[4];
  if (kb < 0 || ke <= kb || ke > a.ld || first < 0 || count < 1 || count > j.max_members ||
      first + count > a.B || rec_off < 0) {
    if (g == 0 && a.err) rkv::raise_flag(a.err);
    return;
  }
  const int rep = j.perm[first];
  if ((unsigned)rep >= (unsigned)a.B) {
    if (g == 0 && a.err) rkv::raise_flag(a.err);
    return;
  }
  const int l16 = threadIdx.x & 15;
  const int ncb = (count * a.G + 15) / 16;
  bf16x8 qreg[CB][D / 32];
  int req[CB], head[CB];
  bool valid[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = cb * 16 + l16;
    const int mem = col / a.G;
    valid[cb] = mem < count;
    req[cb] = valid[cb] ? j.perm[first + mem] : 0;
    if ((unsigned)req[cb] >= (unsigned)a.B) {
      if (a.err) rkv::raise_flag(a.err);
      valid[cb] = false;
      req[cb] = 0;
    }
    head[cb] = g * a.G + col % a.G;
    load_q<D>(a.q, (int64_t)req[cb] * a.hq + head[cb], valid[cb], qreg[cb]);
  }
  State<D, CB> st;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) st.o[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.l[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m[cb] = -INFINITY;
  }
  walk<D, CB, false, KLDS>(a, a.r2t + (int64_t)rep * a.ld, kb, ke, g, qreg, ncb, st, V0, V1, KS);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (!valid[cb]) continue;
    const int r = req[cb];
    const int r0 = a.rec_indptr[r], r1 = a.rec_indptr[r + 1];
    const int rec = r0 + rec_off;
    if (r0 < 0 || rec >= r1 || r1 > a.n_records || !a.ws) {
      if (a.err) rkv::raise_flag(a.err);
      continue;
    }
    store_partial<D>(ws_row(a, D, r, head[cb], rec), st.o[cb], st.m[cb], st.l[cb][0]);
  }
}

// Block b of a prefix-shared launch on the matrix cores of `total` blocks,
// `sb` of them shared (both multiples of 8, total > 0): whether it runs a
// shared item, and its index among the blocks of its kind.  The kinds are
// interleaved in groups of 8 consecutive blocks (one per XCD) in proportion
// to their counts, so the latency-bound shared items run beside the
// bandwidth-bound tails instead of all before them; group g of a kind holds
// that kind's blocks 8g .. 8g+7, so each kind keeps its XCD-contiguous item
// ranges.
__device__ __forceinline__ bool cascade_block(int64_t b, int64_t sb, int64_t total, int64_t& idx) {
  const int64_t gt = total / rkv::kXcds, gs = sb / rkv::kXcds, g = b / rkv::kXcds;
  const int64_t c0 = g * gs / gt, c1 = (g + 1) * gs / gt;   // shared groups before g, and through g
  idx = (c1 > c0 ? c0 : g - c0) * rkv::kXcds + b % rkv::kXcds;
  return c1 > c0;
}

// Phase 1.  Work item = (request, split, block of HB kv heads [, q-head
// group]).  A key's rows for the HB heads are HB*D contiguous elements of the
// slot, so the workgroup reads them as one contiguous run: lane group
// (LPR lanes) hl handles kv head hb*HB + hl, and RPI = 256/(HB*LPR) keys are
// read per instruction (one per row group ri, which is wave-uniform, so the
// slot index is a scalar load).  Each lane group walks the keys of the split
// with its own fp32 online softmax; row groups (RPI > 1) merge in LDS.
//
// CB > 0 makes the prefix-shared variant (bf16): blocks [0, shared_blocks)
// run four shared items each on the matrix cores (one per wave, with its own
// V stages; see shared_item), the rest run the tail splits as above, so the
// shared work overlaps the long private tails in one launch.  Each range has
// its own XCD-aware order.  The body stays in the kernel itself: moved into
// a device function, the compiler takes 256 + 90 registers for U = 16 and
// the kernel drops to one wave per SIMD.  The prefix-shared variant asks for
// two waves per SIMD and runs its tails with U = 8 (242 registers with two
// shared column blocks); U = 16 under that request spills.
template <typename T, int D, int G, int U, int CB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CB > 0 ? 2 : 1))) void decode_partial(
    DecodeArgs a, SharedJobs j, int32_t shared_blocks) {
  using E = Elem<T>;
  extern __shared__ float red[];
  int64_t w;
  if constexpr (CB > 0) {
    // the two V stages of each wave, as two arrays (see walk)
    __shared__ __attribute__((aligned(16))) char V0[4][32 * D * 2];
    __shared__ __attribute__((aligned(16))) char V1[4][32 * D * 2];
    // shared blocks first: interleaved with the tails (as the matrix-core
    // kernel does) the 32-head batch ran 2 % slower, its shared runs no
    // longer read side by side from L2
    const int b = (int)blockIdx.x;
    if (b < shared_blocks) {
      const int wave = (int)(threadIdx.x >> 6);
      const int64_t item = rkv::xcd_work_item(b, shared_blocks) * 4 + wave;
      if (item < (int64_t)j.n_jobs * a.hkv) shared_item<D, CB, false>(a, j, item, V0[wave], V1[wave], nullptr);
      return;
    }
    w = rkv::xcd_work_item(b - shared_blocks, (int64_t)gridDim.x - shared_blocks);
  } else {
    w = rkv::xcd_work_item(blockIdx.x, gridDim.x);
  }
  constexpr int VEC = E::kVec;
  constexpr int LPR = D / VEC;          // lanes per (slot, kv head) row
  static_assert(LPR >= 8 && LPR <= 32, "row width");
  const int HB = a.hb;                  // kv heads per workgroup
  const int RPI = 256 / (HB * LPR);     // keys per instruction (row groups)

  // item order: (head block, sub-group) outermost, then request, then split,
  // so neighbouring requests (siblings in the tree) share an XCD
  const int s = (int)(w % a.splits);
  int64_t rest = w / a.splits;
  int r = (int)(rest % a.B);
  rest /= a.B;
  const int sub = (int)(rest % a.hg);
  const int hblk = (int)(rest / a.hg);
  if (hblk * HB >= a.hkv) return;
  if (a.tail_order) {
    r = a.tail_order[r];
    if ((unsigned)r >= (unsigned)a.B) return;
  }
  const int L = min(a.seq_lens[r], a.max_seq_len);
  int k_begin, k_end, rec, nsplit;
  if (!split_span(a, r, s, L, k_begin, k_end, rec, nsplit)) return;
  const int h0 = sub * kMaxG;                   // first q head of this group within a kv group
  const int nh = min(G, a.G - h0);              // q heads handled here (<= G)

  const int tid = threadIdx.x;
  const int lr = tid % LPR;                     // lane within row
  const int hl = (tid / LPR) % HB;              // kv head within the block
  // row group; wave-uniform (scalar slot loads) when a row group spans whole waves
  const int ri = (HB * LPR >= 64) ? __builtin_amdgcn_readfirstlane(tid / (HB * LPR)) : tid / (HB * LPR);
  const int g = hblk * HB + hl;                 // kv head of this lane group
  const bool gvalid = g < a.hkv;
  const int gg = gvalid ? g : a.hkv - 1;

  // queries, pre-scaled into the log2 domain
  float qv[G][VEC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int qh = min(hh, nh - 1);
    const int64_t qoff = ((int64_t)r * a.hq + (int64_t)gg * a.G + h0 + qh) * D + lr * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) qv[hh][e] = E::load1(a.q, qoff + e) * a.scale_log2e;
  }
  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
  }

  const int32_t* row_tab = a.r2t + (int64_t)r * a.ld;
  const uint32_t P = (uint32_t)min(a.pool_slots, (int64_t)0x7fffffff);
  const uint32_t slot_bytes = (uint32_t)a.hkv * D * (uint32_t)sizeof(T);
  const char* kbase = (const char*)a.kp + ((uint64_t)gg * LPR + lr) * 16;
  const char* vbase = (const char*)a.vp + ((uint64_t)gg * LPR + lr) * 16;
  const int step = U * RPI;

  // slot indices run one iteration ahead of the K/V gathers that use them
  int32_t slots[U];
  auto fetch_slots = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) slots[u] = row_tab[min(base + u * RPI + ri, k_end - 1)];
  };
  fetch_slots(k_begin);
  for (int base = k_begin; base < k_end; base += step) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * RPI + ri;       // wave-uniform
      ok[u] = key < k_end;
      int32_t slot = slots[u];
      if ((uint32_t)slot >= P) {
        if (a.err) rkv::raise_flag(a.err);
        ok[u] = false;
        slot = 0;
      }
      const uint64_t off = (uint64_t)(uint32_t)slot * slot_bytes;
      kr[u] = load_kv<(CB > 0)>(kbase + off);
      vr[u] = load_kv<(CB > 0)>(vbase + off);
    }
    if (base + step < k_end) fetch_slots(base + step);
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      E::unpack(kr[u], kf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) t = fmaf(qv[hh][e], kf[e], t);
        sc[u][hh] = rkv::group_sum<LPR>(t);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) sc[u][hh] = -INFINITY;
        mx = fmaxf(mx, sc[u][hh]);
      }
      const float mn = fmaxf(m[hh], mx);
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - mref);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] *= alpha;
      m[hh] = mn;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = __builtin_amdgcn_exp2f(sc[u][hh] - mref);
        l[hh] += p;
        float vf[VEC];
        E::unpack(vr[u], vf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[hh][e] = fmaf(p, vf[e], acc[hh][e]);
      }
    }
  }

  // row groups (RPI > 1) merge in LDS: [row group][head in block][G][D + 2]
  if (RPI > 1) {
    if (ri > 0) {
      float* dst = red + (((ri - 1) * HB + hl) * G) * (D + 2);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[hh * (D + 2) + lr * VEC + e] = acc[hh][e];
        if (lr == 0) {
          dst[hh * (D + 2) + D] = m[hh];
          dst[hh * (D + 2) + D + 1] = l[hh];
        }
      }
    }
    __syncthreads();
    if (ri > 0) return;
    for (int rr = 1; rr < RPI; ++rr) {
      const float* src = red + (((rr - 1) * HB + hl) * G) * (D + 2);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float ab[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) ab[e] = src[hh * (D + 2) + lr * VEC + e];
        merge_state(m[hh], l[hh], acc[hh], src[hh * (D + 2) + D], src[hh * (D + 2) + D + 1], ab, VEC);
      }
    }
  }
  if (!gvalid) return;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (hh >= nh) break;
    const int head = g * a.G + h0 + hh;
    if (rec < 0) {
      const float inv = 1.f / l[hh];
      const int64_t ooff = ((int64_t)r * a.hq + head) * D + lr * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) E::store1(a.o, ooff + e, acc[hh][e] * inv);
      if (a.lse && lr == 0) a.lse[(int64_t)r * a.hq + head] = (m[hh] + log2f(l[hh])) * 0.69314718055994531f;
    } else {
      float* dst = ws_row(a, D, r, head, rec);
#pragma unroll
      for (int e = 0; e < VEC; ++e) dst[lr * VEC + e] = acc[hh][e];
      if (lr == 0) {
        dst[D] = m[hh];
        dst[D + 1] = l[hh];
      }
    }
  }
}

// One wave per workgroup with 24 KB of LDS at D = 128 (two V stages and the
// K stage): six waves per CU.  The hint caps the registers for two waves per
// SIMD.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_gqa(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char V0[32 * D * 2];
  __shared__ __attribute__((aligned(16))) char V1[32 * D * 2];
  __shared__ __attribute__((aligned(16))) char KS[32 * D * 2];
  gqa_item<D, false>(a, rkv::xcd_work_item(blockIdx.x, gridDim.x), V0, V1, KS);
}

// Prefix-shared phase 1 in one launch when the tails run on the matrix
// cores (Hq/Hkv >= 4): blocks [0, shared_blocks) run the shared jobs, the
// rest the tail splits, one wave per item, so the shared work (a few hundred
// keys per item) overlaps the long private tails instead of running,
// latency-bound, before them.  Each range has its own XCD-aware order.  Two
// waves per SIMD at most (24 KB of LDS per wave at D = 128 allows six per
// CU): the register budget of 256 per lane holds CB = 2 at D = 128 (without
// the hint the compiler takes more and runs one).
// TAIL_STREAM: the tails' V tiles come in by non-temporal DMA (their rows are
// read by no other item); chosen by the host for launches with many tail
// items (see launch_cascade_cb).
template <int D, int CB, bool TAIL_STREAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_cascade_mfma(
    DecodeArgs a, SharedJobs j, int32_t shared_blocks) {
  __shared__ __attribute__((aligned(16))) char V0[32 * D * 2];
  __shared__ __attribute__((aligned(16))) char V1[32 * D * 2];
  __shared__ __attribute__((aligned(16))) char KS[32 * D * 2];
  int64_t idx;
  if (cascade_block(blockIdx.x, shared_blocks, gridDim.x, idx)) {
    const int64_t w = rkv::xcd_work_item(idx, shared_blocks);
    if (w < (int64_t)j.n_jobs * a.hkv) shared_item<D, CB, true>(a, j, w, V0, V1, KS);
    return;
  }
  gqa_item<D, TAIL_STREAM>(a, rkv::xcd_work_item(idx, (int64_t)gridDim.x - shared_blocks), V0, V1, KS);
}

// Phase 2: one wave per (request, q head); lanes cover D.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge(DecodeArgs a) {
  using E = Elem<T>;
  const int64_t w = blockIdx.x;
  const int r = (int)(w / a.hq);
  const int head = (int)(w % a.hq);
  // partials: plain layout = this request's splits; prefix-shared layout =
  // its records (shared ranges first, then the tail splits)
  int nsplit, rec0;
  if (a.rec_indptr) {
    rec0 = a.rec_indptr[r];
    const int r1 = a.rec_indptr[r + 1];
    if (rec0 < 0 || r1 > a.n_records || !a.ws) return;     // reported by phase 1
    nsplit = r1 - rec0;
  } else {
    const int L = min(a.seq_lens[r], a.max_seq_len);
    const int chunk = split_chunk(L, a.num_splits);
    nsplit = (L + chunk - 1) / chunk;
    rec0 = 0;
  }
  if (nsplit <= 1) return;
  const int lane = threadIdx.x;
  const float* src = ws_row(a, D, r, head, rec0);
  const int64_t stride = a.rec_indptr ? (int64_t)a.hq * (D + 4) : (D + 4);
  constexpr int PER = D / 64;
  // The partials are combined in split order against their common maximum
  // M.  They are loaded UNR splits at a time, every load of a group issued
  // before any is used (an index past the last split reads the last split
  // again and is not added): a request of up to UNR splits waits one memory
  // latency for all of them, and its group also gives M.  With more splits
  // a first pass over the maxima gives M.
  constexpr int UNR = 8;
  float ms[UNR], ls[UNR], v[UNR][PER];
  auto load_group = [&](int s) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const float* p = src + (int64_t)min(s + u, nsplit - 1) * stride;
      ms[u] = p[D];
      ls[u] = p[D + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) v[u][i] = p[lane + 64 * i];
    }
  };
  float M = -INFINITY;
  if (nsplit <= UNR) {
    load_group(0);
#pragma unroll
    for (int u = 0; u < UNR; ++u) M = fmaxf(M, ms[u]);     // indices past the last repeat it
  } else {
    for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, src[(int64_t)s * stride + D]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  }
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  float lsum = 0.f;
  for (int s = 0; s < nsplit; s += UNR) {
    if (nsplit > UNR) load_group(s);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (s + u >= nsplit) break;
      const float f = (ms[u] == -INFINITY) ? 0.f : exp2f(ms[u] - M);
      lsum += ls[u] * f;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += v[u][i] * f;
    }
  }
  const float inv = 1.f / lsum;
  const int64_t ooff = ((int64_t)r * a.hq + head) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) E::store1(a.o, ooff + lane + 64 * i, acc[i] * inv);
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.hq + head] = (M + log2f(lsum)) * 0.69314718055994531f;
}

template <typename T, int D, int G>
void launch_partial(const DecodeArgs& a, int64_t grid, hipStream_t st) {
  constexpr int U = (G >= 4) ? 2 : (G >= 2 ? 4 : 16);
  constexpr int LPR = D / Elem<T>::kVec;
  const int rpi = 256 / (a.hb * LPR);
  const size_t lds = rpi > 1 ? (size_t)(rpi - 1) * a.hb * G * (D + 2) * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_partial<T, D, G, U, 0>), dim3((unsigned)grid), dim3(256), lds, st, a, SharedJobs{},
                     0);
}

template <typename T, int D>
void launch_all(const DecodeArgs& a, int64_t grid, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (a.G >= 4) {
      // grouped heads: matrix cores, one wave per (request, kv head, split)
      int64_t g2 = (int64_t)a.splits * a.B * a.hkv;
      g2 = (g2 + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
      hipLaunchKernelGGL((decode_gqa<D>), dim3((unsigned)g2), dim3(64), 0, st, a);
      hipLaunchKernelGGL((decode_merge<T, D>), dim3((unsigned)((int64_t)a.B * a.hq)), dim3(64), 0, st, a);
      return;
    }
  }
  const int g = a.G < kMaxG ? a.G : kMaxG;
  if (g <= 1) launch_partial<T, D, 1>(a, grid, st);
  else if (g <= 2) launch_partial<T, D, 2>(a, grid, st);
  else if (g <= 4) launch_partial<T, D, 4>(a, grid, st);
  else launch_partial<T, D, 8>(a, grid, st);
  hipLaunchKernelGGL((decode_merge<T, D>), dim3((unsigned)((int64_t)a.B * a.hq)), dim3(64), 0, st, a);
}

// Query columns per prefix-shared wave: two 16-column blocks at D = 128 and
// four at D = 64 fit two waves per SIMD without spills.
constexpr int kMaxSharedColumns(int d) { return d == 128 ? 32 : 64; }
constexpr int64_t kStreamTailItems = 2048;

template <int D, int CB>
void launch_cascade_cb(const DecodeArgs& a, const SharedJobs& j, hipStream_t st) {
  const int64_t items = (int64_t)j.n_jobs * a.hkv;
  if (a.G >= 4) {
    // one wave per shared item and per tail item
    const int64_t sb = (items + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
    int64_t tb = (int64_t)a.splits * a.B * a.hkv;
    tb = (tb + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
    // Non-temporal tail loads pay when the tails fill the chip (c4, 64/8
    // heads, 4096 tail slots: 240 -> 230 us) and cost on small, latency-bound
    // launches (one GPU's 8/1 heads of c4, 512 slots: 37 -> 42 us); the
    // threshold is the chip's resident waves of this kernel (256 CUs x 8).
    if (tb >= kStreamTailItems)
      hipLaunchKernelGGL((decode_cascade_mfma<D, CB, true>), dim3((unsigned)(sb + tb)), dim3(64), 0, st, a, j,
                         (int32_t)sb);
    else
      hipLaunchKernelGGL((decode_cascade_mfma<D, CB, false>), dim3((unsigned)(sb + tb)), dim3(64), 0, st, a, j,
                         (int32_t)sb);
    return;
  }
  // four shared items per block; tail blocks as the vector kernel's grid
  const int64_t sb = ((items + 3) / 4 + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
  int64_t tb = (int64_t)a.splits * a.B * ((a.hkv + a.hb - 1) / a.hb) * a.hg;
  tb = (tb + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
  constexpr int LPR = D / 8;
  const int rpi = 256 / (a.hb * LPR);
  const int g = a.G < kMaxG ? a.G : kMaxG;
  auto go = [&](auto gtag) {
    constexpr int GT = decltype(gtag)::value;
    constexpr int U = (GT >= 4) ? 2 : (GT >= 2 ? 4 : 8);
    const size_t lds = rpi > 1 ? (size_t)(rpi - 1) * a.hb * GT * (D + 2) * sizeof(float) : 0;
    hipLaunchKernelGGL((decode_partial<uint16_t, D, GT, U, CB>), dim3((unsigned)(sb + tb)), dim3(256), lds, st, a,
                       j, (int32_t)sb);
  };
  if (g <= 1) go(std::integral_constant<int, 1>{});
  else if (g <= 2) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 4>{});
}

template <int D>
void launch_cascade(const DecodeArgs& a, const SharedJobs& j, int cb, hipStream_t st) {
  if (cb <= 1) launch_cascade_cb<D, 1>(a, j, st);
  else if (cb <= 2 || D == 128) launch_cascade_cb<D, 2>(a, j, st);
  else if constexpr (D == 64) launch_cascade_cb<D, 4>(a, j, st);
  hipLaunchKernelGGL((decode_merge<uint16_t, D>), dim3((unsigned)((int64_t)a.B * a.hq)), dim3(64), 0, st, a);
}

// kv heads per workgroup of the vector kernel (a power of two, at most 4):
// a key's rows for them are one contiguous run of the slot, and
// 256 / (hb * lpr) keys are read per instruction.  Measured on the 32-head
// decode batches: 4 heads (1 KB runs, 4 keys per instruction) beat 16 (4 KB
// runs, 1 key) by 5-8 %, and 2 or 1 heads; more distinct slots in flight
// spread better over HBM.
int heads_per_block(int d, int dtype, int hkv) {
  const int lpr = d * (dtype == RKV_BF16 ? 2 : 4) / 16;
  int hb = 256 / lpr;
  if (hb > 4) hb = 4;
  while (hb > 1 && hb / 2 >= hkv) hb /= 2;
  return hb;
}

int64_t splits_extent(int32_t max_seq_len, int32_t num_splits) {
  if (num_splits > 0) return num_splits;
  return ((int64_t)max_seq_len + kChunk - 1) / kChunk;
}

}  // namespace

extern "C" size_t rkv_attn_decode_workspace_bytes(int32_t B, int32_t hq, int32_t d, int32_t max_seq_len,
                                                  int32_t num_splits) {
  if (B < 0 || hq < 1 || (d != 64 && d != 128) || max_seq_len < 1 || num_splits < 0) return 0;
  const int64_t S = splits_extent(max_seq_len, num_splits);
  return (size_t)B * hq * S * (d + 4) * sizeof(float);
}

namespace {

// Plain split-KV decode for both entry points: `workspace` holds the split
// partials, `flag` (nullable) the debug error flag.
int decode_launch(const char* who, const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                  const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens, int32_t B,
                  int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t dtype,
                  int32_t num_splits, void* workspace, int64_t pool_slots, int* flag, hipStream_t st) {
  const int64_t S = splits_extent(max_seq_len, num_splits);
  DecodeArgs a;
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.o = o; a.lse = lse;
  a.r2t = req_to_token; a.ld = ld; a.seq_lens = seq_lens;
  a.B = B; a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
  a.hg = (a.G + kMaxG - 1) / kMaxG;
  a.max_seq_len = max_seq_len;
  a.hb = heads_per_block(d, dtype, hkv);
  a.splits = (int32_t)S;
  a.num_splits = num_splits;
  a.scale_log2e = sm_scale * 1.4426950408889634f;
  a.pool_slots = pool_slots;
  a.ws = (float*)workspace;
  a.rec_indptr = nullptr;
  a.tail_begin = nullptr;
  a.n_records = 0;
  a.tail_chunk = 0;
  a.tail_order = nullptr;
  a.err = flag;
  int64_t grid = (int64_t)S * B * ((hkv + a.hb - 1) / a.hb) * a.hg;
  grid = (grid + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
  if (grid > 0x7fffffff) return rkv::fail(RKV_ENOTSUP, std::string(who) + ": grid too large");
  if (dtype == RKV_BF16) {
    if (d == 128) launch_all<uint16_t, 128>(a, grid, st); else launch_all<uint16_t, 64>(a, grid, st);
  } else {
    if (d == 128) launch_all<float, 128>(a, grid, st); else launch_all<float, 64>(a, grid, st);
  }
  return rkv::finish_launch(who, st, a.err);
}

// Argument checks shared by both entry points (everything but the workspace).
int decode_check(const char* who, const void* q, const void* k_pool, const void* v_pool, const void* o,
                 const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens, int32_t B,
                 int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t dtype,
                 int32_t num_splits, int64_t pool_slots) {
  const std::string w(who);
  if (B < 0 || hq < 1 || hkv < 1 || max_seq_len < 1 || ld < max_seq_len || pool_slots < 1 ||
      num_splits < 0 || !(sm_scale > 0.f))
    return rkv::fail(RKV_EINVAL, w + ": bad sizes");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, w + ": dtype");
  if (d != 64 && d != 128) return rkv::fail(RKV_ENOTSUP, w + ": head_dim must be 64 or 128");
  if (hq % hkv != 0 || hq / hkv > 16) return rkv::fail(RKV_ENOTSUP, w + ": Hq/Hkv must be an integer <= 16");
  if (B == 0) return RKV_OK;
  if (!q || !k_pool || !v_pool || !o || !req_to_token || !seq_lens) return rkv::fail(RKV_EINVAL, w + ": NULL pointer");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o;
  if (al & 15) return rkv::fail(RKV_EINVAL, w + ": tensors must be 16-byte aligned");
  return RKV_OK;
}

// ---- scratch of the decode entry point that allocates nothing
// A file-scope device array, one per GPU the library runs on, held until the
// process ends; its device address (and that of a debug flag beside it) is
// taken once per device with hipGetSymbolAddress, with the device current,
// and kept.  In host code `scratch` names a host-side stand-in, never the
// device memory: only the kept pointers are passed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
__device__ int scratch_flag;

struct ScratchPtrs {
  void* ws = nullptr;
  int* flag = nullptr;
};
std::mutex g_scratch_mu;
ScratchPtrs g_scratch[64];

int scratch_ptrs(ScratchPtrs* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return rkv::fail(RKV_EHIP, "rkv_attn_decode_noalloc: hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchPtrs& s = g_scratch[dev];
  if (!s.ws) {
    void* ws = nullptr;
    void* flag = nullptr;
    if (hipGetSymbolAddress(&ws, HIP_SYMBOL(scratch)) != hipSuccess || !ws)
      return rkv::fail(RKV_EHIP, "rkv_attn_decode_noalloc: hipGetSymbolAddress(scratch) failed");
    if (hipGetSymbolAddress(&flag, HIP_SYMBOL(scratch_flag)) != hipSuccess || !flag)
      return rkv::fail(RKV_EHIP, "rkv_attn_decode_noalloc: hipGetSymbolAddress(scratch_flag) failed");
    s.ws = ws;
    s.flag = (int*)flag;
  }
  *out = s;
  return RKV_OK;
}

}  // namespace

extern "C" int rkv_attn_decode(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                               const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                               int32_t B, int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d,
                               float sm_scale, int32_t dtype, int32_t num_splits, void* workspace,
                               size_t ws_bytes, int64_t pool_slots, void* stream) {
  rkv::clear_error();
  const char* who = "rkv_attn_decode";
  if (int rc = decode_check(who, q, k_pool, v_pool, o, req_to_token, ld, seq_lens, B, max_seq_len, hq, hkv, d,
                            sm_scale, dtype, num_splits, pool_slots))
    return rc;
  if (B == 0) return RKV_OK;
  const size_t need = rkv_attn_decode_workspace_bytes(B, hq, d, max_seq_len, num_splits);
  const int64_t S = splits_extent(max_seq_len, num_splits);
  if (S > 1 && (!workspace || ws_bytes < need || ((uintptr_t)workspace & 15)))
    return rkv::fail(RKV_EINVAL, "rkv_attn_decode: workspace missing or too small");
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  return decode_launch(who, q, k_pool, v_pool, o, lse, req_to_token, ld, seq_lens, B, max_seq_len, hq, hkv, d,
                       sm_scale, dtype, num_splits, workspace, pool_slots, flag, (hipStream_t)stream);
}

extern "C" int rkv_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                                       const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                                       int32_t B, int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d,
                                       float sm_scale, int32_t dtype, int32_t num_splits, int64_t pool_slots,
                                       void* stream) {
  rkv::clear_error();
  const char* who = "rkv_attn_decode_noalloc";
  if (int rc = decode_check(who, q, k_pool, v_pool, o, req_to_token, ld, seq_lens, B, max_seq_len, hq, hkv, d,
                            sm_scale, dtype, num_splits, pool_slots))
    return rc;
  if (B == 0) return RKV_OK;
  const size_t need = rkv_attn_decode_workspace_bytes(B, hq, d, max_seq_len, num_splits);
  if (need > kScratchBytes)
    return rkv::fail(RKV_EINVAL, "rkv_attn_decode_noalloc: these sizes need " + std::to_string(need) +
                                     " bytes of split partials, more than the " + std::to_string(kScratchBytes) +
                                     " this entry point holds; use rkv_attn_decode with a workspace");
  ScratchPtrs sp;
  if (int rc = scratch_ptrs(&sp)) return rc;
  // the partials are written before they are read, so nothing needs clearing;
  // the debug flag starts at zero and finish_launch clears it after a report
  return decode_launch(who, q, k_pool, v_pool, o, lse, req_to_token, ld, seq_lens, B, max_seq_len, hq, hkv, d,
                       sm_scale, dtype, num_splits, sp.ws, pool_slots, rkv::debug_mode() ? sp.flag : nullptr,
                       (hipStream_t)stream);
}

extern "C" size_t rkv_attn_decode_cascade_workspace_bytes(int64_t n_records, int32_t hq, int32_t d) {
  if (n_records < 0 || hq < 1 || (d != 64 && d != 128)) return 0;
  return (size_t)n_records * hq * (d + 4) * sizeof(float);
}

extern "C" int rkv_attn_decode_cascade(const void* q, const void* k_pool, const void* v_pool, void* o,
                                       float* lse, const int32_t* req_to_token, int64_t ld,
                                       const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t hq,
                                       int32_t hkv, int32_t d, float sm_scale, int32_t dtype,
                                       const int32_t* perm, const int32_t* rec_indptr,
                                       const int32_t* tail_begin, const int32_t* jobs, int64_t n_jobs,
                                       const int32_t* tail_order, int32_t max_members, int32_t tail_chunk,
                                       int32_t tail_splits,
                                       int64_t n_records, void* workspace, size_t ws_bytes,
                                       int64_t pool_slots, void* stream) {
  rkv::clear_error();
  if (B < 0 || hq < 1 || hkv < 1 || max_seq_len < 1 || ld < max_seq_len || pool_slots < 1 ||
      !(sm_scale > 0.f) || n_jobs < 0 || max_members < 1 || tail_chunk < 1 || tail_splits < 0 ||
      n_records < 0 || n_records > 0x7fffffff || n_jobs > 0x7fffffff)
    return rkv::fail(RKV_EINVAL, "rkv_attn_decode_cascade: bad sizes");
  if (dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, "rkv_attn_decode_cascade: bf16 only");
  if (d != 64 && d != 128) return rkv::fail(RKV_ENOTSUP, "rkv_attn_decode_cascade: head_dim must be 64 or 128");
  if (hq % hkv != 0 || hq / hkv > 16)
    return rkv::fail(RKV_ENOTSUP, "rkv_attn_decode_cascade: Hq/Hkv must be an integer <= 16");
  const int G = hq / hkv;
  if ((int64_t)max_members * G > kMaxSharedColumns(d))
    return rkv::fail(RKV_ENOTSUP, "rkv_attn_decode_cascade: max_members * Hq/Hkv must be <= " +
                                      std::to_string(kMaxSharedColumns(d)));
  if (B == 0) return RKV_OK;
  if (!q || !k_pool || !v_pool || !o || !req_to_token || !seq_lens || !perm || !rec_indptr || !tail_begin ||
      (n_jobs > 0 && !jobs))
    return rkv::fail(RKV_EINVAL, "rkv_attn_decode_cascade: NULL pointer");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o;
  if (al & 15) return rkv::fail(RKV_EINVAL, "rkv_attn_decode_cascade: tensors must be 16-byte aligned");
  const size_t need = rkv_attn_decode_cascade_workspace_bytes(n_records, hq, d);
  if ((n_records > B || n_jobs > 0) && (!workspace || ws_bytes < need || ((uintptr_t)workspace & 15)))
    return rkv::fail(RKV_EINVAL, "rkv_attn_decode_cascade: workspace missing or too small");
  if (tail_splits < 1) return rkv::fail(RKV_EINVAL, "rkv_attn_decode_cascade: tail_splits must be >= 1");
  DecodeArgs a;
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.o = o; a.lse = lse;
  a.r2t = req_to_token; a.ld = ld; a.seq_lens = seq_lens;
  a.B = B; a.hq = hq; a.hkv = hkv; a.G = G;
  a.hg = (G + kMaxG - 1) / kMaxG;
  a.max_seq_len = max_seq_len;
  a.hb = heads_per_block(d, dtype, hkv);
  a.splits = tail_splits;
  a.num_splits = 0;
  a.scale_log2e = sm_scale * 1.4426950408889634f;
  a.pool_slots = pool_slots;
  a.ws = (float*)workspace;
  a.rec_indptr = rec_indptr;
  a.tail_begin = tail_begin;
  a.n_records = (int32_t)n_records;
  a.tail_chunk = tail_chunk;
  a.tail_order = tail_order;
  if (int rc = rkv::debug_flag(&a.err)) return rc;
  SharedJobs j;
  j.jobs = jobs;
  j.perm = perm;
  j.n_jobs = (int32_t)n_jobs;
  j.max_members = max_members;
  const int cb = (max_members * G + 15) / 16;
  if ((int64_t)n_jobs * hkv + (int64_t)tail_splits * B * hkv + 64 > 0x7fffffff)
    return rkv::fail(RKV_ENOTSUP, "rkv_attn_decode_cascade: grid too large");
  hipStream_t st = (hipStream_t)stream;
  if (d == 128) launch_cascade<128>(a, j, cb, st); else launch_cascade<64>(a, j, cb, st);
  return rkv::finish_launch("rkv_attn_decode_cascade", st, a.err);
}
