// Extend (prefill) attention over a cached prefix in the token-slot pool.
//
// With RadixAttention a request reuses the KV of its longest cached prefix and
// only its new tokens are computed (unite.ai, "SGLang: Efficient Execution of
// Structured Language Model Programs", walkthrough Step 3 in section "SGLang:
// Modelo de programacion y metodologia").  Their queries attend causally to
// the cached prefix plus their own new keys, all gathered from the pool through
// the request's req_to_token row.
//
// bf16 path (gfx950 MFMA, v_mfma_f32_16x16x32_bf16):
//   * work item = (kv head g, request r, tile of 128 query rows); a query row
//     is a (new token j, head-in-group hh) pair, row = j*G + hh, so grouped
//     heads share every K/V tile they read.  Work items are ordered kv-head
//     major and dealt to XCDs in contiguous ranges (requests sharing a prefix
//     read the same rows of one head from one L2).
//   * 4 waves x 32 rows.  Each wave keeps its Q (two 16-row blocks) in
//     registers for the whole key loop.
//   * K/V tiles of 64 keys are gathered row by row (16-byte loads, one slot
//     lookup per row) into registers one tile ahead, then written to LDS: K
//     as rows, V transposed (d-major) so both MFMA operands are single 16-byte
//     LDS reads.
//   * S^T = K Q^T, so a lane owns one query: its row max / row sum are lane
//     values plus a 4-lane exchange.  K rows are placed in LDS in an order
//     that makes the S^T accumulator of a lane hold 8 consecutive keys, which
//     is exactly the bf16 B operand of O^T += V^T P^T: the softmax weights
//     never leave registers.
//   * fp32 online softmax in the log2 domain (exp2 with log2(e) folded into
//     the scale); weights rounded to bf16 for PV; o rounded to bf16 (RNE).
//   * causal masking only on tiles that reach past a wave's first query.
// fp32 path: one wave per (query row, head), fp32 FMA throughout.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "device.h"
#include "rkv.h"
#include "rkv_internal.h"

namespace {

using rkv::bf16x8;
using rkv::f32x4;

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile

struct ExtendArgs {
  const void* q;
  const void* kp;
  const void* vp;
  void* o;
  float* lse;
  const int32_t* r2t;
  int64_t ld;
  const int32_t* qo_indptr;
  const int32_t* prefix_lens;
  int32_t B, hq, hkv, G;
  float scale_log2e;
  int64_t pool_slots;
  int64_t tiles_bound;      // work items per kv head
  int64_t total_new;        // q rows; rows at or past it are never read
  int* err;
};

// Finds which request owns global tile index tg (tiles of BM rows, counted
// request by request).  Wave-parallel prefix sum over the requests; the
// result is uniform across the wave.  Returns false when tg is past the end.
__device__ bool locate_tile(const ExtendArgs& a, int64_t tg, int& r, int& t) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int i = base + lane;
    int c = 0;
    if (i < a.B) {
      const int64_t n = (int64_t)a.qo_indptr[i + 1] - a.qo_indptr[i];
      c = (int)((n * a.G + BM - 1) / BM);
    }
    int s = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    const int tot = __shfl(s, 63);
    if (tg < acc + tot) {
      const unsigned long long mask = __ballot(acc + s > tg);
      const int first = __ffsll((long long)mask) - 1;
      const int s_first = __shfl(s, first);
      const int c_first = __shfl(c, first);
      r = base + first;
      t = (int)(tg - (acc + s_first - c_first));
      return true;
    }
    acc += tot;
  }
  return false;
}

// Physical 16-byte chunk of logical chunk `ch` (8 keys) in V^T row d.
__device__ __forceinline__ int vt_chunk(int ch, int d) { return ch ^ ((d ^ (d >> 3)) & 7); }

// Key held by K LDS row rho of a 64-key tile.  Within each 32-key chunk,
// rows 0..15 hold keys 8*(i/4) + i%4 and rows 16..31 hold 8*(i/4) + 4 + i%4,
// so MFMA block kb = 2c + half gives lane group gq the keys
// c*32 + 8*gq + 4*half + [0..3]: two blocks together = 8 consecutive keys.
__device__ __forceinline__ int key_of_row(int rho) {
  const int c = rho >> 5, rr = rho & 31, half = rr >> 4, i = rr & 15;
  return c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
}

// Softmax weights are kept relative to a per-row reference maximum that is
// only raised when a tile's maximum exceeds it by more than 2^8 (log2 units):
// weights stay <= 256, harmless in fp32 and bf16, and the O accumulators are
// rescaled only on those rare tiles instead of on every tile.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
__global__ __launch_bounds__(256, 2) void extend_bf16(ExtendArgs a) {
  // LDS layouts, chosen with a bank-conflict probe on gfx950: a 16-row
  // ds_read_b128 pattern is conflict-free when the row pitch is 2 mod 4
  // 16-byte chunks (K: D + 16 elements), or at a 128-byte pitch when the
  // chunk index is XOR-swizzled by the row (V^T, see vt_chunk)
  constexpr int KP = D + 16;         // K row pitch in LDS (elements)
  constexpr int VP = BN;             // V^T row pitch in LDS (elements)
  constexpr int KSTEPS = D / 32;     // QK contraction steps
  constexpr int DBLK = D / 16;       // PV output blocks
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int KROWS = 256 / CPR;   // K rows loaded per pass
  constexpr int KPASS = BN / KROWS;  // passes per tile
  constexpr int KPT = BN * CPR / 256;  // V keys per thread (transposed group)
  static_assert(KPT == 2 || KPT == 4, "V transpose group");

  // two stages: the next tile is written while the current one is read;
  // slot indices run one more tile ahead in three small stages, so a K/V
  // gather never waits on a global index load
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VP];
  __shared__ __attribute__((aligned(16))) int32_t Sl[3][BN];

  const int64_t w = rkv::xcd_work_item(blockIdx.x, gridDim.x);
  const int g = (int)(w / a.tiles_bound);
  const int64_t tg = w % a.tiles_bound;
  if (g >= a.hkv) return;
  int r = 0, t = 0;
  if (!locate_tile(a, tg, r, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int q0 = a.qo_indptr[r];
  const int n = a.qo_indptr[r + 1] - q0;
  const int p = a.prefix_lens[r];
  const int G = a.G;
  const int rows_total = n * G;
  const int row0 = t * BM;
  const int row_last = min(row0 + BM, rows_total) - 1;
  // keys never reach past the table row, whatever the lengths say
  const int kv_end = (int)min((int64_t)p + row_last / G + 1, a.ld);
  const int ntiles = (kv_end + BN - 1) / BN;
  // tiles before this one are fully visible to every row of the workgroup
  const int first_mask_tile = min(ntiles, (p + row0 / G) / BN);

  // ---- queries of this wave: rows row0 + wave*32 + qb*16 + l16
  bf16x8 qreg[2][KSTEPS];
  int qlim[2], qhead[2], qtok[2];
  bool qvalid[2];
  const uint16_t* qbase = (const uint16_t*)a.q;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = row0 + wave * 32 + qb * 16 + l16;
    qvalid[qb] = row < rows_total && (int64_t)q0 + row / G < a.total_new && p + row / G < kv_end;
    const int j = qvalid[qb] ? row / G : 0;
    const int hh = qvalid[qb] ? row % G : 0;
    qtok[qb] = q0 + j;
    qhead[qb] = g * G + hh;
    // last visible key, relative to the first key this lane holds in a tile
    qlim[qb] = (qvalid[qb] ? p + j : kv_end - 1) - 8 * gq;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid[qb])
        v = *(const uint4*)(qbase + ((int64_t)qtok[qb] * a.hq + qhead[qb]) * D + s * 32 + gq * 8);
      qreg[qb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[2][DBLK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  // row sums of the bf16 weights, accumulated on the MFMA (all-ones A
  // operand) so that numerator and denominator use the same rounded weights;
  // every element of lacc[qb] holds the lane's full row sum
  f32x4 lacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const float c = a.scale_log2e;

  // ---- tile loader: every gathered row index is clamped into [0, kv_end)
  //      and every slot into [0, pool_slots), so no access leaves the table or
  //      the pool; keys past kv_end are masked by the causal test.
  const int32_t* row_tab = a.r2t + (int64_t)r * a.ld;
  const char* kp = (const char*)a.kp;
  const char* vp = (const char*)a.vp;
  constexpr int ROWB = D * 2;          // bytes of one (slot, kv head) row
  const int kc = tid % CPR;            // K chunk (16 bytes) this thread moves
  const int krow = tid / CPR;          // first K LDS row this thread moves
  // V: each 16-lane group takes 8 d groups x 2 key groups, so both its
  // global loads (8 lanes = one 128-byte line) and its transposed LDS writes
  // (8 rows x 2 halves of a chunk) are conflict-free
  const int vrest = tid >> 4;
  const int vdg = (lane & 7) + 8 * (vrest % (CPR / 8));           // 8-wide d group
  const int vkq = ((lane >> 3) & 1) + 2 * (vrest / (CPR / 8));    // group of KPT keys
  const uint32_t P = (uint32_t)min(a.pool_slots, (int64_t)0x7fffffff);

  // slot of a key of this request, clamped into the table and the pool
  auto fetch_slot = [&](int key) -> int32_t {
    int32_t slot = row_tab[min(key, kv_end - 1)];
    if ((uint32_t)slot >= P) {
      if (a.err) rkv::raise_flag(a.err);
      slot = 0;
    }
    return slot;
  };
  // per-thread bases (kv head g, this thread's 16-byte chunk): a gathered
  // row is then base + slot * slot_bytes, one 64-bit multiply-add
  const uint32_t slot_bytes = (uint32_t)a.hkv * ROWB;
  const char* kbase = kp + (uint64_t)g * ROWB + kc * 16;
  const char* vbase = vp + (uint64_t)g * ROWB + vdg * 16;
  int krel[KPASS];
#pragma unroll
  for (int i = 0; i < KPASS; ++i) krel[i] = key_of_row(krow + i * KROWS);
  auto gather = [&](const char* base, int32_t slot) -> uint4 {
    return *(const uint4*)(base + (uint64_t)(uint32_t)slot * slot_bytes);
  };
  uint4 kreg[KPASS], vreg[KPT];
  auto load_tile = [&](int tile) {
    const int32_t* sl = Sl[tile % 3];
#pragma unroll
    for (int i = 0; i < KPASS; ++i) kreg[i] = gather(kbase, sl[krel[i]]);
#pragma unroll
    for (int u = 0; u < KPT; ++u) vreg[u] = gather(vbase, sl[vkq * KPT + u]);
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = Ks[buf];
    uint16_t* vt = Vt[buf];
#pragma unroll
    for (int i = 0; i < KPASS; ++i)
      *(uint4*)(ks + (krow + i * KROWS) * KP + kc * 8) = kreg[i];
    // V transposed: element (d, key) at vt[d*VP + vt_chunk(key/8, d)*8 + key%8]
    const int key0 = vkq * KPT;
    const int wswz = ((key0 >> 3) ^ vdg) & 7;
    const uint32_t* w32[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) w32[u] = (const uint32_t*)&vreg[u];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int d = vdg * 8 + e2 * 2 + hi;
        // vt_chunk(key0/8, d) with d%8 = 2*e2 + hi and d/8 = vdg
        const int phys = (wswz ^ (e2 * 2 + hi)) * 8 + (key0 & 7);
        uint32_t pk[2];
#pragma unroll
        for (int u = 0; u < KPT; u += 2) {
          const uint32_t x0 = w32[u][e2], x1 = w32[u + 1][e2];
          pk[u / 2] = hi ? __builtin_amdgcn_perm(x1, x0, 0x07060302u) : __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        }
        if constexpr (KPT == 4)
          *(uint2*)(vt + d * VP + phys) = make_uint2(pk[0], pk[1]);
        else
          *(uint32_t*)(vt + d * VP + phys) = pk[0];
      }
    }
  };

  const int rswz = ((l16 & 7) ^ (l16 >> 3)) & 7;   // V^T read swizzle of this lane's rows
  // one 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  auto tile_body = [&](int tile, int buf, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* ks = Ks[buf];
    const uint16_t* vt = Vt[buf];
    f32x4 sacc[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const uint4*)(ks + (kb * 16 + l16) * KP + s * 32 + gq * 8));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[qb][s], sacc[qb][kb], 0, 0, 0);
      }
    }
    // lane owns query l16 of each block and keys
    //   tile*64 + 32*(kb/2) + 8*gq + 4*(kb%2) + i   (block kb, element i)
    bf16x8 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (MASK) {
        const int lim = qlim[qb] - tile * BN;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (32 * (kb >> 1) + 4 * (kb & 1) + i > lim) sacc[qb][kb][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(sacc[qb][0][0], sacc[qb][0][1]), fmaxf(sacc[qb][0][2], sacc[qb][0][3]));
#pragma unroll
      for (int kb = 1; kb < 4; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(sacc[qb][kb][0], sacc[qb][kb][1]), fmaxf(sacc[qb][kb][2], sacc[qb][kb][3])));
      mx = rkv::max_xor16(mx);
      mx = rkv::max_xor32(mx);
      const float mt = mx * c;
      if (__builtin_amdgcn_ballot_w64(mt > mref[qb] + kRescaleThreshold)) {
        const float mn = fmaxf(mref[qb], mt);
        const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
        mref[qb] = mn;
        lacc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[qb][db] *= alpha;
      }
      const float m = mref[qb];
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][i], c, -m));
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        uint4 u;
        u.x = rkv::pack_bf16x2(pv[2 * cc][0], pv[2 * cc][1]);
        u.y = rkv::pack_bf16x2(pv[2 * cc][2], pv[2 * cc][3]);
        u.z = rkv::pack_bf16x2(pv[2 * cc + 1][0], pv[2 * cc + 1][1]);
        u.w = rkv::pack_bf16x2(pv[2 * cc + 1][2], pv[2 * cc + 1][3]);
        pb[qb][cc] = __builtin_bit_cast(bf16x8, u);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb][cc], lacc[qb], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d = db * 16 + l16;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        // vt_chunk(cc*4 + gq, d) with d%8 = l16%8 and d/8 = 2*db + l16/8
        const int phys = ((cc * 4 + gq) ^ rswz ^ ((2 * db) & 7)) * 8;
        const bf16x8 va = __builtin_bit_cast(bf16x8, *(const uint4*)(vt + d * VP + phys));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qb][cc], oacc[qb][db], 0, 0, 0);
      }
    }
  };

  // prologue: slots of tiles 0 and 1, then tile 0 itself
  if (tid < BN) Sl[0][tid] = fetch_slot(tid);
  else if (tid < 2 * BN && ntiles > 1) Sl[1][tid - BN] = fetch_slot(tid);
  __syncthreads();
  load_tile(0);
  store_tile(0);
  __syncthreads();
  // iteration t: gather tile t+1 and the slots of tile t+2 while computing
  // tile t; then publish both and meet at the barrier
  for (int tile = 0; tile < ntiles; ++tile) {
    const bool more = tile + 1 < ntiles;
    const bool more2 = tile + 2 < ntiles;
    if (more) load_tile(tile + 1);
    int32_t sreg = 0;
    if (more2 && tid < BN) sreg = fetch_slot((tile + 2) * BN + tid);
    if (tile < first_mask_tile)
      tile_body(tile, tile & 1, std::false_type{});
    else
      tile_body(tile, tile & 1, std::true_type{});
    if (more) store_tile((tile + 1) & 1);
    if (more2 && tid < BN) Sl[(tile + 2) % 3][tid] = sreg;
    __syncthreads();
  }

  // ---- epilogue: lane holds o[query l16][d = db*16 + 4*gq + 0..3]
  uint16_t* obase = (uint16_t*)a.o;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = lacc[qb][0];
    if (!qvalid[qb]) continue;
    const float inv = 1.f / lsum;
    uint16_t* orow = obase + ((int64_t)qtok[qb] * a.hq + qhead[qb]) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const f32x4 v = oacc[qb][db];
      *(uint2*)(orow + db * 16 + 4 * gq) =
          make_uint2(rkv::pack_bf16x2(v[0] * inv, v[1] * inv), rkv::pack_bf16x2(v[2] * inv, v[3] * inv));
    }
    if (a.lse && gq == 0)
      a.lse[(int64_t)qtok[qb] * a.hq + qhead[qb]] = (mref[qb] + log2f(lsum)) * 0.69314718055994531f;
  }
}

// fp32: one wave per (query row, q head).  Lanes split D; keys are walked in
// order with an fp32 online softmax.
template <int D>
__global__ __launch_bounds__(256) void extend_f32(ExtendArgs a) {
  constexpr int PER = D / 64;
  const int64_t gw = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;  // global wave
  const int lane = threadIdx.x & 63;
  const int64_t T = a.qo_indptr[a.B];
  if (gw >= T * a.hq) return;
  const int64_t row = gw / a.hq;
  const int head = (int)(gw % a.hq);
  // request owning this row: binary search over qo_indptr
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qo_indptr[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int j = (int)(row - a.qo_indptr[r]);
  const int c = (int)min((int64_t)a.prefix_lens[r] + j, a.ld - 1);
  const int g = head / a.G;
  const float* qf = (const float*)a.q + (row * a.hq + head) * D;
  float qv[PER], acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    qv[i] = qf[lane + 64 * i] * a.scale_log2e;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int32_t* row_tab = a.r2t + (int64_t)r * a.ld;
  for (int key = 0; key <= c; ++key) {
    const int32_t slot = row_tab[key];
    if (slot < 0 || (int64_t)slot >= a.pool_slots) {
      rkv::raise_flag(a.err);
      continue;
    }
    const int64_t off = ((int64_t)slot * a.hkv + g) * D;
    const float* kf = (const float*)a.kp + off;
    const float* vf = (const float*)a.vp + off;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) s = fmaf(qv[i], kf[lane + 64 * i], s);
    s = rkv::group_sum<64>(s);
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn);
    const float pw = exp2f(s - mn);
    l = l * alpha + pw;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = fmaf(pw, vf[lane + 64 * i], acc[i] * alpha);
    m = mn;
  }
  float* of = (float*)a.o + (row * a.hq + head) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < PER; ++i) of[lane + 64 * i] = acc[i] * inv;
  if (a.lse && lane == 0) a.lse[row * a.hq + head] = (m + log2f(l)) * 0.69314718055994531f;
}

}  // namespace

extern "C" int rkv_attn_extend(const void* q, const void* k_pool, const void* v_pool, void* o, float* lse,
                               const int32_t* req_to_token, int64_t ld, const int32_t* qo_indptr,
                               const int32_t* prefix_lens, int32_t B, int64_t total_new,
                               int32_t max_new, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                               int32_t dtype, int64_t pool_slots, void* stream) {
  rkv::clear_error();
  if (B < 0 || total_new < 0 || max_new < 0 || hq < 1 || hkv < 1 || ld < 1 || pool_slots < 1 ||
      !(sm_scale > 0.f))
    return rkv::fail(RKV_EINVAL, "rkv_attn_extend: bad sizes");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: dtype");
  if (d != 64 && d != 128) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: head_dim must be 64 or 128");
  if (hq % hkv != 0 || hq / hkv > 16) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: Hq/Hkv must be an integer <= 16");
  if (B == 0 || total_new == 0) return RKV_OK;
  if (!q || !k_pool || !v_pool || !o || !req_to_token || !qo_indptr || !prefix_lens)
    return rkv::fail(RKV_EINVAL, "rkv_attn_extend: NULL pointer");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o;
  if (al & 15) return rkv::fail(RKV_EINVAL, "rkv_attn_extend: tensors must be 16-byte aligned");
  ExtendArgs a;
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.o = o; a.lse = lse;
  a.r2t = req_to_token; a.ld = ld; a.qo_indptr = qo_indptr; a.prefix_lens = prefix_lens;
  a.B = B; a.hq = hq; a.hkv = hkv; a.G = hq / hkv;
  a.scale_log2e = sm_scale * 1.4426950408889634f;
  a.pool_slots = pool_slots;
  a.total_new = total_new;
  if (int rc = rkv::debug_flag(&a.err)) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == RKV_BF16) {
    // tiles per kv head: exact for equal lengths, bounded for ragged batches
    const int64_t per_req = ((int64_t)max_new * a.G + BM - 1) / BM;
    const int64_t ragged = (total_new * a.G + BM - 1) / BM + B;
    a.tiles_bound = per_req * B < ragged ? per_req * B : ragged;
    int64_t grid = a.tiles_bound * hkv;
    grid = (grid + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
    if (grid > 0x7fffffff) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: grid too large");
    if (d == 128)
      hipLaunchKernelGGL(extend_bf16<128>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(extend_bf16<64>, dim3((unsigned)grid), dim3(256), 0, st, a);
  } else {
    a.tiles_bound = 0;
    const int64_t waves = total_new * hq;
    const int64_t grid = (waves + 3) / 4;
    if (grid > 0x7fffffff) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: grid too large");
    if (d == 128)
      hipLaunchKernelGGL(extend_f32<128>, dim3((unsigned)grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(extend_f32<64>, dim3((unsigned)grid), dim3(256), 0, st, a);
  }
  return rkv::finish_launch("rkv_attn_extend", st, a.err);
}
