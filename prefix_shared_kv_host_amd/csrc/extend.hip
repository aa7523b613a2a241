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
//   * 4 waves x 32 rows per workgroup, two workgroups per CU: two waves per
//     SIMD, each keeping its Q (two 16-row blocks) in registers.  Within a
//     wave the key loop is software pipelined by hand, so that a stall of one
//     wave does not have to be covered by the other: the softmax runs on
//     32-key half tiles, and each half tile is one block of fenced stages in
//     which the QK MFMAs of the next half tile sit beside the exponentials of
//     this one, and its PV MFMAs beside the row maxima of the next.
//   * K/V tiles of 64 keys go global -> LDS by 16-byte LDS DMA
//     (global_load_lds), one slot lookup per row.  The K tiles are shifted
//     half a tile against V (K tile t holds keys 64t-32 .. 64t+31), so QK
//     runs one half tile ahead of PV while an iteration still consumes one K
//     and one V tile.  K runs two tiles ahead, V one; the slot indices reach
//     LDS by 4-byte DMA straight from the table, one more tile ahead.  The
//     gathers of a tile are spread over the first QK stages of the
//     iteration before.  K is read as 16-byte rows (ds_read_b128); V stays row-major
//     and the V^T operand comes from transposed reads (ds_read_b64_tr_b16).
//     Gathered slots are clamped into the pool; a separate check kernel,
//     launched only in debug mode, reports table entries outside it.
//   * S^T = K Q^T, so a lane owns one query: its row max / row sum are lane
//     values plus cross-lane swaps.  K rows are placed in LDS in an order
//     that makes the S^T accumulator of a lane hold 8 consecutive keys, which
//     is exactly the bf16 B operand of O^T += V^T P^T: the softmax weights
//     never leave registers.
//   * fp32 online softmax in the log2 domain (exp2 with log2(e) folded into
//     the scale); weights rounded to bf16 for PV; o rounded to bf16 (RNE).
//   * causal masking only on tiles that reach past a workgroup's first query.
//   * when every request has the same number of new tokens, a work item's
//     request follows from its index and the prefix length is loaded beside
//     the first slot indices (one dependent round trip less); the output
//     rows leave through LDS as whole rows.
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
constexpr int NWAVES = 4; // waves per workgroup
constexpr int QB = 2;     // 16-row query blocks per wave (32 rows)
static_assert(NWAVES * QB * 16 == BM, "waves x rows cover the workgroup's rows");

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
  const int32_t* order;     // optional: requests in the order their tiles are handed out
  int32_t B, hq, hkv, G;
  float scale_log2e;
  int64_t pool_slots;
  int64_t tiles_bound;      // work items per kv head
  int64_t total_new;        // q rows; rows at or past it are never read
  int32_t uni_n;            // > 0: every request has this many new tokens
  int64_t tiles_per_req;    // work items per request when uni_n > 0
  uint32_t g_magic;         // ceil(2^32 / G) for G > 1: x / G = mulhi(x, g_magic) for x < 2^28
  int* err;
};

// Finds which request owns global tile index tg (tiles of BM rows, counted
// request by request, in request order or in a.order's).  Wave-parallel
// prefix sum over the requests; the result is uniform across the wave.
// Returns false when tg is past the end.  An a.order entry outside [0, B)
// owns no tiles.  The request's first q row, new-token count and prefix
// length come back with it: every lane loads them for its own request in the
// same pass, so they cost no further dependent memory round trip.
__device__ bool locate_tile(const ExtendArgs& a, int64_t tg, int& r, int& t, int& q0, int& n, int& p) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int base = 0; base < a.B; base += 64) {
    const int i = base + lane;
    int c = 0, ri = i, q0i = 0, ni = 0, pi = 0;
    if (i < a.B) {
      if (a.order) ri = a.order[i];
      if ((unsigned)ri < (unsigned)a.B) {
        q0i = a.qo_indptr[ri];
        ni = a.qo_indptr[ri + 1] - q0i;
        pi = a.prefix_lens[ri];
        c = (int)(((int64_t)ni * a.G + BM - 1) / BM);
      }
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
      // (uniform: readfirstlane keeps them in scalar registers)
      r = __builtin_amdgcn_readfirstlane(__shfl(ri, first));
      t = __builtin_amdgcn_readfirstlane((int)(tg - (acc + s_first - c_first)));
      q0 = __builtin_amdgcn_readfirstlane(__shfl(q0i, first));
      n = __builtin_amdgcn_readfirstlane(__shfl(ni, first));
      p = __builtin_amdgcn_readfirstlane(__shfl(pi, first));
      return true;
    }
    acc += tot;
  }
  return false;
}

// Key held by K LDS row rho of a 64-key tile.  Within each 32-key chunk,
// rows 0..15 hold keys 8*(i/4) + i%4 and rows 16..31 hold 8*(i/4) + 4 + i%4,
// so MFMA block kb = 2c + half gives lane group gq the keys
// c*32 + 8*gq + 4*half + [0..3]: two blocks together = 8 consecutive keys.
__device__ __forceinline__ int key_of_row(int rho) {
  const int c = rho >> 5, rr = rho & 31, half = rr >> 4, i = rr & 15;
  return c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
}

// XOR swizzles of the 16-byte chunk index by LDS row (tiles are stored with
// no padding, rows of D*2 bytes).  K is read as 16 consecutive rows per
// instruction, one chunk each: XOR by the row spreads them over all chunks.
// V is read transposed: each 16-lane group reads one 32-byte chunk pair from
// each of 4 consecutive rows, the 4 groups rows 8 apart; XOR of the pair
// index by the row's low bits (and bit 3) puts the 4 rows of a group on
// distinct banks and every bank of the wave's 512 bytes under exactly two.
template <int CH>
__device__ __forceinline__ int swz_k(int row) { return row & (CH - 1); }
template <int CH>
__device__ __forceinline__ int swz_v(int row) {
  return CH == 16 ? (((row & 3) << 1) | (((row >> 3) & 1) << 3)) : ((row & 2) | (((row >> 3) & 1) << 2));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define RKV_LDS __attribute__((address_space(3)))

// Global -> LDS copies (gfx950 LDS DMA): lane l's 16 (4) bytes land at
// lds_base + 16*l (4*l).  Issued as inline assembly: the compiler counts a
// global_load_lds it emits itself as an LDS access that may complete out of
// order, and then waits for every LDS operation (lgkmcnt(0)) wherever it
// needs any one of them, so each operand read fetched ahead would be drained
// together with the one it waits for.  From assembly the copy is invisible
// to that bookkeeping; it writes LDS only (no register), and every stage it
// fills is read only after a full s_waitcnt and a barrier.  Every LDS DMA
// of this file's kernels goes through these two, so no compiler-generated
// code there keeps a value in M0 across them (the compiler warns that a
// clobbered M0 is reserved; nothing of its own relies on M0 here).
// The LDS address is the low half of the generic address: the shared
// aperture is 4 GiB aligned, so that half is the LDS offset itself (a cast
// to the LDS address space would add a null test per copy).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Softmax weights are kept relative to a per-row reference maximum that is
// only raised when a tile's maximum exceeds it by more than 2^8 (log2 units):
// weights stay <= 256, harmless in fp32 and bf16, and the O accumulators are
// rescaled only on those rare tiles instead of on every tile.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
__global__ __launch_bounds__(NWAVES * 64, 2) void extend_bf16(ExtendArgs a) {
  constexpr int ROWB = D * 2;              // bytes of one (slot, kv head) row
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int KSTEPS = D / 32;           // QK contraction steps
  constexpr int DBLK = D / 16;             // PV output blocks
  constexpr int RPI = 1024 / ROWB;         // rows one wave moves per DMA instruction
  constexpr int NDMA = BN / (RPI * NWAVES);  // DMA instructions per wave per tile (each of K, V)
  constexpr int TILEB = BN * ROWB;         // bytes of one K or V tile

  // K runs one tile ahead of V, each in two stages; slot indices run one
  // more tile ahead.  The stages are separate LDS objects addressed with a
  // compile-time parity (the key loop is unrolled by two), so the compiler
  // can tell that the operand reads of one stage never alias the DMA still
  // writing the other and does not wait for that DMA before them.
  __shared__ __attribute__((aligned(16))) char K0[TILEB];
  __shared__ __attribute__((aligned(16))) char K1[TILEB];
  __shared__ __attribute__((aligned(16))) char V0[TILEB];
  __shared__ __attribute__((aligned(16))) char V1[TILEB];
  // slot indices of four tiles, stored in the order the gather lanes use
  // them (each lane's NDMA slots of a tile are contiguous)
  __shared__ __attribute__((aligned(16))) int32_t SlK[4][BN];
  __shared__ __attribute__((aligned(16))) int32_t SlV[4][BN];
  auto kbuf = [&](auto par) -> char* {
    if constexpr (decltype(par)::value == 0) return K0; else return K1;
  };
  auto vbuf = [&](auto par) -> char* {
    if constexpr (decltype(par)::value == 0) return V0; else return V1;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // item decode in 32 bits (the grid is below 2^31): a 64-bit division by a
  // run-time value costs hundreds of instructions
  const uint32_t w = (uint32_t)rkv::xcd_work_item(blockIdx.x, gridDim.x);
  const uint32_t tb = (uint32_t)a.tiles_bound;
  const int g = (int)(w / tb);
  const int64_t tg = w - (uint32_t)g * tb;
  if (g >= a.hkv) return;
  int r = 0, t = 0, q0 = 0, n = 0, p = 0;
  const bool uni = a.uni_n > 0;
  if (uni) {
    // every request has uni_n new tokens (so its q rows start at r * uni_n):
    // the request and tile follow from the work item's index, and the
    // prefix length is loaded beside the first slot indices and queries
    // below instead of before them (one dependent memory round trip less)
    const uint32_t tpr = (uint32_t)a.tiles_per_req;
    const uint32_t i = (uint32_t)tg / tpr;
    if (i >= (uint32_t)a.B) return;
    t = (int)((uint32_t)tg - i * tpr);
    r = (int)i;
    if (a.order) {
      r = a.order[i];
      if ((unsigned)r >= (unsigned)a.B) return;
    }
    n = a.uni_n;
    q0 = r * n;
  } else if (!locate_tile(a, tg, r, t, q0, n, p)) {
    return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int G = a.G;
  // row / G for the non-negative row numbers of a request (below 2^28); the
  // high half of the product is written out (the library's __umulhi is a
  // call that is not inlined here)
  auto div_g = [&](int x) -> int {
    return G == 1 ? x : (int)(((uint64_t)(uint32_t)x * a.g_magic) >> 32);
  };
  const int rows_total = n * G;
  const int row0 = t * BM;
  const int row_last = min(row0 + BM, rows_total) - 1;

  // ---- queries of this wave: rows row0 + wave*32 + qb*16 + l16.  Every
  //      lane loads a query, so the loads need no branch: a row past the
  //      request's rows reads q row 0, and a row whose key position lies
  //      past the table row still reads its own.  Only valid rows are
  //      written.
  bf16x8 qreg[QB][KSTEPS];
  int qlim[QB], qhead[QB], qtok[QB], qj[QB];
  bool qvalid[QB];
  const uint16_t* qbase = (const uint16_t*)a.q;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = row0 + wave * (QB * 16) + qb * 16 + l16;
    const int j = div_g(row);
    qvalid[qb] = row < rows_total && (int64_t)q0 + j < a.total_new;
    qj[qb] = qvalid[qb] ? j : 0;
    const int hh = qvalid[qb] ? row - j * G : 0;
    qtok[qb] = q0 + qj[qb];
    qhead[qb] = g * G + hh;
    const uint16_t* qp = qbase + (qvalid[qb] ? ((int64_t)qtok[qb] * a.hq + qhead[qb]) * D : 0) + gq * 8;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[qb][s] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + s * 32));
  }

  f32x4 oacc[QB][DBLK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mref[qb] = -INFINITY;
  // row sums of the bf16 weights, accumulated on the MFMA (all-ones A
  // operand) so that numerator and denominator use the same rounded weights;
  // every element of lacc[qb] holds the lane's full row sum
  f32x4 lacc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const float c = a.scale_log2e;

  // keys never reach past the table row, whatever the lengths say; the
  // bounds that follow from the prefix length are set once it has arrived
  int kv_end = 0, ntiles = 0, first_mask_tile = 0;
  auto set_bounds = [&]() {
    kv_end = (int)min((int64_t)p + div_g(row_last) + 1, a.ld);
    ntiles = (kv_end + BN - 1) / BN;
    // tiles before this one are fully visible to every row of the workgroup
    first_mask_tile = min(ntiles, (p + div_g(row0)) / BN);
  };
  if (!uni) set_bounds();

  // ---- gathers: every row index is clamped into the table row (into
  //      [0, kv_end) once the prefix length is known) and every slot into
  //      [0, pool_slots), so no access leaves the table or the pool; keys
  //      past kv_end are masked by the causal test
  const int32_t* row_tab = a.r2t + (int64_t)r * a.ld;
  const uint32_t P = (uint32_t)min(a.pool_slots, (int64_t)0x7fffffff);
  const uint32_t slot_bytes = (uint32_t)a.hkv * ROWB;
  // DMA lane roles: row (within the wave's run of RPI rows) and LDS chunk
  const int drow = lane / CH;
  const int dch = lane % CH;
  // LDS tile row handled by DMA instruction j of (wave w, lane row dr)
  auto dma_row = [](int w, int j, int dr) { return (w * NDMA + j) * RPI + dr; };
  // slot-table position p <-> (wave, lane row, instruction): the key whose
  // slot a gather lane needs, for the K tile (rows permuted) and the V tile
  auto pos_row = [&](int p) { return dma_row(p / (NDMA * RPI), p % NDMA, (p / NDMA) % RPI); };
  const int key_k = key_of_row(pos_row(lane));
  const int key_v = pos_row(lane);
  const char* kg = (const char*)a.kp + (uint64_t)g * ROWB;
  const char* vg = (const char*)a.vp + (uint64_t)g * ROWB;
  // A gather lane's NDMA slots of a tile are contiguous in the slot stage:
  // one LDS read brings them all (the copies are assembly with a memory
  // clobber, so a slot read between two of them would have to complete
  // before the second could issue).
  typedef int32_t slotv __attribute__((ext_vector_type(NDMA)));
  auto lane_slots = [&](const int32_t* stage) -> slotv {
    return *(const slotv*)(stage + (wave * RPI + drow) * NDMA);
  };
  // gather instruction j of a tile; a slot outside [0, pool_slots) is
  // clamped to the pool's last slot
  auto gather1 = [&](int32_t slot_in, char* dst, const char* src, int j, auto is_k) {
    const uint32_t slot = min((uint32_t)slot_in, P - 1);
    const int R = dma_row(wave, j, drow);
    const int lch = dch ^ (decltype(is_k)::value ? swz_k<CH>(R) : swz_v<CH>(R));
    dma16(src + (uint64_t)slot * slot_bytes + lch * 16, dst + (wave * NDMA + j) * 1024);
  };
  // slot indices of tile `tile` into stage tile & 3 (wave 0 for K, wave 1
  // for V, one 4-byte DMA each, straight from the table; keys clamped into
  // [0, hi]).  K tile k holds keys [64k - 32, 64k + 32): shifted half a
  // tile against V, so that QK runs one half tile ahead of PV while each
  // iteration still reads one K tile and one V tile.
  auto dma_slots = [&](int tile, int hi) {
    hi = max(hi, 0);
    if (wave == 0) dma4(row_tab + min(max(tile * BN - BN / 2 + key_k, 0), hi), SlK[tile & 3]);
    else if (wave == 1) dma4(row_tab + min(tile * BN + key_v, hi), SlV[tile & 3]);
  };

  // The softmax runs on 32-key halves of a tile ("half tiles", numbered u =
  // 2*tile + h), so that QK of half tile u+1 overlaps the exponentials of u
  // and PV of u overlaps the row maxima of u+1, with the scores of just two
  // half tiles live: s_ev / s_od hold the even / odd half tiles, and
  // s[qb][kk] holds, for lane group gq, the keys 8*gq + 4*kk + [0..3] of the
  // half tile for its query (K rows are placed in LDS so).

  // this lane's part of the raw row maxima of the latest half tile, and the
  // raise thresholds
  float mt[QB], thr[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) thr[qb] = -INFINITY;
  // the rare rescale: raise the reference of every row of the wave to its
  // row maximum (the 4 lane groups' parts) and rescale its O and row sum (PV
  // of the previous half tile has been issued)
  auto rescale = [&](const float (&mtv)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float rmx = rkv::max_xor32(rkv::max_xor16(mtv[qb]));
      const float mn = fmaxf(mref[qb], rmx * c);
      const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
      mref[qb] = mn;
      thr[qb] = (mn + kRescaleThreshold) / c;
      lacc[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[qb][db] *= alpha;
    }
  };

  // ---- operands and softmax pieces of one half tile
  // K operand i = (contraction step i/2, 16-key block i%2) of half h of the
  // K tile in ks
  auto k_op = [&](const char* ks, int h, int i) __attribute__((always_inline)) -> bf16x8 {
    const int row = (2 * h + (i & 1)) * 16 + l16;
    return __builtin_bit_cast(bf16x8, *(const uint4*)(ks + row * ROWB + ((((i >> 1) * 4 + gq) ^ swz_k<CH>(row)) << 4)));
  };
  // V^T operand of output block db, half h of the V tile in vs: two
  // transposed reads of 4 keys each.  Lane p of group gq points at key row
  // 32*h + 8*gq + 4*hh + p/4, d = 16*db + 4*(p%4); lane i then receives
  // keys [0..3] of that row run at d = 16*db + i.
  auto v_op = [&](const char* vs, int h, int db) __attribute__((always_inline)) -> bf16x8 {
    v4i16 part[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = h * 32 + gq * 8 + hh * 4 + (l16 >> 2);
      const int d = db * 16 + 4 * (l16 & 3);
      const char* ptr = vs + row * ROWB + ((((d >> 3) ^ swz_v<CH>(row))) << 4) + ((d & 7) << 1);
      part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RKV_LDS v4i16*)ptr);
    }
    return __builtin_bit_cast(
        bf16x8, make_uint4(__builtin_bit_cast(uint2, part[0]).x, __builtin_bit_cast(uint2, part[0]).y,
                           __builtin_bit_cast(uint2, part[1]).x, __builtin_bit_cast(uint2, part[1]).y));
  };
  // softmax weights e = 2w, 2w+1 (w < 4) of query block qb, rounded to bf16
  // and packed: word w of the B operand of its PV
  auto exp_word = [&](const f32x4 (&sacc)[QB][2], int qb, int w) __attribute__((always_inline)) -> uint32_t {
    const int kk = w >> 1, i = 2 * (w & 1);
    const float m = mref[qb];
    return rkv::pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sacc[qb][kk][i], c, -m)),
                            __builtin_amdgcn_exp2f(fmaf(sacc[qb][kk][i + 1], c, -m)));
  };
  // this lane's part of the row maximum of query block qb over a half tile
  // whose first key is key0 (causal mask first when MASK): the maximum of
  // its 8 scores
  auto lane_max = [&](f32x4 (&sacc)[QB][2], int qb, int key0, auto mask_tag) __attribute__((always_inline)) -> float {
    if constexpr (decltype(mask_tag)::value) {
      const int lim = qlim[qb] - key0;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * kk + i > lim) sacc[qb][kk][i] = -INFINITY;
    }
    // three-input maxima: 8 values in 4 instructions
    const float m1 = fmaxf(fmaxf(sacc[qb][0][0], sacc[qb][0][1]), sacc[qb][0][2]);
    const float m2 = fmaxf(fmaxf(sacc[qb][0][3], sacc[qb][1][0]), sacc[qb][1][1]);
    const float m3 = fmaxf(fmaxf(m1, m2), sacc[qb][1][2]);
    return fmaxf(m3, sacc[qb][1][3]);
  };
  // the reference is raised when the raw row maximum mx of the latest half
  // tile has mx * c > mref + threshold, i.e. mx > thr = (mref + threshold) / c
  // (c > 0).  A row's maximum exceeds thr exactly when one of its 4 lanes'
  // parts does, so the common case costs one compare per lane and a ballot;
  // the cross-lane maximum is taken only in the rescale.
  auto row_max = [&](float mx, int qb) __attribute__((always_inline)) -> bool {
    mt[qb] = mx;
    return mx > thr[qb];
  };

  // ---- one half-tile block, software pipelined in stages separated by
  //      scheduling fences (operands are fetched two stages ahead and every
  //      group of MFMAs has VALU work beside it, so the wave keeps the
  //      matrix unit fed on its own and the SIMD's other wave fills gaps):
  //   X: S^T(u+1) = K Q^T on half hk of the K tile in ks (QK), 2*KSTEPS
  //      stages of QB MFMAs, beside the exponentials of half tile u
  //      (scores s_old) and, with GATHER, all gathers of K tile gk (into
  //      kdst) and V tile gk-1 (into vdst), one per stage;
  //   Y: row sums and O^T += V^T P^T on half hv of the V tile in vs, DBLK
  //      stages of QB MFMAs, beside the row maxima of half tile u+1 (QK)
  //      whose first key is key0.
  //   Returns whether some row's reference must be raised.
  auto block = [&](const char* ks, int hk, f32x4 (&s_new)[QB][2], const f32x4 (&s_old)[QB][2],
                   const char* vs, int hv, int key0, auto qk_tag, auto mask_tag, auto gather_tag, int gk,
                   char* kdst, char* vdst) __attribute__((always_inline)) -> bool {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool GATHER = decltype(gather_tag)::value;
    constexpr int NK = 2 * KSTEPS;          // X stages
    constexpr int WPS = 4 * QB / NK;        // exponential words per X stage
    constexpr int NG = 2 * NDMA;            // gathers of this block (K and V alternating)
    static_assert(WPS * NK == 4 * QB, "exponential words split evenly over X");
    // slots of this block's gathers, read before its first operands (the
    // first stage's wait then covers them)
    slotv ksl, vsl;
    if constexpr (GATHER) {
      ksl = lane_slots(SlK[gk & 3]);
      vsl = lane_slots(SlV[(gk - 1) & 3]);
    }
    bf16x8 kop[NK];
    if constexpr (QK) {
      kop[0] = k_op(ks, hk, 0);
      kop[1] = k_op(ks, hk, 1);
    }
    uint32_t wv[QB][4];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if constexpr (QK) {
        if (i + 2 < NK) kop[i + 2] = k_op(ks, hk, i + 2);
        const int st = i >> 1, kk = i & 1;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s_new[qb][kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kop[i], qreg[qb][st], st == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s_new[qb][kk], 0, 0, 0);
      }
#pragma unroll
      for (int e = i * WPS; e < (i + 1) * WPS; ++e) wv[e >> 2][e & 3] = exp_word(s_old, e >> 2, e & 3);
      if constexpr (GATHER) {
#pragma unroll
        for (int gi = i * NG / NK; gi < (i + 1) * NG / NK; ++gi) {
          const int j = gi >> 1;
          // out-of-range slots are clamped into the pool (the debug check
          // runs beside the kernel)
          const uint32_t slot = min((uint32_t)((gi & 1) ? vsl[gi >> 1] : ksl[gi >> 1]), P - 1);
          const int R = dma_row(wave, j, drow);
          if (gi & 1)
            dma16(vg + (uint64_t)slot * slot_bytes + (dch ^ swz_v<CH>(R)) * 16, vdst + (wave * NDMA + j) * 1024);
          else
            dma16(kg + (uint64_t)slot * slot_bytes + (dch ^ swz_k<CH>(R)) * 16, kdst + (wave * NDMA + j) * 1024);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 pb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      pb[qb] = __builtin_bit_cast(bf16x8, make_uint4(wv[qb][0], wv[qb][1], wv[qb][2], wv[qb][3]));
    bf16x8 vop[DBLK];
    vop[0] = v_op(vs, hv, 0);
    vop[1] = v_op(vs, hv, 1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      lacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb], lacc[qb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    bool raise = false;
    float lm[QB];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      if (db + 2 < DBLK) vop[db + 2] = v_op(vs, hv, db + 2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db], pb[qb], oacc[qb][db], 0, 0, 0);
      if constexpr (QK) {
        // the maxima of query blocks spread over the Y stages: the lane's
        // part of block qb, then its compare a stage later
        constexpr int SPQ = DBLK / QB;        // Y stages per query block (2 or 1)
        const int qb = db / SPQ;
        if (SPQ == 1 || db % SPQ == 0) lm[qb] = lane_max(s_new, qb, key0, mask_tag);
        if (SPQ == 1 || db % SPQ == SPQ - 1) raise |= row_max(lm[qb], qb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return raise;
  };

  // scores of the even and the odd half tiles
  f32x4 s_ev[QB][2], s_od[QB][2];

  // prologue: slots of tiles 0..2; K tiles 0 and 1 (keys -32..95), V tile 0;
  // QK of half tile 0 (the second half of K tile 0) and its maxima.  With
  // uniform new-token counts the prefix length is still in flight: the slot
  // indices are read up to the end of the table row, and read again with
  // the request's own bound if it ends inside these three tiles (so that no
  // row outside the request is gathered).
  {
    const int hi0 = uni ? (int)min(a.ld, (int64_t)0x7fffffff) - 1 : kv_end - 1;
    if (uni) p = a.prefix_lens[r];
    dma_slots(0, hi0);
    dma_slots(1, hi0);
    dma_slots(2, hi0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (uni) {
      set_bounds();
      if (kv_end < min(3 * BN, hi0 + 1)) {
        dma_slots(0, kv_end - 1);
        dma_slots(1, kv_end - 1);
        dma_slots(2, kv_end - 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qvalid[qb] = qvalid[qb] && p + qj[qb] < kv_end;
    // last visible key, relative to the first key this lane holds in a
    // 32-key half tile
    qlim[qb] = (qvalid[qb] ? p + qj[qb] : kv_end - 1) - 8 * gq;
  }
  {
    // the three tiles' slots first, so their LDS reads overlap
    const slotv sk0 = lane_slots(SlK[0]), sv0 = lane_slots(SlV[0]), sk1 = lane_slots(SlK[1]);
#pragma unroll
    for (int j = 0; j < NDMA; ++j) gather1(sk0[j], K0, kg, j, std::true_type{});
#pragma unroll
    for (int j = 0; j < NDMA; ++j) gather1(sv0[j], V0, vg, j, std::false_type{});
#pragma unroll
    for (int j = 0; j < NDMA; ++j) gather1(sk1[j], K1, kg, j, std::true_type{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2 * KSTEPS; ++i) {
    const bf16x8 ka = k_op(K0, 1, i);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s_ev[qb][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          ka, qreg[qb][i >> 1], (i >> 1) == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s_ev[qb][i & 1], 0, 0, 0);
  }
  {
    bool raise0 = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lm = first_mask_tile == 0 ? lane_max(s_ev, qb, 0, std::true_type{})
                                            : lane_max(s_ev, qb, 0, std::false_type{});
      raise0 |= row_max(lm, qb);
    }
    // first half tile: O and the row sums are still zero, so only the
    // reference and the threshold are set
    if (__builtin_amdgcn_ballot_w64(raise0)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float rmx = rkv::max_xor32(rkv::max_xor16(mt[qb]));
        mref[qb] = rmx * c;
        thr[qb] = (mref[qb] + kRescaleThreshold) / c;
      }
    }
  }

  // iteration t (half tile 2t's maxima taken; K tile t+1 = half tiles 2t+1
  // and 2t+2, V tile t = half tiles 2t and 2t+1 resident): two blocks
  //   exp(2t) || QK(2t+1), then PV(2t) || max(2t+1)
  //   exp(2t+1) || QK(2t+2), then PV(2t+1) || max(2t+2)
  // with the gathers of K tile t+2 and V tile t+1 spread over the first QK
  // phase (as early as their stages are free: issuing half of them in the
  // second phase left the end-of-iteration wait exposed), then wait for them
  // and meet at the barrier.  MASK covers both
  // maxima taken here (half tiles of tiles t and t+1); on a fully visible
  // half tile the mask changes nothing.  Without NEXT (the last tile) there
  // is no half tile 2t+2 and nothing to gather.
  auto iteration = [&](int tile, auto par, auto mask_tag, auto next_tag) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    using NPAR = std::integral_constant<int, 1 - decltype(par)::value>;
    using GT = std::integral_constant<bool, NEXT>;
    // The slot indices of tile t+3 go straight from the table into their
    // LDS stage (one 4-byte DMA per wave; they are range-checked where the
    // gathers read them), so no register has to wait for them.  Past the
    // last tile the keys are clamped: the gathers then refill the stage
    // consumed in the previous iteration with rows nobody reads again.
    dma_slots(tile + 3, kv_end - 1);
    char* kn = kbuf(NPAR{});      // K tile t+1
    char* kd = kbuf(par);         // K tile t+2 lands in the stage K tile t used
    char* vs = vbuf(par);         // V tile t
    char* vd = vbuf(NPAR{});      // V tile t+1
    bool up = block(kn, 0, s_od, s_ev, vs, 0, tile * BN + 32, std::true_type{}, mask_tag, GT{}, tile + 2, kd, vd);
    if (__builtin_amdgcn_ballot_w64(up)) rescale(mt);
    up = block(kn, 1, s_ev, s_od, vs, 1, tile * BN + BN, GT{}, mask_tag, std::false_type{}, tile + 2, kd, vd);
    if constexpr (NEXT) {
      if (__builtin_amdgcn_ballot_w64(up)) rescale(mt);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    const bool m0 = tile + 1 >= first_mask_tile, n0 = tile + 1 < ntiles;
    if (m0) {
      if (n0) iteration(tile, I0{}, std::true_type{}, std::true_type{});
      else iteration(tile, I0{}, std::true_type{}, std::false_type{});
    } else {
      iteration(tile, I0{}, std::false_type{}, std::true_type{});
    }
    if (tile + 1 < ntiles) {
      const bool m1 = tile + 2 >= first_mask_tile, n1 = tile + 2 < ntiles;
      if (m1) {
        if (n1) iteration(tile + 1, I1{}, std::true_type{}, std::true_type{});
        else iteration(tile + 1, I1{}, std::true_type{}, std::false_type{});
      } else {
        iteration(tile + 1, I1{}, std::false_type{}, std::true_type{});
      }
    }
  }

  // ---- epilogue: lane holds o[query l16][d = db*16 + 4*gq + 0..3].  The
  //      normalized rows go through this wave's 32 rows of LDS (the K stages
  //      are free after the loop's last barrier: no read of them and no copy
  //      into them is outstanding), so that each store instruction writes
  //      whole rows of D bf16 instead of 32-byte pieces of 16 rows.
  static_assert(2 * 32 * ROWB <= TILEB, "two waves' rows fit one K stage");
  char* stage = (wave < 2 ? K0 : K1) + (wave & 1) * (32 * ROWB);
  uint16_t* obase = (uint16_t*)a.o;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = lacc[qb][0];
    const float inv = 1.f / lsum;
    const int r = qb * 16 + l16;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const f32x4 v = oacc[qb][db];
      const int c16 = db * 2 + (gq >> 1);
      *(uint2*)(stage + r * ROWB + ((c16 ^ (r & (CH - 1))) << 4) + (gq & 1) * 8) =
          make_uint2(rkv::pack_bf16x2(v[0] * inv, v[1] * inv), rkv::pack_bf16x2(v[2] * inv, v[3] * inv));
    }
    if (qvalid[qb] && a.lse && gq == 0)
      a.lse[(int64_t)qtok[qb] * a.hq + qhead[qb]] = (mref[qb] + log2f(lsum)) * 0.69314718055994531f;
  }
  {
    constexpr int RPS = 64 / CH;            // rows per store instruction
    const int c = lane % CH;
#pragma unroll
    for (int k = 0; k < 32 / RPS; ++k) {
      const int r = k * RPS + lane / CH;
      const uint4 val = *(const uint4*)(stage + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
      const int row = row0 + wave * 32 + r;
      const int j = div_g(row);
      if (row < rows_total && (int64_t)q0 + j < a.total_new && p + j < kv_end)
        *(uint4*)(obase + ((int64_t)(q0 + j) * a.hq + g * G + (row - j * G)) * D + c * 8) = val;
    }
  }
}

// Debug check beside the bf16 kernel, which clamps every gathered slot into
// the pool: one workgroup per request over the table entries of the keys it
// reads, [0, p + n) (within ld); an entry outside [0, pool_slots) raises the
// flag.
__global__ __launch_bounds__(256) void check_slots(ExtendArgs a) {
  const int r = blockIdx.x;
  if (r >= a.B) return;
  const int64_t n = (int64_t)a.qo_indptr[r + 1] - a.qo_indptr[r];
  const int64_t L = min((int64_t)a.prefix_lens[r] + n, a.ld);
  const int32_t* row = a.r2t + (int64_t)r * a.ld;
  bool bad = false;
  for (int64_t i = threadIdx.x; i < L; i += blockDim.x) bad |= (uint32_t)row[i] >= (uint64_t)a.pool_slots;
  if (bad) rkv::raise_flag(a.err);
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
  // l is summed with compensation (Kahan): over a long context a plain
  // running sum of the weights loses ~sqrt(n) ulps, which lse shows directly
  // (120k keys: 1.5e-5); lc carries the low-order part lost by each addition
  float m = -INFINITY, l = 0.f, lc = 0.f;
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
    l *= alpha;
    lc *= alpha;
    const float y = pw - lc;
    const float t = l + y;
    lc = (t - l) - y;
    l = t;
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
                               const int32_t* prefix_lens, const int32_t* req_order, int32_t B,
                               int64_t total_new,
                               int32_t max_new, int32_t hq, int32_t hkv, int32_t d, float sm_scale,
                               int32_t dtype, int64_t pool_slots, void* stream) {
  rkv::clear_error();
  if (B < 0 || total_new < 0 || max_new < 0 || hq < 1 || hkv < 1 || ld < 1 || pool_slots < 1 ||
      !(sm_scale > 0.f))
    return rkv::fail(RKV_EINVAL, "rkv_attn_extend: bad sizes");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: dtype");
  if (d != 64 && d != 128) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: head_dim must be 64 or 128");
  if (hq % hkv != 0 || hq / hkv > 16) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: Hq/Hkv must be an integer <= 16");
  if ((int64_t)max_new * (hq / hkv) >= ((int64_t)1 << 28))
    return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: max_new * Hq/Hkv must be below 2^28");
  if (B == 0 || total_new == 0) return RKV_OK;
  if (!q || !k_pool || !v_pool || !o || !req_to_token || !qo_indptr || !prefix_lens)
    return rkv::fail(RKV_EINVAL, "rkv_attn_extend: NULL pointer");
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o;
  if (al & 15) return rkv::fail(RKV_EINVAL, "rkv_attn_extend: tensors must be 16-byte aligned");
  ExtendArgs a;
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.o = o; a.lse = lse;
  a.r2t = req_to_token; a.ld = ld; a.qo_indptr = qo_indptr; a.prefix_lens = prefix_lens;
  a.order = req_order;
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
    // with total_new == B * max_new and every n_r <= max_new, every request
    // has max_new new tokens
    a.uni_n = total_new == (int64_t)B * max_new ? max_new : 0;
    a.tiles_per_req = per_req;
    a.g_magic = a.G > 1 ? (uint32_t)((((uint64_t)1 << 32) + a.G - 1) / a.G) : 0u;
    int64_t grid = a.tiles_bound * hkv;
    grid = (grid + rkv::kXcds - 1) / rkv::kXcds * rkv::kXcds;
    if (grid > 0x7fffffff) return rkv::fail(RKV_ENOTSUP, "rkv_attn_extend: grid too large");
    if (a.err) hipLaunchKernelGGL(check_slots, dim3((unsigned)B), dim3(256), 0, st, a);
    if (d == 128)
      hipLaunchKernelGGL(extend_bf16<128>, dim3((unsigned)grid), dim3(NWAVES * 64), 0, st, a);
    else
      hipLaunchKernelGGL(extend_bf16<64>, dim3((unsigned)grid), dim3(NWAVES * 64), 0, st, a);
  } else {
    a.tiles_bound = 0;
    a.uni_n = 0;
    a.tiles_per_req = 0;
    a.g_magic = 0;
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
