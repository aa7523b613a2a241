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

// Key held by K LDS row rho of a 64-key tile.  Within each 32-key chunk,
// rows 0..15 hold keys 8*(i/4) + i%4 and rows 16..31 hold 8*(i/4) + 4 + i%4,
// so MFMA block kb = 2c + half gives lane group gq the keys
// c*32 + 8*gq + 4*half + [0..3]: two blocks together = 8 consecutive keys.
__device__ __forceinline__ int key_of_row(int rho) {
  const int c = rho >> 5, rr = rho & 31, half = rr >> 4, i = rr & 15;
  return c * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void extend_bf16(ExtendArgs a) {
  constexpr int KP = D + 8;          // K row pitch in LDS (elements)
  constexpr int VP = BN + 8;         // V^T row pitch in LDS (elements)
  constexpr int KSTEPS = D / 32;     // QK contraction steps
  constexpr int DBLK = D / 16;       // PV output blocks
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int KROWS = 256 / CPR;   // K rows loaded per pass
  constexpr int KPASS = BN / KROWS;  // passes per tile
  constexpr int KPT = BN * CPR / 256;  // V keys per thread (transposed group)
  static_assert(KPT == 2 || KPT == 4, "V transpose group");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  const int64_t w = rkv::xcd_work_item(blockIdx.x, gridDim.x);
  const int g = (int)(w / a.tiles_bound);
  const int64_t tg = w % a.tiles_bound;
  if (g >= a.hkv) return;
  int r = 0, t = 0;
  if (!locate_tile(a, tg, r, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // ---- queries of this wave: rows row0 + wave*32 + qb*16 + l16
  bf16x8 qreg[2][KSTEPS];
  int qpos[2], qhead[2], qtok[2];
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
    qpos[qb] = qvalid[qb] ? p + j : kv_end - 1;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid[qb])
        v = *(const uint4*)(qbase + ((int64_t)qtok[qb] * a.hq + qhead[qb]) * D + s * 32 + gq * 8);
      qreg[qb][s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const int wave_row0 = row0 + wave * 32;
  const int wave_qmin = p + min(wave_row0, rows_total - 1) / G;

  f32x4 oacc[2][DBLK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) oacc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.f, 0.f};

  // ---- tile loader assignments
  const int32_t* row_tab = a.r2t + (int64_t)r * a.ld;
  const uint4* kp = (const uint4*)a.kp;
  const uint4* vp = (const uint4*)a.vp;
  const int64_t slot_stride = (int64_t)a.hkv * CPR;  // uint4 per slot
  const int64_t head_off = (int64_t)g * CPR;
  const int kc = tid % CPR;            // K chunk (16 bytes) this thread moves
  const int krow = tid / CPR;          // first K LDS row this thread moves
  const int vdg = tid % CPR;           // V: 8-wide d group
  const int vkq = tid / CPR;           // V: group of KPT keys

  uint4 kreg[KPASS], vreg[KPT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int key = tile * BN + key_of_row(krow + i * KROWS);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < kv_end) {
        const int32_t slot = row_tab[key];
        if (slot >= 0 && (int64_t)slot < a.pool_slots)
          v = kp[(int64_t)slot * slot_stride + head_off + kc];
        else
          rkv::raise_flag(a.err);
      }
      kreg[i] = v;
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int key = tile * BN + vkq * KPT + u;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < kv_end) {
        const int32_t slot = row_tab[key];
        if (slot >= 0 && (int64_t)slot < a.pool_slots)
          v = vp[(int64_t)slot * slot_stride + head_off + vdg];
        else
          rkv::raise_flag(a.err);
      }
      vreg[u] = v;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPASS; ++i)
      *(uint4*)(Ks + (krow + i * KROWS) * KP + kc * 8) = kreg[i];
    // V transposed: element (d, key) at Vt[d*VP + ((key/8) ^ (d/8 & 7))*8 + key%8]
    const int key0 = vkq * KPT;
    const int phys = ((key0 >> 3) ^ (vdg & 7)) * 8 + (key0 & 7);
    const uint32_t* w32[KPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) w32[u] = (const uint32_t*)&vreg[u];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int d = vdg * 8 + e2 * 2 + hi;
        uint32_t pk[KPT / 2];
#pragma unroll
        for (int u = 0; u < KPT; u += 2) {
          const uint32_t x0 = w32[u][e2], x1 = w32[u + 1][e2];
          pk[u / 2] = hi ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
        }
        if (KPT == 4)
          *(uint2*)(Vt + d * VP + phys) = make_uint2(pk[0], pk[KPT / 2 - 1]);
        else
          *(uint32_t*)(Vt + d * VP + phys) = pk[0];
      }
    }
  };

  load_tile(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile + 1 < ntiles) load_tile(tile + 1);

    // ---- S^T = K Q^T for 64 keys x 2 query blocks
    f32x4 sacc[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 ka = __builtin_bit_cast(bf16x8, *(const uint4*)(Ks + (kb * 16 + l16) * KP + s * 32 + gq * 8));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[qb][s], sacc[qb][kb], 0, 0, 0);
      }
    }

    // ---- online softmax; lane owns query l16 of each block, keys
    //      tile*64 + c*32 + 8*gq + 4*half + i  for block kb = 2c + half
    const bool need_mask = tile * BN + BN - 1 > wave_qmin;
    bf16x8 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[qb][kb][i];
          if (need_mask) {
            const int key = tile * BN + (kb >> 1) * 32 + 8 * gq + 4 * (kb & 1) + i;
            if (key > qpos[qb]) v = -INFINITY;
          }
          sacc[qb][kb][i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[qb], mx * a.scale_log2e);
      const float alpha = exp2f(mrow[qb] - mnew);
      mrow[qb] = mnew;
      float psum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(fmaf(sacc[qb][kb][i], a.scale_log2e, -mnew));
          pv[kb][i] = e;
          psum += e;
        }
      lrow[qb] = lrow[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[qb][db] *= alpha;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint4 u;
        u.x = rkv::pack_bf16x2(pv[2 * c][0], pv[2 * c][1]);
        u.y = rkv::pack_bf16x2(pv[2 * c][2], pv[2 * c][3]);
        u.z = rkv::pack_bf16x2(pv[2 * c + 1][0], pv[2 * c + 1][1]);
        u.w = rkv::pack_bf16x2(pv[2 * c + 1][2], pv[2 * c + 1][3]);
        pb[qb][c] = __builtin_bit_cast(bf16x8, u);
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d = db * 16 + l16;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int phys = ((c * 4 + gq) ^ ((d >> 3) & 7)) * 8;
        const bf16x8 va = __builtin_bit_cast(bf16x8, *(const uint4*)(Vt + d * VP + phys));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qb][c], oacc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds o[query l16][d = db*16 + 4*gq + 0..3]
  uint16_t* obase = (uint16_t*)a.o;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lsum = lrow[qb];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
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
      a.lse[(int64_t)qtok[qb] * a.hq + qhead[qb]] = (mrow[qb] + log2f(lsum)) * 0.69314718055994531f;
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
