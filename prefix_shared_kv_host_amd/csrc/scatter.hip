// KV scatter: write the new tokens' K and V rows into their pool slots.
//
// RadixAttention computes KV only for the tokens that are not cached and
// stores it so later requests can reuse it (unite.ai, "SGLang: Efficient
// Execution of Structured Language Model Programs", section "Introduccion a
// SGLang", RadixAttention bullet).  The pool is token-slot major: one slot =
// Hkv*D contiguous elements.  This is a plain copy, so it is HBM-bound: every
// byte is read once and written once.  One workgroup walks rows (grid-stride
// over tokens); its 256 lanes move 16-byte chunks of the row, so each wave
// reads and writes 1 KiB contiguous per instruction.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "rkv.h"
#include "rkv_internal.h"

namespace {

__global__ __launch_bounds__(256) void kv_scatter_kernel(const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         const int32_t* __restrict__ slots, int64_t T,
                                                         uint4* __restrict__ k_pool,
                                                         uint4* __restrict__ v_pool,
                                                         int64_t pool_slots, int chunks, int* err) {
  for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
    const int32_t s = slots[row];
    if (s < 0 || (int64_t)s >= pool_slots) {
      if (threadIdx.x == 0) rkv::raise_flag(err);
      continue;
    }
    const int64_t src = row * chunks;
    const int64_t dst = (int64_t)s * chunks;
    for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
      const uint4 kk = k_new[src + c];
      const uint4 vv = v_new[src + c];
      k_pool[dst + c] = kk;
      v_pool[dst + c] = vv;
    }
  }
}

// One lane per request: the decode step's new slot goes after the row's last
// entry and the length grows by one.
__global__ __launch_bounds__(256) void table_append_kernel(int32_t* __restrict__ r2t, int64_t ld,
                                                           int32_t* __restrict__ seq_lens,
                                                           const int32_t* __restrict__ new_slots, int32_t B,
                                                           int* err) {
  const int32_t r = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  if (r >= B) return;
  const int32_t L = seq_lens[r];
  if (L < 0 || (int64_t)L >= ld) {
    rkv::raise_flag(err);
    return;
  }
  r2t[(int64_t)r * ld + L] = new_slots[r];
  seq_lens[r] = L + 1;
}

}  // namespace

extern "C" int rkv_table_append(int32_t* req_to_token, int64_t ld, int32_t* seq_lens, const int32_t* new_slots,
                                int32_t B, void* stream) {
  rkv::clear_error();
  if (B < 0 || ld < 1) return rkv::fail(RKV_EINVAL, "rkv_table_append: bad sizes");
  if (B == 0) return RKV_OK;
  if (!req_to_token || !seq_lens || !new_slots) return rkv::fail(RKV_EINVAL, "rkv_table_append: NULL pointer");
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(table_append_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, req_to_token, ld,
                     seq_lens, new_slots, B, flag);
  return rkv::finish_launch("rkv_table_append", st, flag);
}

extern "C" int rkv_kv_scatter(const void* k_new, const void* v_new, const int32_t* slots, int64_t T,
                              void* k_pool, void* v_pool, int64_t pool_slots, int32_t hkv, int32_t d,
                              int32_t dtype, void* stream) {
  rkv::clear_error();
  if (T < 0 || pool_slots < 1 || hkv < 1) return rkv::fail(RKV_EINVAL, "rkv_kv_scatter: bad sizes");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, "rkv_kv_scatter: dtype");
  if (d != 64 && d != 128) return rkv::fail(RKV_ENOTSUP, "rkv_kv_scatter: head_dim must be 64 or 128");
  if (T == 0) return RKV_OK;
  if (!k_new || !v_new || !slots || !k_pool || !v_pool)
    return rkv::fail(RKV_EINVAL, "rkv_kv_scatter: NULL pointer");
  const uintptr_t al = (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool;
  if (al & 15) return rkv::fail(RKV_EINVAL, "rkv_kv_scatter: tensors must be 16-byte aligned");
  const int64_t row_bytes = (int64_t)hkv * d * (dtype == RKV_BF16 ? 2 : 4);
  const int chunks = (int)(row_bytes / 16);
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  const int64_t grid = T < 65536 ? T : 65536;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(kv_scatter_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                     (const uint4*)k_new, (const uint4*)v_new, slots, T, (uint4*)k_pool,
                     (uint4*)v_pool, pool_slots, chunks, flag);
  return rkv::finish_launch("rkv_kv_scatter", st, flag);
}
