// Batched sampling penalties: frequency, presence, repetition and
// min_new_tokens applied to the next-token logits of the running requests.
//
// SGLang's sampling parameters define the four penalties per request (the
// sampling page, sglang-zh.llamafactory.cn, "sampling_params", Penalties
// block), and its section on the performance implications of penalties says
// they run on the GPU over the whole batch with state of size vocab x running
// requests.  The readings taken for the formulas, which the page leaves open:
//   repetition r on every token of the prompt or the output:
//       x / r if x > 0, else x * r;
//   then frequency f and presence p on every token of the output:
//       x - f * count - p;
//   then, while the output is shorter than min_new_tokens, logit -inf for the
//   EOS and stop token ids.
//
// State per request slot (caller-owned device memory):
//   counts [slots, vocab] int32: bits 0..30 = occurrences of the token in the
//       output so far, bit 31 = the token occurs in the prompt;
//   seen [slots, cap] int32: the distinct tokens of prompt and output (the
//       only vocabulary entries a penalty other than the stop mask can
//       touch), seen_len [slots];
//   out_len [slots]: output tokens so far.
// The dense counts keep admission and the per-step update O(1) per token;
// the list lets apply touch only the affected logits (a few hundred per
// request) instead of sweeping the vocabulary: the kernel reads and writes
// O(prompt + output) entries per request, not O(vocab).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device.h"
#include "rkv.h"
#include "rkv_internal.h"

namespace {

constexpr uint32_t kPromptBit = 0x80000000u;
constexpr uint32_t kCountMask = 0x7fffffffu;

// One workgroup per admitted request: zero its counts row, then mark the
// prompt tokens (bit 31) and list each distinct one once.  The atomic OR
// returns the word before the OR, so exactly one lane sees a token's bit
// clear and lists it; the list order is therefore unspecified.
__global__ __launch_bounds__(256) void penalty_admit_kernel(int32_t* __restrict__ counts, int32_t* __restrict__ seen,
                                                           int32_t* __restrict__ seen_len,
                                                           int32_t* __restrict__ out_len, int32_t n_slots,
                                                           int32_t vocab, int32_t cap, const int32_t* __restrict__ rows,
                                                           const int32_t* __restrict__ prompt_indptr,
                                                           const int32_t* __restrict__ prompt_ids, int* err) {
  __shared__ int n_listed;
  const int i = blockIdx.x;
  const int row = rows[i];
  if (row < 0 || row >= n_slots) {
    if (threadIdx.x == 0 && err) rkv::raise_flag(err);
    return;
  }
  uint32_t* crow = (uint32_t*)counts + (int64_t)row * vocab;
  // zero the row with 16-byte stores between its unaligned ends
  const int head = min(vocab, (int)(((16u - ((uint32_t)(uintptr_t)crow & 15u)) & 15u) >> 2));
  const int nvec = (vocab - head) >> 2;
  for (int v = threadIdx.x; v < head; v += blockDim.x) crow[v] = 0u;
  uint4* mid = (uint4*)(crow + head);
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) mid[v] = make_uint4(0u, 0u, 0u, 0u);
  for (int v = head + 4 * nvec + (int)threadIdx.x; v < vocab; v += blockDim.x) crow[v] = 0u;
  if (threadIdx.x == 0) n_listed = 0;
  // the barrier's work-group release waits for the zero stores to complete
  // in L2, where the atomic ORs below execute (a device-scope fence would
  // write back the whole L2 of this XCD and is not needed)
  __syncthreads();
  const int p0 = prompt_indptr[i], p1 = prompt_indptr[i + 1];
  int32_t* srow = seen + (int64_t)row * cap;
  for (int k = p0 + (int)threadIdx.x; k < p1; k += blockDim.x) {
    const int t = prompt_ids[k];
    if (t < 0 || t >= vocab) {
      if (err) rkv::raise_flag(err);
      continue;
    }
    const uint32_t old = atomicOr(crow + t, kPromptBit);
    if (!(old & kPromptBit)) {
      const int at = atomicAdd(&n_listed, 1);
      if (at < cap) srow[at] = t;
      else if (err) rkv::raise_flag(err);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    seen_len[row] = min(n_listed, cap);
    out_len[row] = 0;
  }
}

// Records output token t of the request in slot `row` (row already checked):
// counted, listed if the request has not seen it before, output length + 1.
__device__ __forceinline__ void record_token(int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len,
                                             int32_t vocab, int32_t cap, int row, int t, int* err) {
  if (t < 0 || t >= vocab) {
    if (err) rkv::raise_flag(err);
    return;
  }
  uint32_t* w = (uint32_t*)counts + (int64_t)row * vocab + t;
  const uint32_t c = *w;
  const int n = seen_len[row];
  if ((c & kCountMask) != kCountMask) *w = c + 1u;
  if (c == 0u) {
    if (n < cap) {
      seen[(int64_t)row * cap + n] = t;
      seen_len[row] = n + 1;
    } else if (err) {
      rkv::raise_flag(err);
    }
  }
  out_len[row] += 1;
}

// One lane per running request.  Rows are distinct within a call, so no two
// lanes touch the same state.
__global__ __launch_bounds__(256) void penalty_accumulate_kernel(int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ seen,
                                                                int32_t* __restrict__ seen_len,
                                                                int32_t* __restrict__ out_len, int32_t n_slots,
                                                                int32_t vocab, int32_t cap, int32_t B,
                                                                const int32_t* __restrict__ rows,
                                                                const int32_t* __restrict__ tokens, int* err) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int row = rows[b];
  if (row < 0 || row >= n_slots) {
    if (err) rkv::raise_flag(err);
    return;
  }
  record_token(counts, seen, seen_len, out_len, vocab, cap, row, tokens[b], err);
}

template <typename T>
struct Logit;
template <>
struct Logit<float> {
  __device__ static float load(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
};
template <>
struct Logit<uint16_t> {
  __device__ static float load(const void* p, int64_t i) { return rkv::bf16_to_f32(((const uint16_t*)p)[i]); }
  __device__ static void store(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = rkv::f32_to_bf16(v); }
};

// One workgroup per batch entry b (state row rows[b], logits row b).  With
// RECORD, lane 0 first records new_tokens[b] (the token sampled at the
// previous step), so one launch per decode step both updates the state and
// penalizes.  Every listed token is then penalized in place; after a barrier
// (so a stop token that is also listed ends at -inf) comes the stop mask.
// The first kPer list entries of every lane are loaded together with the
// list length (the row stride cap bounds them), and then their counts and
// logits together, so the dependent gathers overlap.
template <typename T, bool RECORD>
__global__ __launch_bounds__(256) void penalty_apply_kernel(void* __restrict__ logits, int64_t ld,
                                                           const int32_t* __restrict__ rows, int32_t* counts,
                                                           int32_t* seen, int32_t* seen_len, int32_t* out_len,
                                                           int32_t n_slots, int32_t vocab, int32_t cap,
                                                           const float* __restrict__ freq,
                                                           const float* __restrict__ pres, const float* __restrict__ rep,
                                                           const int32_t* __restrict__ min_new,
                                                           const int32_t* __restrict__ stop_indptr,
                                                           const int32_t* __restrict__ stop_ids,
                                                           const int32_t* __restrict__ new_tokens, int* err) {
  using L = Logit<T>;
  constexpr int kPer = 4;
  const int b = blockIdx.x;
  const int row = rows[b];
  if (row < 0 || row >= n_slots) {
    if (threadIdx.x == 0 && err) rkv::raise_flag(err);
    return;
  }
  if constexpr (RECORD) {
    // the record and its readers are in this work-group: the barrier's
    // work-group release and acquire make the record visible to them
    if (threadIdx.x == 0) record_token(counts, seen, seen_len, out_len, vocab, cap, row, new_tokens[b], err);
    __syncthreads();
  }
  const float f = freq[b], p = pres[b], r = rep[b];
  const uint32_t* crow = (const uint32_t*)counts + (int64_t)row * vocab;
  const int32_t* srow = seen + (int64_t)row * cap;
  const int64_t lbase = (int64_t)b * ld;
  const int n = min(seen_len[row], cap);
  for (int k0 = 0; k0 == 0 || k0 < n; k0 += kPer * blockDim.x) {
    int t[kPer];
    uint32_t c[kPer];
    float x[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = k0 + u * blockDim.x + threadIdx.x;
      t[u] = k < cap ? srow[k] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = k0 + u * blockDim.x + threadIdx.x;
      if (k >= n) t[u] = -1;
      if (t[u] >= vocab) {
        if (err) rkv::raise_flag(err);
        t[u] = -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) c[u] = t[u] >= 0 ? crow[t[u]] : 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) x[u] = t[u] >= 0 ? L::load(logits, lbase + t[u]) : 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (t[u] < 0) continue;
      const uint32_t g = c[u] & kCountMask;
      float v = x[u];
      if (g != 0u || (c[u] & kPromptBit)) v = v > 0.f ? v / r : v * r;
      if (g != 0u) {
        v = fmaf(-f, (float)g, v);
        v = v - p;
      }
      L::store(logits, lbase + t[u], v);
    }
  }
  __syncthreads();
  if (out_len[row] < min_new[b]) {
    const int s0 = stop_indptr[b], s1 = stop_indptr[b + 1];
    for (int k = s0 + (int)threadIdx.x; k < s1; k += blockDim.x) {
      const int s = stop_ids[k];
      if (s < 0 || s >= vocab) {
        if (err) rkv::raise_flag(err);
        continue;
      }
      L::store(logits, lbase + s, -INFINITY);
    }
  }
}

}  // namespace

extern "C" int rkv_penalty_admit(int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len, int32_t n_slots,
                                 int32_t vocab, int32_t cap, int32_t n, const int32_t* rows,
                                 const int32_t* prompt_indptr, const int32_t* prompt_ids, void* stream) {
  rkv::clear_error();
  if (n_slots < 1 || vocab < 1 || cap < 1 || n < 0) return rkv::fail(RKV_EINVAL, "rkv_penalty_admit: bad sizes");
  if (n == 0) return RKV_OK;
  if (!counts || !seen || !seen_len || !out_len || !rows || !prompt_indptr)
    return rkv::fail(RKV_EINVAL, "rkv_penalty_admit: NULL pointer");
  if ((int64_t)n_slots * vocab > ((int64_t)1 << 40)) return rkv::fail(RKV_ENOTSUP, "rkv_penalty_admit: state too large");
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(penalty_admit_kernel, dim3((unsigned)n), dim3(256), 0, st, counts, seen, seen_len, out_len,
                     n_slots, vocab, cap, rows, prompt_indptr, prompt_ids, flag);
  return rkv::finish_launch("rkv_penalty_admit", st, flag);
}

extern "C" int rkv_penalty_accumulate(int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len,
                                      int32_t n_slots, int32_t vocab, int32_t cap, int32_t B, const int32_t* rows,
                                      const int32_t* tokens, void* stream) {
  rkv::clear_error();
  if (n_slots < 1 || vocab < 1 || cap < 1 || B < 0) return rkv::fail(RKV_EINVAL, "rkv_penalty_accumulate: bad sizes");
  if (B == 0) return RKV_OK;
  if (!counts || !seen || !seen_len || !out_len || !rows || !tokens)
    return rkv::fail(RKV_EINVAL, "rkv_penalty_accumulate: NULL pointer");
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(penalty_accumulate_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, st, counts, seen,
                     seen_len, out_len, n_slots, vocab, cap, B, rows, tokens, flag);
  return rkv::finish_launch("rkv_penalty_accumulate", st, flag);
}

extern "C" int rkv_penalty_apply(void* logits, int64_t ld, int32_t dtype, int32_t B, const int32_t* rows,
                                 int32_t* counts, int32_t* seen, int32_t* seen_len, int32_t* out_len,
                                 int32_t n_slots, int32_t vocab, int32_t cap, const float* freq, const float* pres,
                                 const float* rep, const int32_t* min_new, const int32_t* stop_indptr,
                                 const int32_t* stop_ids, const int32_t* new_tokens, void* stream) {
  rkv::clear_error();
  if (n_slots < 1 || vocab < 1 || cap < 1 || B < 0 || ld < vocab)
    return rkv::fail(RKV_EINVAL, "rkv_penalty_apply: bad sizes");
  if (dtype != RKV_F32 && dtype != RKV_BF16) return rkv::fail(RKV_ENOTSUP, "rkv_penalty_apply: dtype");
  if (B == 0) return RKV_OK;
  if (!logits || !rows || !counts || !seen || !seen_len || !out_len || !freq || !pres || !rep || !min_new ||
      !stop_indptr)
    return rkv::fail(RKV_EINVAL, "rkv_penalty_apply: NULL pointer");
  int* flag = nullptr;
  if (int rc = rkv::debug_flag(&flag)) return rc;
  hipStream_t st = (hipStream_t)stream;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)B), dim3(256), 0, st, logits, ld, rows, counts, seen, seen_len,
                       out_len, n_slots, vocab, cap, freq, pres, rep, min_new, stop_indptr, stop_ids, new_tokens, flag);
  };
  if (dtype == RKV_F32) {
    if (new_tokens) go(penalty_apply_kernel<float, true>); else go(penalty_apply_kernel<float, false>);
  } else {
    if (new_tokens) go(penalty_apply_kernel<uint16_t, true>); else go(penalty_apply_kernel<uint16_t, false>);
  }
  return rkv::finish_launch("rkv_penalty_apply", st, flag);
}
