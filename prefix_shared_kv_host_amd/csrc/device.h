// Device-side helpers for the gfx950 kernels: bf16 conversion, wavefront
// reductions, the XCD-aware block order, and the debug error flag.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace rkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with its own L2.  Work item = (block % 8) * (grid / 8) + block / 8 hands
// every XCD one contiguous range of work items, so items that read the same
// K/V rows (same kv head, neighbouring requests) share an L2.  The grid is
// always a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_work_item(int64_t block, int64_t grid) {
  const int64_t per = grid / kXcds;
  return (block % kXcds) * per + block / kXcds;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16x2 (lo in bits 0..15), RNE, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// DPP lane exchange inside one row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16

// Sum over aligned groups of LANES consecutive lanes (LANES in 2..64); every
// lane of the group receives the sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES >= 2 && LANES <= 64 && (LANES & (LANES - 1)) == 0, "power of two");
  x += dpp<kDppXor1>(x);
  if (LANES >= 4) x += dpp<kDppXor2>(x);
  if (LANES >= 8) x += dpp<kDppHalfMirror>(x);
  if (LANES >= 16) x += dpp<kDppMirror>(x);
  if (LANES >= 32) x += __shfl_xor(x, 16);
  if (LANES >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Max over lanes l and l^32 (resp. l^16): gfx950 permlane swaps exchange
// the two 32-lane halves (resp. neighbouring 16-lane rows) in VALU, without
// an LDS round trip.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// Raises the debug error flag (a plain vector store; any writer stores 1).
__device__ __forceinline__ void raise_flag(int* err) {
  if (err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace rkv

// Host side: launch checks and the debug flag.
namespace rkv {
// Device pointer of this device's error flag (allocated on first use), or
// nullptr when RKV_DEBUG is off.  Returns RKV_EHIP on a runtime failure.
int debug_flag(int** out);
// After a launch: checks hipGetLastError; in debug mode synchronizes the
// stream and turns a raised flag into RKV_EINVAL.
int finish_launch(const char* what, hipStream_t stream, int* flag);
}  // namespace rkv
