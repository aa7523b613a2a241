// Achievable-peak probes on one MI355X, for context beside the spec peaks:
//   stream_read  sums a 4 GiB buffer (16-byte loads, grid-stride)
//   copy         copies 1 GiB (16-byte loads and stores); also the calibration
//                kernel for FETCH_SIZE / WRITE_SIZE (known bytes per launch)
//   row_gather   reads 256-byte rows of random slots from an 8 GiB pool, the
//                access pattern of decode attention with one kv head per row
//   mfma_loop    back-to-back independent v_mfma_f32_16x16x32_bf16
// Prints one JSON line.  Every index stays inside its buffer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define HIP_OK(x)                                              \
  do {                                                         \
    if ((x) != hipSuccess) {                                   \
      std::fprintf(stderr, "HIP error at line %d\n", __LINE__); \
      std::exit(1);                                            \
    }                                                          \
  } while (0)

__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ p, size_t n, uint32_t* out) {
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x12345678u) out[0] = acc;  // keeps the loads alive
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

// 16 lanes per 256-byte row; 8 rows in flight per lane.
__global__ __launch_bounds__(256) void row_gather(const uint4* __restrict__ pool, const int* __restrict__ slots,
                                                  int nrows, int row_chunks, uint32_t* out) {
  const int lane16 = threadIdx.x & 15;
  const int group = (blockIdx.x * 256 + threadIdx.x) >> 4;
  const int ngroups = (gridDim.x * 256) >> 4;
  uint32_t acc = 0;
  for (int base = group * 8; base < nrows; base += ngroups * 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(base + u, nrows - 1);
      v[u] = pool[(size_t)slots[r] * row_chunks + lane16];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].w;
  }
  if (acc == 0x12345678u) out[0] = acc;
}

__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (threadIdx.x - i));
  }
  f32x4 c[8];
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == 123.456f) out[0] = s;
}

template <typename F>
static float time_ms(F launch, int reps) {
  hipEvent_t a, b;
  HIP_OK(hipEventCreate(&a));
  HIP_OK(hipEventCreate(&b));
  launch();
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipEventRecord(a));
  for (int i = 0; i < reps; ++i) launch();
  HIP_OK(hipEventRecord(b));
  HIP_OK(hipEventSynchronize(b));
  float ms = 0.f;
  HIP_OK(hipEventElapsedTime(&ms, a, b));
  return ms / reps;
}

int main() {
  const size_t big = (size_t)4 << 30, cp = (size_t)1 << 30, pool_bytes = (size_t)8 << 30;
  uint4 *buf = nullptr, *dst = nullptr, *pool = nullptr;
  uint32_t* out = nullptr;
  float* fout = nullptr;
  HIP_OK(hipMalloc(&buf, big));
  HIP_OK(hipMalloc(&dst, cp));
  HIP_OK(hipMalloc(&pool, pool_bytes));
  HIP_OK(hipMalloc(&out, 64));
  HIP_OK(hipMalloc(&fout, 64));
  HIP_OK(hipMemset(buf, 1, big));
  HIP_OK(hipMemset(pool, 2, pool_bytes));
  // random distinct rows: 2^25 rows of 256 B in 8 GiB; gather 2^22 of them
  const int total_rows = (int)(pool_bytes / 256), nrows = 1 << 22;
  std::vector<int> h(nrows);
  uint64_t x = 88172645463325252ull;
  for (int i = 0; i < nrows; ++i) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    h[i] = (int)(x % (uint64_t)total_rows);
  }
  int* slots = nullptr;
  HIP_OK(hipMalloc(&slots, nrows * sizeof(int)));
  HIP_OK(hipMemcpy(slots, h.data(), nrows * sizeof(int), hipMemcpyHostToDevice));

  const int grid = 256 * 32;
  const float t_read = time_ms([&] { hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, 0, buf, big / 16, out); }, 10);
  const float t_copy = time_ms([&] { hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, buf, dst, cp / 16); }, 10);
  const float t_gather = time_ms([&] { hipLaunchKernelGGL(row_gather, dim3(grid), dim3(256), 0, 0, pool, slots, nrows, 16, out); }, 10);
  const int iters = 4096;
  const float t_mfma = time_ms([&] { hipLaunchKernelGGL(mfma_loop, dim3(256 * 8), dim3(256), 0, 0, iters, fout); }, 3);
  const double mfma_flops = 256.0 * 8 * 4 * iters * 8 * (16.0 * 16 * 32 * 2);
  std::printf("{\"stream_read_gbs\": %.1f, \"copy_gbs\": %.1f, \"copy_bytes_per_launch\": %zu, "
              "\"row_gather_256B_gbs\": %.1f, \"mfma_bf16_tflops\": %.1f}\n",
              big / (t_read * 1e-3) / 1e9, 2.0 * cp / (t_copy * 1e-3) / 1e9, 2 * cp,
              (double)nrows * 256 / (t_gather * 1e-3) / 1e9, mfma_flops / (t_mfma * 1e-3) / 1e12);
  HIP_OK(hipFree(buf)); HIP_OK(hipFree(dst)); HIP_OK(hipFree(pool)); HIP_OK(hipFree(out));
  HIP_OK(hipFree(fout)); HIP_OK(hipFree(slots));
  return 0;
}
