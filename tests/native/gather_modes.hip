// Gather-rate probe for the grouped-head decode pattern on one MI355X: 256-byte
// reads at offset g*256 inside random 2 KB slot rows of an 8 GiB pool (a slot
// of 8 kv heads x 128 bf16), with g chosen per mode:
//   0: g = 0 for every row, 1: g = the XCD of the block (blockIdx % 8),
//   2: g = row % 8, 3: whole 2 KB rows (two 1 KB runs per row).
// U rows in flight per group of 16 lanes (16 B per lane).  Slots are below
// pool / 2 KB and row indices are clamped to the slot list, so every access
// stays inside its buffer.  Prints one line per mode.
// Build: hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops gather_modes.hip -o gather_modes
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int U, int MODE>
__global__ __launch_bounds__(256) void g(const char* __restrict__ pool, const int* __restrict__ slots, int nrows,
                                         uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * 256) >> 6;
  uint32_t acc = 0;
  // MODE 3: a 2 KB row is read by 2 instructions of 64 lanes x 16 B (1 KB each)
  constexpr int RPW = MODE == 3 ? 1 : 4;       // rows per instruction
  constexpr int RUNS = MODE == 3 ? 2 : 1;
  for (int base = wave * U * RPW; base < nrows; base += nwaves * U * RPW) {
    u32x4 v[U][RUNS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(base + u * RPW + (MODE == 3 ? 0 : lane / 16), nrows - 1);
      int gg = 0;
      if (MODE == 1) gg = blockIdx.x & 7;
      if (MODE == 2) gg = r & 7;
      const char* rp = pool + (size_t)slots[r] * 2048 + (MODE == 3 ? lane * 16 : gg * 256 + (lane % 16) * 16);
#pragma unroll
      for (int q = 0; q < RUNS; ++q) v[u][q] = *(const u32x4*)(rp + q * 1024);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < RUNS; ++q) acc ^= v[u][q][0] ^ v[u][q][3];
  }
  if (acc == 0x12345678u) out[0] = acc;
}
template <int U, int MODE>
void run(const char* pool, const int* slots, int nrows, uint32_t* out) {
  hipEvent_t a, b; (void)hipEventCreate(&a); (void)hipEventCreate(&b);
  const int grid = 8192;
  hipLaunchKernelGGL((g<U, MODE>), dim3(grid), dim3(256), 0, 0, pool, slots, nrows, out);
  (void)hipDeviceSynchronize();
  (void)hipEventRecord(a);
  for (int i = 0; i < 5; ++i) hipLaunchKernelGGL((g<U, MODE>), dim3(grid), dim3(256), 0, 0, pool, slots, nrows, out);
  (void)hipEventRecord(b); (void)hipEventSynchronize(b);
  float ms = 0; (void)hipEventElapsedTime(&ms, a, b);
  const double bytes = (double)nrows * (MODE == 3 ? 2048 : 256) * 5;
  std::printf("mode %d U=%2d: %.0f GB/s\n", MODE, U, bytes / (ms * 1e-3) / 1e9);
}
int main() {
  const size_t pool_bytes = (size_t)8 << 30;
  const int total = (int)(pool_bytes / 2048);            // 2 KB slot rows
  char* pool; uint32_t* out; int* slots;
  if (hipMalloc(&pool, pool_bytes) != hipSuccess || hipMalloc(&out, 64) != hipSuccess) return 1;
  if (hipMemset(pool, 3, pool_bytes) != hipSuccess) return 2;
  const int nrows = 1 << 23;                            // 8M rows: 2 GiB of 256 B gathers
  if (hipMalloc(&slots, (size_t)nrows * 4) != hipSuccess) return 3;
  std::vector<int> h(nrows);
  uint64_t x = 88172645463325252ull;
  for (int i = 0; i < nrows; ++i) { x ^= x << 13; x ^= x >> 7; x ^= x << 17; h[i] = (int)(x % (uint64_t)total); }
  if (hipMemcpy(slots, h.data(), (size_t)nrows * 4, hipMemcpyHostToDevice) != hipSuccess) return 4;
  run<8, 0>(pool, slots, nrows, out);
  run<8, 1>(pool, slots, nrows, out);
  run<8, 2>(pool, slots, nrows, out);
  run<16, 2>(pool, slots, nrows, out);
  run<4, 3>(pool, slots, nrows / 8, out);
  return 0;
}
