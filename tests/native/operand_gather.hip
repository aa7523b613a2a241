// Gather-rate probe: the two operand patterns of the grouped-head decode walk
// over random 256-byte rows (one kv head of a 2 KB slot row):
//   mode 0 (K operands): per instruction 16 rows x 64 B; lane (l16 = row,
//          gq = lane / 16) reads bytes gq*16 + k*64 of its row, k = 0..3
//   mode 1 (V tile):     per instruction 4 rows x 256 B; 16 consecutive lanes
//          per row
// Each wave keeps U groups of 4 instructions (16 KB) in flight.  Slots are
// below pool / 2 KB and row indices are clamped to the slot list, so every
// access stays inside its buffer.  Prints one line per (grid, mode, U).
// Build: hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops operand_gather.hip -o operand_gather
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int MODE, int U>
__global__ __launch_bounds__(256) void g(const char* __restrict__ pool, const int* __restrict__ slots, int nrows,
                                         uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * 256) >> 6;
  uint32_t acc = 0;
  // one group = 16 rows (mode 0) or 16 rows as 4 instructions x 4 rows (mode 1)
  for (int base = wave * 16 * U; base < nrows; base += nwaves * 16 * U) {
    u32x4 v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        int r;
        int off;
        if (MODE == 0) { r = base + u * 16 + (lane & 15); off = (lane >> 4) * 16 + k * 64; }
        else { r = base + u * 16 + k * 4 + (lane >> 4); off = (lane & 15) * 16; }
        r = min(r, nrows - 1);
        v[u][k] = *(const u32x4*)(pool + (size_t)slots[r] * 2048 + (slots[r] & 7) * 256 + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[u][k][0] ^ v[u][k][3];
  }
  if (acc == 0x12345678u) out[0] = acc;
}
template <int MODE, int U>
void run(const char* pool, const int* slots, int nrows, uint32_t* out, int grid) {
  hipEvent_t a, b; (void)hipEventCreate(&a); (void)hipEventCreate(&b);
  hipLaunchKernelGGL((g<MODE, U>), dim3(grid), dim3(256), 0, 0, pool, slots, nrows, out);
  (void)hipDeviceSynchronize();
  (void)hipEventRecord(a);
  for (int i = 0; i < 5; ++i) hipLaunchKernelGGL((g<MODE, U>), dim3(grid), dim3(256), 0, 0, pool, slots, nrows, out);
  (void)hipEventRecord(b); (void)hipEventSynchronize(b);
  float ms = 0; (void)hipEventElapsedTime(&ms, a, b);
  std::printf("mode %d U=%d grid %d: %.0f GB/s\n", MODE, U, grid, (double)nrows * 256 * 5 / (ms * 1e-3) / 1e9);
}
int main() {
  const size_t pool_bytes = (size_t)8 << 30;
  const int total = (int)(pool_bytes / 2048);
  char* pool; uint32_t* out; int* slots;
  if (hipMalloc(&pool, pool_bytes) != hipSuccess || hipMalloc(&out, 64) != hipSuccess) return 1;
  if (hipMemset(pool, 3, pool_bytes) != hipSuccess) return 2;
  const int nrows = 1 << 23;
  if (hipMalloc(&slots, (size_t)nrows * 4) != hipSuccess) return 3;
  std::vector<int> h(nrows);
  uint64_t x = 88172645463325252ull;
  for (int i = 0; i < nrows; ++i) { x ^= x << 13; x ^= x >> 7; x ^= x << 17; h[i] = (int)(x % (uint64_t)total); }
  if (hipMemcpy(slots, h.data(), (size_t)nrows * 4, hipMemcpyHostToDevice) != hipSuccess) return 4;
  for (int grid : {512, 2048, 8192}) {
    run<0, 1>(pool, slots, nrows, out, grid);
    run<1, 1>(pool, slots, nrows, out, grid);
    run<0, 2>(pool, slots, nrows, out, grid);
    run<1, 2>(pool, slots, nrows, out, grid);
  }
  return 0;
}
