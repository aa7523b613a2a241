// Host-side launch bookkeeping shared by the device entry points.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "device.h"
#include "rkv.h"
#include "rkv_internal.h"

namespace rkv {

namespace {
std::mutex g_flag_mu;
int* g_flags[64] = {nullptr};
}  // namespace

int debug_flag(int** out) {
  *out = nullptr;
  if (!debug_mode()) return RKV_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(RKV_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_flag_mu);
  if (!g_flags[dev]) {
    int* p = nullptr;
    if (hipMalloc(&p, sizeof(int)) != hipSuccess) return fail(RKV_EHIP, "hipMalloc of the debug flag failed");
    if (hipMemset(p, 0, sizeof(int)) != hipSuccess) return fail(RKV_EHIP, "hipMemset of the debug flag failed");
    g_flags[dev] = p;
  }
  *out = g_flags[dev];
  return RKV_OK;
}

int finish_launch(const char* what, hipStream_t stream, int* flag) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RKV_EHIP, std::string(what) + ": launch failed: " + hipGetErrorString(e));
  if (!flag) return RKV_OK;
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(RKV_EHIP, std::string(what) + ": sync failed");
  int h = 0;
  if (hipMemcpy(&h, flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RKV_EHIP, std::string(what) + ": reading the debug flag failed");
  if (h) {
    int zero = 0;
    (void)hipMemcpy(flag, &zero, sizeof(int), hipMemcpyHostToDevice);
    return fail(RKV_EINVAL, std::string(what) + ": an index (slot, token, request or plan entry) was out of range");
  }
  return RKV_OK;
}

}  // namespace rkv
