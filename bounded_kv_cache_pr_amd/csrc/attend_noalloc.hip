// pr_sink_attend without a caller-side workspace: the rotated keys of the
// current block, the only per-call scratch an unsplit attention call needs,
// go to a static device array of this library instead of the arena, so a
// caller that must not allocate (code under stream capture, serving loops)
// can still issue the call on any cache.
//
// The array lives for the whole process on every GPU the library runs on.
// Host code never passes its name to a kernel: that would be a host-side
// stand-in, not a device address.  Its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept in a
// per-device table; kernels receive that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pr_sink.h"
#include "prsink_internal.h"

namespace {

// 64 MiB: the rotated keys of one block of up to 64 MiB (a 480x480 block of
// 40 heads x 128 dims in bf16 is 27.6 MB, 384x672 is 31.0 MB).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_lock;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// Device address of the scratch array on the current device.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int pr_sink_attend_noalloc(pr_sink_cache* c, int32_t layer, const void* q_raw,
                                      const void* k_cur_raw, const void* v_cur_raw, void* out,
                                      void* stream) {
  prsink::AttendWorkspace ws{nullptr, kScratchBytes};
  if (c && !prsink::cache_is_dry(c)) {  // a dry-run cache never touches a device
    const hipError_t e = scratch_ptr(&ws.cur_rot);
    if (e != hipSuccess) return prsink::report_hip_error(e, "hipGetSymbolAddress(scratch)");
  }
  return prsink::attend_with_workspace(c, layer, q_raw, k_cur_raw, v_cur_raw, out, stream, &ws);
}
