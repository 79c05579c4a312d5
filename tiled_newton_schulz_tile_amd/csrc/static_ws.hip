// himuon_step_static: the HiMuon step with the large-tile path's workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot allocate
// device memory (code under HIP graph capture, tight loops, harnesses that forbid it).
//
// The array is one per GPU the library runs on (each device holds its own copy, at its
// own address) and lives until the process ends.  Its address is taken once per device
// with hipGetSymbolAddress; host code uses that address only, never the array's name
// (which, on the host, only stands in for the symbol).  Calls on one GPU share the array:
// two steps that overlap on one device race on it.  Nothing in it has to start at zero:
// every kernel of the large-tile path writes each workspace plane (zero padding included)
// before any kernel of the same step reads it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "himuon.h"
#include "himuon_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[HIMUON_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_ptr[kMaxDevices];   // device address of scratch, per device
std::mutex g_mu;

// The device address of this device's scratch array (taken on the first call on it).
hipError_t scratch_of(int dev, void **out) {
  void *p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" HIMUON_API himuon_status himuon_step_static(himuon_plan_t *p, float lr, void *hip_stream) {
  if (!p) return himuon_step(nullptr, nullptr, 0, lr, hip_stream);   // the usual EINVAL
  size_t need = 0;
  himuon_status s = himuon_workspace_size(p, &need);
  if (s != HIMUON_OK) return s;
  if (need == 0) return himuon_step(p, nullptr, 0, lr, hip_stream);   // fused path only
  if (need > (size_t)HIMUON_STATIC_WORKSPACE_BYTES)
    return himuon::set_error(HIMUON_EBUDGET,
                             "himuon_step_static: the plan needs " + std::to_string(need) +
                                 " B of workspace, more than the static workspace of " +
                                 std::to_string((size_t)HIMUON_STATIC_WORKSPACE_BYTES) +
                                 " B; plan with workspace_budget <= HIMUON_STATIC_WORKSPACE_BYTES "
                                 "(smaller chunks) or call himuon_step");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return himuon::set_error(HIMUON_EDEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return himuon::set_error(HIMUON_EUNSUPPORTED, "himuon_step_static: device index beyond 63");
  void *ws = nullptr;
  if ((e = scratch_of(dev, &ws)) != hipSuccess)
    return himuon::set_error(HIMUON_EDEVICE, std::string("hipGetSymbolAddress of the static workspace: ") +
                                                 hipGetErrorString(e));
  return himuon_step(p, ws, (size_t)HIMUON_STATIC_WORKSPACE_BYTES, lr, hip_stream);
}
