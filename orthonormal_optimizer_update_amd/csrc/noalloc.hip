// dion_step_noalloc: dion_step with its workspace taken from a static device
// array instead of a caller buffer, for callers that cannot allocate.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ortho.h"
#include "plan.h"
#include "run.h"

namespace {

constexpr size_t kScratchBytes = ORTHO_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU, alive until the process ends.  Host code never passes the
// array's name to a kernel or a copy (on the host it only names the symbol):
// every use goes through the device address that hipGetSymbolAddress returns
// for the current device.
static __device__ __align__(256) char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device with that
// device current.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    d.ptr = d.err == hipSuccess ? p : nullptr;
  });
  if (d.err != hipSuccess) return d.err;
  if (d.ptr == nullptr) return hipErrorInvalidSymbol;
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace

extern "C" ortho_status dion_step_noalloc(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q,
                                         int32_t r, float mu, float lr, void* stream) {
  using namespace ortho;
  // Argument errors exactly as dion_step reports them; the workspace test is
  // given an aligned stand-in that is never dereferenced.
  const ortho_status st = validate_dion(1, &X, &G, &M, &Q, r, mu, lr, 1.0f, nullptr, nullptr,
                                        reinterpret_cast<const void*>(kWsAlign), SIZE_MAX);
  if (st != ORTHO_OK) return st;
  DionPlan plan;
  if (!plan_dion(X.rows, X.cols, r, 1, &plan)) return ORTHO_E_SHAPE;
  if (plan.total_bytes > kScratchBytes) return ORTHO_E_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return ORTHO_E_HIP;
  return dion_run(1, &X, &G, &M, &Q, r, mu, lr, 1.0f, ws, stream);
}
