// moe_unpermute_noalloc: moe_unpermute whose workspace is a static device array of the
// library instead of caller memory, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It runs
// exactly the kernels of moe_unpermute; only where the workspace lives differs.
#include <mutex>

#include "internal.hpp"

namespace ffnwb {

// The workspace of every moe_unpermute_noalloc call on a GPU.  Each GPU the library runs
// on holds its own copy, at its own address, until the process ends.  The unpermute's
// kernels need no part of their workspace cleared, so the contents left by the previous
// call do not matter.  Calls that overlap on one GPU share it and race.
static __device__ __align__(256) uint8_t scratch[FFNWB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];

int stream_device(hipStream_t s) {
  if (s != nullptr) return hipGetStreamDeviceId(s);
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

// The device address of `scratch` on device `dev`, looked up once per device with that
// device current (in host code the array's name is only a stand-in for it).
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    if (!have_cur || cur != dev) {
      if (hipSetDevice(dev) != hipSuccess) return;
    }
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = p;
    if (have_cur && cur != dev) (void)hipSetDevice(cur);
  });
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace ffnwb

using namespace ffnwb;

extern "C" int moe_unpermute_noalloc(const moe_unpermute_desc* d, void* stream) {
  UnpermutePlan p;
  const int st = plan_unpermute(d, &p);
  if (st != FFNWB_OK) return st;
  if (p.ws_bytes > FFNWB_NOALLOC_SCRATCH_BYTES) return FFNWB_ERR_SCRATCH;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = scratch_on(stream_device(s));
  if (ws == nullptr) return FFNWB_ERR_RUNTIME;
  return launch_unpermute(d, p, ws, s);
}
