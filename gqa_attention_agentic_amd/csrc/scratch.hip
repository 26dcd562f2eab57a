// Library-owned device scratch for forwards that must not allocate
// (gqa_attn_forward_noalloc): the plan, the arrival counters and the
// split-KV partials of such a forward live in one static device array per
// GPU instead of buffers the handle allocates.
//
// The array's host-side name is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, looked up once per device (with
// that device current) and kept here. Every user of the scratch takes that
// address, never the array's name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

static __device__ __align__(256) char scratch[gqa::kScratchBytes];

constexpr int kMaxDevices = 64;

struct Slot {
  void* ptr = nullptr;   // device address of `scratch` on this device
  bool cleared = false;  // its counter region has been zero-filled
};

std::mutex g_mu;
Slot g_slot[kMaxDevices];

}  // namespace

namespace gqa {

hipError_t scratch_setup(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  Slot& s = g_slot[device];
  if (!s.ptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    s.ptr = p;
  }
  if (!s.cleared) {
    // The counters must start at zero; every forward leaves them at zero.
    hipError_t e = launch_zero_i32((int32_t*)s.ptr, (int64_t)(kScratchCounterBytes / sizeof(int32_t)), nullptr);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) return e;
    s.cleared = true;
  }
  *ptr = s.ptr;
  return hipSuccess;
}

}  // namespace gqa
