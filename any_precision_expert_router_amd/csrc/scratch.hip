// moe_layer_forward_noalloc: the whole layer for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
// workspace is `scratch`, a file-scope device array of kScratchBytes in the library's code
// object: each GPU the library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address (in host code it names a host-side stand-in):
// the device address comes from hipGetSymbolAddress, once per device with that device
// current, and only that address is passed to the kernels.
#include <mutex>

#include "internal.hpp"

namespace moeapq {
namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_WORKSPACE_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {nullptr};

// The device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(MOE_EHIP, "could not read the current device");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                       hipGetErrorString(e));
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moeapq

using namespace moeapq;

extern "C" int moe_layer_forward_noalloc(const float* logits, const uint16_t* x, int T, int E, int H, int I,
                                         int k, const moe_apq_block* table, const moe_apq_block* shared,
                                         int I_shared, const float* shared_scale, int prefill_threshold,
                                         uint16_t* y, int32_t* status, void* stream) {
  clear_error();
  if (int rc = check_layer_args(logits, x, T, E, H, I, k, table, shared, I_shared, y)) return rc;
  if (T == 0) return MOE_OK;
  const int ish = shared ? I_shared : 0;
  const size_t need = carve_workspace(nullptr, T, E, H, I, k, ish).bytes;
  if (need > kScratchBytes)
    return set_error(MOE_EWORKSPACE,
                     "this call needs %zu bytes of workspace; the allocation-free entry point has %zu "
                     "(use moe_layer_forward with a caller-owned workspace)",
                     need, kScratchBytes);
  void* base = nullptr;
  if (int rc = scratch_address(&base)) return rc;
  const ProfilePause no_timer_events;
  const Workspace ws = carve_workspace(base, T, E, H, I, k, ish);
  return layer_forward_ws(logits, x, T, E, H, I, k, table, shared, I_shared, shared_scale, prefill_threshold,
                          y, ws, true, status, static_cast<hipStream_t>(stream));
}
