// verify_attn_mla_static: the verify step with the library's own workspace,
// for callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The workspace is a file-scope device array, `scratch`, of
// VAMLA_STATIC_WORKSPACE_BYTES.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a
// stand-in for the symbol, so its device address is looked up once per
// device, with that device current, and kept; every use goes through that
// address.  The kernels write every byte of workspace they later read (chunk
// partials, the debug record), so nothing needs clearing between calls.
// Calls on one GPU share the array: two calls in flight at once on one GPU
// (different streams, or threads) race on it.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "vamla.h"

namespace {

static __device__ __align__(256) uint8_t scratch[VAMLA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch_ptr[kMaxDevices];      // device address of `scratch`, per device (null: not looked up yet)

// The address of this device's copy of `scratch`, looked up on the first
// call on the device.  Returns VAMLA_OK or VAMLA_ERR_ARCH.
int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VAMLA_ERR_ARCH;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return VAMLA_ERR_ARCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VAMLA_OK;
}

}  // namespace

extern "C" int verify_attn_mla_static(const vamla_params* p, const uint16_t* q, const uint16_t* kv_pool,
                                      const int32_t* prefix_slot_idx, const int32_t* tree_slot_idx,
                                      const int32_t* parent, uint16_t* out, float* lse, void* stream) {
  if (!p) return VAMLA_ERR_INVALID_ARG;
  // the plan is host-only: a problem whose workspace exceeds the static
  // array is refused before any HIP call
  size_t need = 0;
  const int st = vamla_workspace_size(p, &need);
  if (st != VAMLA_OK) return st;
  if (need > (size_t)VAMLA_STATIC_WORKSPACE_BYTES) return VAMLA_ERR_STATIC_LIMIT;
  void* ws = nullptr;
  const int st2 = scratch_of_current_device(&ws);
  if (st2 != VAMLA_OK) return st2;
  vamla_params local = *p;
  local.workspace = ws;
  local.workspace_bytes = VAMLA_STATIC_WORKSPACE_BYTES;
  return verify_attn_mla(&local, q, kv_pool, prefix_slot_idx, tree_slot_idx, parent, out, lse, stream);
}
