// Forward pass for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): jfa_forward_noalloc runs the forward
// exactly as jfa_forward does, with its workspace in a fixed device array instead of a
// caller-allocated buffer.
//
// The array (`scratch`, JFA_NOALLOC_SCRATCH_BYTES) is a file-scope device variable: every GPU
// the library runs on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.  Every call on a GPU shares that GPU's array, so calls that overlap on one
// GPU (concurrent streams or threads) race; calls ordered on one stream do not.  The forward's
// scheduler rewrites everything a call reads back (list counts, work tickets, status) at the
// start of every call, so nothing carries over from the previous call.
#include <mutex>
#include <unordered_map>

#include "jfa_internal.h"

namespace jfa {

static __device__ __align__(256) unsigned char scratch[JFA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device (looked up once per device).
jfa_status scratch_of_current_device(void** out) {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return JFA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *out = it->second;
    return JFA_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
    return JFA_ERR_LAUNCH;
  addr[dev] = ptr;
  *out = ptr;
  return JFA_OK;
}

}  // namespace
}  // namespace jfa

extern "C" jfa_status jfa_forward_noalloc(const jfa_problem* p, const void* q, const void* k,
                                          const void* v, const uint8_t* q_scale,
                                          const uint8_t* k_scale, const uint8_t* v_scale,
                                          const int32_t* q_offsets, const int32_t* kv_offsets,
                                          const void* bias, void* o, float* lse, void* stream) {
  const size_t need = jfa_workspace_bytes(p, 0);
  if (need == 0) {
    // an invalid problem: jfa_forward reports why (it returns before touching the workspace)
    return jfa_forward(p, q, k, v, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, o,
                       lse, nullptr, 0, stream);
  }
  if (need > JFA_NOALLOC_SCRATCH_BYTES) return JFA_ERR_WORKSPACE;
  void* ws = nullptr;
  const jfa_status st = jfa::scratch_of_current_device(&ws);
  if (st != JFA_OK) return st;
  return jfa_forward(p, q, k, v, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, o, lse,
                     ws, JFA_NOALLOC_SCRATCH_BYTES, stream);
}
