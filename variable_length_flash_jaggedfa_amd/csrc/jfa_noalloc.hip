// Allocation-free backward: jfa_bwd with its workspace taken from a static
// device array instead of a caller-supplied buffer, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in this file's code object, so every GPU the library runs on
// holds its own copy for as long as the process lives. In host code the array's
// name is only a host-side stand-in; its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) on the first call made
// there and kept. The kernels then receive that address exactly as they receive
// a caller's workspace in jfa_bwd.
//
// Nothing in the workspace needs to start at zero: the dQ pass writes every
// -Di and -lse/scale entry (and every broadcast-Q partial) before the dK/dV pass
// reads it, in stream order. Calls that overlap on one GPU (two streams, or two
// threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "jfa_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[JFA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array.
jfa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return jfa::fail(JFA_ERR_HIP, "hipGetDevice failed");
  if (dev >= kMaxDevices)
    return jfa::fail(JFA_ERR_UNSUPPORTED, "device index " + std::to_string(dev) + " >= " +
                                              std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return jfa::fail(JFA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                        hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return JFA_OK;
}

}  // namespace

extern "C" jfa_status jfa_bwd_noalloc(const jfa_problem* p, const void* q, const void* k,
                                      const void* v, const void* out, const void* dout,
                                      const float* lse, const int32_t* offsets_dev,
                                      const int32_t* q_slot_ptr_dev, const int32_t* q_tiles_dev,
                                      int32_t q_num_slots, const int32_t* kv_slot_ptr_dev,
                                      const int32_t* kv_tiles_dev, int32_t kv_num_slots, void* dq,
                                      void* dk, void* dv, void* stream) {
  jfa::set_error("");
  if (jfa_status s = jfa::check_problem(p)) return s;
  const size_t need = jfa_bwd_workspace_bytes(p);
  if (need > size_t(JFA_NOALLOC_SCRATCH_BYTES))
    return jfa::fail(JFA_ERR_WORKSPACE,
                     "jfa_bwd_noalloc: this problem needs " + std::to_string(need) +
                         " bytes of workspace; the static scratch holds " +
                         std::to_string(size_t(JFA_NOALLOC_SCRATCH_BYTES)) +
                         " (use jfa_bwd with a caller-allocated workspace)");
  void* ws = nullptr;
  if (jfa_status s = scratch_of_current_device(&ws)) return s;
  return jfa_bwd_passes(p, q, k, v, out, dout, lse, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
                        q_num_slots, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv, ws,
                        size_t(JFA_NOALLOC_SCRATCH_BYTES), JFA_PASS_ALL, stream);
}
