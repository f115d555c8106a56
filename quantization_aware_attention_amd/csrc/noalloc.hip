// qat_attn_bwd_noalloc: the backward with no allocation and no workspace
// argument.  Its scratch (Delta, and with Q/K/V quantization the quantized
// copies) lives in one file-scope
// device array, `scratch`, that every GPU the library runs on holds from
// module load until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address is taken once
// per device with hipGetSymbolAddress and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qat_attn.h"
#include "api_internal.hpp"

static __device__ __align__(256) char scratch[QAT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of this device's `scratch` (the current device), looked up
// on the first call on that device.  Null on failure.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int qat_attn_bwd_noalloc(const qat_attn_dims* dims, const void* q, const void* k, const void* v,
                                    const float* v_scale, const void* o_hp, const float* lse, const void* dout,
                                    float sm_scale, int causal, uint32_t quant_flags, void* dq, void* dk,
                                    void* dv, void* stream) {
  if (!dims) return QAT_EINVAL;
  const size_t need = qat::bwd_bytes_whole(dims, quant_flags);
  if (need > QAT_NOALLOC_SCRATCH_BYTES) return QAT_ESCRATCH;
  void* ws = device_scratch();
  if (!ws) return QAT_EHIP;
  // every other check (arguments, flags, shapes) is bwd_impl's, before any launch
  return qat::bwd_impl(dims, q, k, v, v_scale, o_hp, lse, dout, sm_scale, causal, quant_flags, dq, dk, dv, ws,
                       QAT_NOALLOC_SCRATCH_BYTES, QAT_BWD_ALL, false, stream);
}
