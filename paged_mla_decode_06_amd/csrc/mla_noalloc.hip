// mla_noalloc.hip -- mla_decode_noalloc: the decode with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array lives in this file's code object: each device the library runs
// on holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory, so its device
// address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/libmla.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

// The decode's workspace (request offsets, partial LSEs, partial outputs).
// Nothing in it must start at zero: every byte a call reads it has written
// first in the same call.  Calls that overlap on one device share it.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, null until taken

// The device address of this device's copy of `scratch`, taken on the first
// call on the device.
mla_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_pool,
                                         const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                         void* stream) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  size_t need = 0;
  mla_status s = mla_decode_workspace_size(p, &need);
  if (s != MLA_OK) return s;
  if (need > kScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != MLA_OK) return s;
  return mla_decode(p, q, kv_pool, block_table, seq_lens, out, lse, ws, kScratchBytes, stream);
}
