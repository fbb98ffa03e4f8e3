// host_stubs.cpp -- stand-ins for the device side of libmla, so that the host
// code (argument checks, workspace layout, the planner's host mirror) can be
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// exercised without a GPU: every launcher reports failure, and the HIP
// runtime calls behave as on a machine with no device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libmla.h"
#include "mla_args.h"

extern "C" {

hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600*, int) { return hipErrorNoDevice; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNoDevice; }

hipError_t mla_launch_split(const mla::SplitArgs*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t mla_launch_combine(const mla::CombineArgs*, hipStream_t) { return hipErrorNoDevice; }
hipError_t mla_launch_gather(const void*, const int32_t*, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                             int32_t, int32_t, void*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t mla_launch_plan(const int32_t*, int32_t, int32_t, int32_t, int32_t, int64_t, int32_t, int32_t, int32_t*,
                           int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t mla_launch_append(const mla::AppendArgs*, hipStream_t) { return hipErrorNoDevice; }
mla_status mla_decode_noalloc(const mla_decode_params*, const void*, const void*, const int32_t*, const int32_t*,
                              void*, float*, void*) {
  return MLA_ERR_HIP;
}

}  // extern "C"
