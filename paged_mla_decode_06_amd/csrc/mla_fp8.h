// mla_fp8.h -- OCP e4m3fn encoding on gfx950, shared by the KV-cache append
// and the split kernel's fp8 query.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Four floats to four e4m3fn codes (byte e = code of v[e]): saturate to
// +-448, then the gfx950 conversion (round to nearest even, OCP e4m3fn); NaN
// becomes 0x7F.
__device__ __forceinline__ uint32_t e4m3fn_x4(float v0, float v1, float v2, float v3) {
  const float v[4] = {v0, v1, v2, v3};
  float c[4];
  uint32_t nan_mask = 0;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const bool nan = v[e] != v[e];
    nan_mask |= nan ? (0xFFu << (8 * e)) : 0u;
    c[e] = nan ? 0.f : __builtin_fminf(__builtin_fmaxf(v[e], -448.f), 448.f);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return ((uint32_t)w & ~nan_mask) | (0x7F7F7F7Fu & nan_mask);
}

}  // namespace mla
