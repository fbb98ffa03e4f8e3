// mla_rope.h -- rotary embedding of the 64-wide rope part (internal to the
// GPU path): the 32 pairs (x1, x2) of a row, pairs (i, i+32) in the
// rotate-half layout or (2i, 2i+1) interleaved, turned by the angle whose
// cosine and sine are columns i and 32+i of the cos/sin cache row of the
// token's position:  y1 = x1 cos - x2 sin,  y2 = x2 cos + x1 sin.
// Each product and the difference or sum is rounded to fp32 (contraction
// into fused multiply-adds is off here), the results to bf16 (nearest even).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint32_t rope_u32x4_t __attribute__((ext_vector_type(4)));
typedef float rope_f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 rope_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float rope_f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float rope_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float rope_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t rope_pack(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((rope_f32x2_t){lo, hi}, rope_bf16x2_t));
}

__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float s, float& y1, float& y2) {
#pragma clang fp contract(off)
  const float a = x1 * c, b = x2 * s, d = x2 * c, e = x1 * s;
  y1 = a - b;
  y2 = d + e;
}

// Rotate-half layout: element k of `lo` (rope dim d0 + k, d0 < 32) pairs with
// element k of `hi` (rope dim 32 + d0 + k); cs = the cache row.
__device__ __forceinline__ void rope_rotate_halves(rope_u32x4_t& lo, rope_u32x4_t& hi, const float* cs, int d0) {
  const rope_f32x4_t c0 = *(const rope_f32x4_t*)(cs + d0), c1 = *(const rope_f32x4_t*)(cs + d0 + 4);
  const rope_f32x4_t s0 = *(const rope_f32x4_t*)(cs + 32 + d0), s1 = *(const rope_f32x4_t*)(cs + 32 + d0 + 4);
  const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  rope_u32x4_t a = lo, b = hi;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    float y1l, y2l, y1h, y2h;
    rope_pair(rope_lo(lo[w]), rope_lo(hi[w]), c[2 * w], s[2 * w], y1l, y2l);
    rope_pair(rope_hi(lo[w]), rope_hi(hi[w]), c[2 * w + 1], s[2 * w + 1], y1h, y2h);
    a[w] = rope_pack(y1l, y1h);
    b[w] = rope_pack(y2l, y2h);
  }
  lo = a;
  hi = b;
}

// Interleaved layout: the 8 elements of `x` (rope dims d0 .. d0+7, d0 even)
// are the pairs i = d0/2 .. d0/2+3.
__device__ __forceinline__ void rope_rotate_interleaved(rope_u32x4_t& x, const float* cs, int d0) {
  const rope_f32x4_t c = *(const rope_f32x4_t*)(cs + d0 / 2), s = *(const rope_f32x4_t*)(cs + 32 + d0 / 2);
  rope_u32x4_t y = x;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    float y1, y2;
    rope_pair(rope_lo(x[w]), rope_hi(x[w]), c[w], s[w], y1, y2);
    y[w] = rope_pack(y1, y2);
  }
  x = y;
}

// The cache row of a position, clamped into the cache.
__device__ __forceinline__ const float* rope_row(const float* cs, const int64_t* positions, int64_t t, int32_t max_pos) {
  int64_t p = positions[t];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  return cs + p * 64;
}

}  // namespace mla
