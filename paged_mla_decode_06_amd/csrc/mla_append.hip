// mla_append.hip -- gfx950 kernel of libmla's KV-cache append: the cache
// write that precedes each decode step (set_mla_kv_buffer(layer,
// out_cache_loc, k_nope, k_rope) in TRTLLMMLABackend.forward_decode on
// "sglang trtllm_mla_backend.py" and "tokenspeed trtllm_mla.py").
//
// Row i = [k_nope[i] (512) | k_rope[i] (64)] lands in flat slot
// out_cache_loc[i] of the pool, i.e. page loc / P, slot loc % P.  A bf16 pool
// takes the bits unchanged; an fp8 pool takes the OCP e4m3fn code of
// x / k_scale (fp32 quotient, saturated to +-448, round to nearest even; NaN
// stores 0x7F), the per-tensor scale convention of scaled_fp8_quant in
// _quantize_fp8_qkv on "sglang trtllm_mla_backend.py".  With a rotary
// embedding (mla_kv_append_rope) the rope part is first turned at the row's
// position (mla_rope.h) and rounded to bf16, then stored or quantised.
//
// HBM-bound and embarrassingly parallel: one thread per 16-byte input chunk
// (8 bf16 elements), 72 chunks per row, consecutive threads on consecutive
// chunks, so every row is read as 1152 contiguous bytes and written as 1152
// (bf16) or 576 (fp8) contiguous bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_args.h"
#include "mla_fp8.h"
#include "mla_rope.h"

namespace mla {

typedef uint32_t app_u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t app_u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kAppendThreads = 256;
constexpr int kAppendChunks = 72;       // 16-byte chunks of a 576-wide bf16 row
constexpr int kAppendNopeChunks = 64;   // the first 64 come from k_nope

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// x / k_scale in fp32 with IEEE rounding: the quotient of two floats taken in
// double and rounded once to float is the correctly rounded float quotient
// (53 >= 2 * 24 + 2 bits), whatever the float division lowering.
__device__ __forceinline__ float scaled(float x, float k_scale) { return (float)((double)x / (double)k_scale); }

__global__ __launch_bounds__(kAppendThreads) void mla_append_kernel(AppendArgs a) {
  const int64_t n = (int64_t)a.T * kAppendChunks;
  for (int64_t ci = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x; ci < n;
       ci += (int64_t)gridDim.x * kAppendThreads) {
    const int64_t i = ci / kAppendChunks;
    const int c = (int)(ci - i * kAppendChunks);
    const int64_t loc = a.loc[i];
    if ((uint64_t)loc >= (uint64_t)a.slots) continue;   // out-of-range slots are skipped
    const uint16_t* src = c < kAppendNopeChunks ? a.nope + i * a.nope_stride + 8 * c
                                                : a.rope + i * a.rope_stride + 8 * (c - kAppendNopeChunks);
    app_u32x4_t x = *(const app_u32x4_t*)src;
    auto put = [&](int cc, app_u32x4_t v) {
      if (!a.fp8) {
        *(app_u32x4_t*)((uint16_t*)a.pool + loc * 576 + 8 * cc) = v;
      } else {
        const float s = a.k_scale;
        app_u32x2_t y;
        y[0] = e4m3fn_x4(scaled(bf16_lo(v[0]), s), scaled(bf16_hi(v[0]), s), scaled(bf16_lo(v[1]), s),
                         scaled(bf16_hi(v[1]), s));
        y[1] = e4m3fn_x4(scaled(bf16_lo(v[2]), s), scaled(bf16_hi(v[2]), s), scaled(bf16_lo(v[3]), s),
                         scaled(bf16_hi(v[3]), s));
        *(app_u32x2_t*)((uint8_t*)a.pool + loc * 576 + 8 * cc) = y;
      }
    };
    if (a.rope_cs != nullptr && c >= kAppendNopeChunks) {
      // rotary embedding of the key's rope part before it is stored: chunk
      // q holds rope dims 8q..8q+7
      const int q = c - kAppendNopeChunks;
      const float* cs = rope_row(a.rope_cs, a.positions, i, a.rope_max_pos);
      if (a.rope_neox) {
        if (q >= 4) continue;   // rotated and stored with its partner chunk q - 4
        app_u32x4_t x2 = *(const app_u32x4_t*)(src + 32);
        rope_rotate_halves(x, x2, cs, 8 * q);
        put(c + 4, x2);
      } else {
        rope_rotate_interleaved(x, cs, 8 * q);
      }
    }
    put(c, x);
  }
}

}  // namespace mla

extern "C" hipError_t mla_launch_append(const mla::AppendArgs* a, hipStream_t stream) {
  const int64_t chunks = (int64_t)a->T * mla::kAppendChunks;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + mla::kAppendThreads - 1) / mla::kAppendThreads;
  if (blocks > (1 << 20)) blocks = 1 << 20;   // the grid-stride loop covers the rest
  hipLaunchKernelGGL(mla::mla_append_kernel, dim3((unsigned)blocks), dim3(mla::kAppendThreads), 0, stream, *a);
  return hipGetLastError();
}
