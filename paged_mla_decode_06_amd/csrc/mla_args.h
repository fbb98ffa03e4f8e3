// mla_args.h -- kernel argument blocks and launchers of libmla (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct SplitArgs {
  const uint16_t* q;        // latent part of query row (token, h): q + token*qn_tok + h*qn_head, 512 bf16
  const uint16_t* q_rope;   // rope part: q_rope + token*qr_tok + h*qr_head, 64 bf16 (token = b*q_len + j)
  int64_t qn_tok, qn_head, qr_tok, qr_head;   // element strides
  const void* pool;         // [N][P][576] bf16 or e4m3fn
  const int32_t* bt;        // [B][W]
  const int32_t* seq_lens;  // [B]
  uint16_t* out;            // [B][q_len][H][512] bf16
  float* lse;               // [B][q_len][H] or null
  uint16_t* part_o;         // [slots][64][512] bf16, normalised partial outputs
  float* part_lse;          // [slots][64]
  int32_t* pos_off_ws;      // [B+1] cost-position offsets (balanced mode), written by workgroup 0
  const int32_t* qo_indptr;  // ragged batch: request b's query tokens are [qo_indptr[b], qo_indptr[b+1]); null: b*q_len + j
  int32_t total_q;          // ragged batch: query tokens in q / out (bounds the offsets)
  // rotary embedding of the query's rope part (null rope_cs: none): token t
  // is turned by row clamp(positions[t], 0, rope_max_pos-1) of rope_cs
  const int64_t* positions;
  const float* rope_cs;     // [rope_max_pos][64] fp32: cos 0..31, sin 32..63
  int32_t rope_max_pos, rope_neox;
  int32_t B, q_len, H, P, W, N, max_seq_len, nrb, R, num_splits;
  int32_t p_shift;          // log2(P)
  // ragged batch, balanced mode: plan the requests in row-block classes
  // when they fit (class_S workgroup slots in all, class_C per XCD);
  // class_tab receives the plan for the combine
  int32_t class_plan, class_S, class_C;
  int32_t* class_tab;
  int32_t vg_per;           // plan groups walked by each launched group (balanced mode), else 1
  int64_t NG;               // groups of the plan
  int64_t NGL;              // groups of the launch: ceil(NG / vg_per)
  float scale_log2;         // softmax_scale * (k_scale for fp8) * log2(e)
  float out_scale;          // k_scale for fp8, else 1
};

struct CombineArgs {
  const uint16_t* part_o;
  const float* part_lse;
  const int32_t* pos_off_ws;
  const int32_t* seq_lens;
  uint16_t* out;
  float* lse;
  const int32_t* qo_indptr;
  int32_t total_q;
  int32_t B, q_len, H, nrb, R, max_seq_len, num_splits;
  int64_t NG;   // groups of the plan
  // the split kernel's row-block class plan, or null when none can apply:
  // [0] 1 when it was used; [1+n] T_n, [10+n] G_n, [19+n] base_n (n = 0..8);
  // pos_off_ws then holds each request's offset on its class's line
  const int32_t* class_tab;
};

struct AppendArgs {
  const uint16_t* nope;     // [T][nope_stride] bf16, first 512 elements of a row used
  const uint16_t* rope;     // [T][rope_stride] bf16, first 64 used
  const int64_t* loc;       // [T] flat slots page * P + slot
  void* pool;               // [N * P][576] bf16 or e4m3fn
  int64_t nope_stride, rope_stride;   // elements
  int64_t slots;            // N * P
  int32_t T;
  int32_t fp8;
  float k_scale;            // fp8: stored code = e4m3fn(x / k_scale)
  // rotary embedding of the rope part before it is stored (null rope_cs: none)
  const int64_t* positions;
  const float* rope_cs;
  int32_t rope_max_pos, rope_neox;
};

}  // namespace mla

extern "C" {
// kv_mode: 0 bf16 pool; 1 fp8 pool, codes converted to bf16 at the fragment
// reads; 2 fp8 pool with the query quantised and fp8 score products.
hipError_t mla_launch_split(const mla::SplitArgs* a, int kv_mode, hipStream_t stream);
hipError_t mla_launch_combine(const mla::CombineArgs* a, hipStream_t stream);
hipError_t mla_launch_gather(const void* pool, const int32_t* bt, const int32_t* seq_lens, int32_t W, int32_t P,
                             int32_t N, int32_t max_seq_len, int32_t b, int32_t elem_bytes, void* dst,
                             hipStream_t stream);
hipError_t mla_launch_plan(const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t nrb, int32_t num_splits,
                           int64_t G, int32_t vg_per, int32_t max_per_wg, int32_t* pieces, int32_t* counts,
                           hipStream_t stream);
size_t mla_split_lds_bytes(int32_t B, int32_t num_splits);
hipError_t mla_launch_append(const mla::AppendArgs* a, hipStream_t stream);
}
