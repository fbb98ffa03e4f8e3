// mla_api.cpp -- host side of libmla: argument validation, workspace
// sizing, the host mirror of the work plan, and the launch sequence.
//
// Argument rules follow the decode call of "sglang trtllm_mla_backend.py"
// (TRTLLMMLABackend._run_decode_kernel: query [B, q_len, H, 576], paged pool
// [pages, page_size, 576], int32 block tables and seq_lens, max_seq_len,
// bmm1 scale) and the page-size rule of "tokenspeed trtllm_mla.py"
// (TRTLLMMLABackend.__init__ rejects page sizes other than 32 and 64).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/libmla.h"
#include "mla_args.h"
#include "mla_plan.h"

namespace {

using mla::kRowsPerBlock;
using mla::kLatentDim;

constexpr int32_t kMaxQLen = 64;
constexpr int32_t kMaxHeads = 256;
constexpr int32_t kMaxRows = 4096;
constexpr int32_t kMaxSplits = 1024;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int cus = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];

mla_status device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= 64) return MLA_ERR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev[dev].known) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    g_dev[dev].gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].cus = prop.multiProcessorCount;
    g_dev[dev].known = true;
  }
  *out = g_dev[dev];
  return MLA_OK;
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

// How the split kernel takes the pool's elements (the kKv* modes of the kernels).
int kv_mode(const mla_decode_params* p) {
  if (p->kv_dtype != MLA_KV_FP8_E4M3FN) return 0;
  return p->quantize_q_fp8 ? 2 : 1;
}

// Checks that need no device.  Returns MLA_OK or the error.
mla_status check_params(const mla_decode_params* p) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  if (p->kv_lora_rank != mla::kLatentDim || p->qk_rope_head_dim != mla::kRowDim - mla::kLatentDim)
    return MLA_ERR_NOT_SUPPORTED;
  if (p->batch < 0 || p->q_len < 1 || p->num_heads < 1) return MLA_ERR_INVALID_VALUE;
  if (p->batch > mla::kMaxBatch || p->q_len > kMaxQLen || p->num_heads > kMaxHeads ||
      (int64_t)p->q_len * p->num_heads > kMaxRows)
    return MLA_ERR_NOT_SUPPORTED;
  if (p->page_size != 32 && p->page_size != 64) return MLA_ERR_INVALID_VALUE;
  if (p->num_pages < 1 || p->max_seq_len < 0 || p->block_table_stride < 1) return MLA_ERR_INVALID_VALUE;
  if ((int64_t)p->block_table_stride * p->page_size < p->max_seq_len) return MLA_ERR_INVALID_VALUE;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_VALUE;
  if (!finite_pos(p->softmax_scale)) return MLA_ERR_INVALID_VALUE;
  if (p->kv_dtype == MLA_KV_FP8_E4M3FN && !finite_pos(p->k_scale)) return MLA_ERR_INVALID_VALUE;
  if (p->num_splits < 0 || p->num_splits > kMaxSplits) return MLA_ERR_INVALID_VALUE;
  if (p->min_work_units < 0 || p->num_cus < 0) return MLA_ERR_INVALID_VALUE;
  if (p->quantize_q_fp8 != 0 && (p->quantize_q_fp8 != 1 || p->kv_dtype != MLA_KV_FP8_E4M3FN))
    return MLA_ERR_INVALID_VALUE;
  // Work units and the balanced plan's cost positions are counted in int32 on the device.
  const int64_t nrb = mla::row_blocks(p->q_len, p->num_heads);
  if ((int64_t)p->batch * nrb * mla::positions_of(p->max_seq_len) >= ((int64_t)1 << 31)) return MLA_ERR_NOT_SUPPORTED;
  return MLA_OK;
}

// Workgroups of the balanced planner, resolving the compute-unit count when needed.
mla_status target_units(const mla_decode_params* p, int32_t* target) {
  if (p->min_work_units > 0) {
    *target = p->min_work_units;
  } else if (p->num_cus > 0) {
    *target = p->num_cus;
  } else {
    DeviceInfo di;
    mla_status s = device_info(&di);
    if (s != MLA_OK) return s;
    *target = di.cus;
  }
  return MLA_OK;
}

struct Layout {
  int64_t groups = 0, wgs = 0, slots = 0;
  size_t off_pos = 0, off_lse = 0, off_o = 0, total = 0;
};

mla_status layout_of(const mla_decode_params* p, Layout* lay) {
  const int32_t nrb = mla::row_blocks(p->q_len, p->num_heads);
  int32_t target = 1;
  if (p->num_splits == 0) {
    mla_status s = target_units(p, &target);
    if (s != MLA_OK) return s;
  }
  lay->groups = mla::group_count(p->batch, nrb, p->max_seq_len, p->num_splits, target, p->min_work_units > 0);
  lay->wgs = lay->groups * nrb;
  lay->slots = mla::slot_count(lay->groups, nrb, p->num_splits);
  lay->off_pos = 0;   // offsets [B+1], then the class plan's table
  lay->off_lse = align256(((size_t)p->batch + 1 + mla::kClassTabInts) * sizeof(int32_t));
  lay->off_o = lay->off_lse + align256((size_t)lay->slots * kRowsPerBlock * sizeof(float));
  lay->total = lay->off_o + (size_t)lay->slots * kRowsPerBlock * kLatentDim * sizeof(uint16_t);
  if (mla::launch_grid(lay->groups, nrb) > 0x7fffffff) return MLA_ERR_NOT_SUPPORTED;
  return MLA_OK;
}

}  // namespace

namespace {

// Where the query's two parts live: q_nope + token*nope_token_stride +
// h*nope_head_stride (512 bf16) and q_rope + ... (64 bf16), token = b*q_len + j.
struct QueryParts {
  const void* nope;
  const void* rope;
  mla_query_layout s;
  const int32_t* qo_indptr = nullptr;   // ragged batch: per-request query token offsets [B+1]
  int32_t total_q = 0;                  // ragged batch: query tokens in q and out
  const mla_rope* rotary = nullptr;     // rotary embedding of the rope part, or none
};

// Host checks of a rotary-embedding description.
mla_status check_rope(const mla_rope* r) {
  if (r == nullptr || r->positions == nullptr || r->cos_sin_cache == nullptr) return MLA_ERR_INVALID_VALUE;
  if (r->max_position < 1 || (r->is_neox != 0 && r->is_neox != 1)) return MLA_ERR_INVALID_VALUE;
  if (((uintptr_t)r->cos_sin_cache & 15) != 0 || ((uintptr_t)r->positions & 7) != 0) return MLA_ERR_INVALID_VALUE;
  return MLA_OK;
}

QueryParts merged_query(const mla_decode_params* p, const void* q) {
  QueryParts qp;
  qp.nope = q;
  qp.rope = q == nullptr ? nullptr : (const void*)((const uint16_t*)q + kLatentDim);
  qp.s.nope_token_stride = qp.s.rope_token_stride = (int64_t)p->num_heads * mla::kRowDim;
  qp.s.nope_head_stride = qp.s.rope_head_stride = mla::kRowDim;
  return qp;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_str(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_VALUE: return "MLA_ERR_INVALID_VALUE";
    case MLA_ERR_NOT_SUPPORTED: return "MLA_ERR_NOT_SUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

mla_status mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes) {
  if (bytes == nullptr) return MLA_ERR_INVALID_VALUE;
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  Layout lay;
  s = layout_of(p, &lay);
  if (s != MLA_OK) return s;
  *bytes = lay.total;
  return MLA_OK;
}

static mla_status decode_impl(const mla_decode_params* p, const QueryParts& qp, const void* kv_pool,
                              const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream, void* ev_start,
                              void* ev_mid, void* ev_end) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (p->batch == 0) return MLA_OK;
  if (qp.nope == nullptr || qp.rope == nullptr || kv_pool == nullptr || block_table == nullptr ||
      seq_lens == nullptr || out == nullptr || workspace == nullptr)
    return MLA_ERR_INVALID_VALUE;
  if (((uintptr_t)qp.nope | (uintptr_t)qp.rope | (uintptr_t)kv_pool | (uintptr_t)out) & 15)
    return MLA_ERR_INVALID_VALUE;
  {
    // 16-byte aligned fragments need strides in whole multiples of 8 elements
    const mla_query_layout& l = qp.s;
    if (((l.nope_token_stride | l.nope_head_stride | l.rope_token_stride | l.rope_head_stride) & 7) != 0)
      return MLA_ERR_INVALID_VALUE;
    if (l.nope_token_stride < 0 || l.nope_head_stride < 0 || l.rope_token_stride < 0 || l.rope_head_stride < 0)
      return MLA_ERR_INVALID_VALUE;
  }
  if (((uintptr_t)workspace & 255) != 0) return MLA_ERR_INVALID_VALUE;
  Layout lay;
  s = layout_of(p, &lay);
  if (s != MLA_OK) return s;
  if (workspace_bytes < lay.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
  DeviceInfo di;
  s = device_info(&di);
  if (s != MLA_OK) return s;
  if (!di.gfx950) return MLA_ERR_NOT_SUPPORTED;

  char* ws = (char*)workspace;
  const bool fp8 = p->kv_dtype == MLA_KV_FP8_E4M3FN;
  const float kscale = fp8 ? p->k_scale : 1.f;
  mla::SplitArgs a;
  a.q = (const uint16_t*)qp.nope;
  a.q_rope = (const uint16_t*)qp.rope;
  a.qn_tok = qp.s.nope_token_stride;
  a.qn_head = qp.s.nope_head_stride;
  a.qr_tok = qp.s.rope_token_stride;
  a.qr_head = qp.s.rope_head_stride;
  a.qo_indptr = qp.qo_indptr;
  a.positions = qp.rotary != nullptr ? qp.rotary->positions : nullptr;
  a.rope_cs = qp.rotary != nullptr ? qp.rotary->cos_sin_cache : nullptr;
  a.rope_max_pos = qp.rotary != nullptr ? qp.rotary->max_position : 0;
  a.rope_neox = qp.rotary != nullptr ? qp.rotary->is_neox : 0;
  a.total_q = qp.qo_indptr != nullptr ? qp.total_q : p->batch * p->q_len;
  a.pool = kv_pool;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.part_o = (uint16_t*)(ws + lay.off_o);
  a.part_lse = (float*)(ws + lay.off_lse);
  a.pos_off_ws = (int32_t*)(ws + lay.off_pos);
  a.B = p->batch;
  a.q_len = p->q_len;
  a.H = p->num_heads;
  a.P = p->page_size;
  a.W = p->block_table_stride;
  a.N = p->num_pages;
  a.max_seq_len = p->max_seq_len;
  a.nrb = mla::row_blocks(p->q_len, p->num_heads);
  a.R = p->q_len * p->num_heads;
  a.num_splits = p->num_splits;
  a.NG = lay.groups;
  a.p_shift = p->page_size == 64 ? 6 : 5;
  a.vg_per = mla::fold_factor(lay.groups, a.nrb, p->num_splits, di.cus);
  a.NGL = mla::launched_groups(lay.groups, a.vg_per);
  // a ragged batch in balanced mode, unfolded, with at most kMaxClasses row
  // blocks: the kernel plans it in row-block classes when they fit
  a.class_tab = a.pos_off_ws + p->batch + 1;
  a.class_plan = qp.qo_indptr != nullptr && p->num_splits == 0 && a.vg_per == 1 &&
                 a.nrb <= mla::kMaxClasses;
  a.class_S = (int32_t)std::min<int64_t>(lay.groups * a.nrb, di.cus);
  a.class_C = (int32_t)std::min<int64_t>(mla::launch_grid(lay.groups, a.nrb) / mla::kXcds, di.cus / mla::kXcds);
  a.scale_log2 = (float)((double)p->softmax_scale * (double)kscale * 1.4426950408889634);
  a.out_scale = kscale;
  hipStream_t st = (hipStream_t)stream;
  if (ev_start != nullptr && hipEventRecord((hipEvent_t)ev_start, st) != hipSuccess) return MLA_ERR_HIP;
  if (mla_launch_split(&a, kv_mode(p), st) != hipSuccess) return MLA_ERR_HIP;
  if (ev_mid != nullptr && hipEventRecord((hipEvent_t)ev_mid, st) != hipSuccess) return MLA_ERR_HIP;
  if (p->num_splits != 1) {
    mla::CombineArgs c;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.pos_off_ws = a.pos_off_ws;
    c.seq_lens = seq_lens;
    c.out = a.out;
    c.lse = lse;
    c.qo_indptr = a.qo_indptr;
    c.total_q = a.total_q;
    c.B = a.B;
    c.q_len = a.q_len;
    c.H = a.H;
    c.nrb = a.nrb;
    c.R = a.R;
    c.max_seq_len = a.max_seq_len;
    c.num_splits = a.num_splits;
    c.NG = a.NG;
    c.class_tab = a.class_plan ? a.class_tab : nullptr;
    if (mla_launch_combine(&c, st) != hipSuccess) return MLA_ERR_HIP;
  }
  if (ev_end != nullptr && hipEventRecord((hipEvent_t)ev_end, st) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_decode(const mla_decode_params* p, const void* q, const void* kv_pool, const int32_t* block_table,
                      const int32_t* seq_lens, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  return decode_impl(p, merged_query(p, q), kv_pool, block_table, seq_lens, out, lse, workspace, workspace_bytes,
                     stream, nullptr, nullptr, nullptr);
}

mla_status mla_decode_ragged(const mla_decode_params* p, const void* q, const int32_t* qo_indptr,
                             int32_t total_q_tokens, const void* kv_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  if (total_q_tokens < 0 || (p->batch > 0 && qo_indptr == nullptr)) return MLA_ERR_INVALID_VALUE;
  if ((((uintptr_t)qo_indptr) & 3) != 0) return MLA_ERR_INVALID_VALUE;
  if (total_q_tokens == 0) return check_params(p);   // no query token: nothing to write, q and out may be null
  QueryParts qp;
  qp.nope = q;
  qp.rope = q == nullptr ? nullptr : (const void*)((const uint16_t*)q + kLatentDim);
  qp.s.nope_token_stride = qp.s.rope_token_stride = (int64_t)p->num_heads * mla::kRowDim;
  qp.s.nope_head_stride = qp.s.rope_head_stride = mla::kRowDim;
  qp.qo_indptr = qo_indptr;
  qp.total_q = total_q_tokens;
  return decode_impl(p, qp, kv_pool, block_table, seq_lens, out, lse, workspace, workspace_bytes, stream, nullptr,
                     nullptr, nullptr);
}

mla_status mla_check_qo_indptr_host(const mla_decode_params* p, const int32_t* qo_indptr_host,
                                    int32_t total_q_tokens) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (p->batch > 0 && qo_indptr_host == nullptr) return MLA_ERR_INVALID_VALUE;
  if (p->batch > 0 && qo_indptr_host[0] != 0) return MLA_ERR_INVALID_VALUE;
  for (int32_t b = 0; b < p->batch; b++) {
    const int32_t n = qo_indptr_host[b + 1] - qo_indptr_host[b];
    if (n < 0 || n > p->q_len) return MLA_ERR_INVALID_VALUE;
  }
  if (p->batch > 0 && qo_indptr_host[p->batch] != total_q_tokens) return MLA_ERR_INVALID_VALUE;
  return MLA_OK;
}

mla_status mla_decode_qparts_rope(const mla_decode_params* p, const void* q_nope, const void* q_rope,
                                  const mla_query_layout* layout, const mla_rope* rope, const void* kv_pool,
                                  const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (layout == nullptr) return MLA_ERR_INVALID_VALUE;
  mla_status s = check_rope(rope);
  if (s != MLA_OK) return s;
  QueryParts qp;
  qp.nope = q_nope;
  qp.rope = q_rope;
  qp.s = *layout;
  qp.rotary = rope;
  return decode_impl(p, qp, kv_pool, block_table, seq_lens, out, lse, workspace, workspace_bytes, stream, nullptr,
                     nullptr, nullptr);
}

mla_status mla_decode_qparts(const mla_decode_params* p, const void* q_nope, const void* q_rope,
                             const mla_query_layout* layout, const void* kv_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (layout == nullptr) return MLA_ERR_INVALID_VALUE;
  QueryParts qp;
  qp.nope = q_nope;
  qp.rope = q_rope;
  qp.s = *layout;
  return decode_impl(p, qp, kv_pool, block_table, seq_lens, out, lse, workspace, workspace_bytes, stream, nullptr,
                     nullptr, nullptr);
}

mla_status mla_decode_timed(const mla_decode_params* p, const void* q, const void* kv_pool,
                            const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_split_done,
                            void* ev_end) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  return decode_impl(p, merged_query(p, q), kv_pool, block_table, seq_lens, out, lse, workspace, workspace_bytes,
                     stream, ev_start, ev_split_done, ev_end);
}

mla_status mla_gather_kv(const mla_decode_params* p, const void* kv_pool, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t b, void* dst, void* stream) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (kv_pool == nullptr || block_table == nullptr || seq_lens == nullptr || dst == nullptr)
    return MLA_ERR_INVALID_VALUE;
  if (b < 0 || b >= p->batch) return MLA_ERR_INVALID_VALUE;
  if (((uintptr_t)kv_pool | (uintptr_t)dst) & 15) return MLA_ERR_INVALID_VALUE;
  DeviceInfo di;
  s = device_info(&di);
  if (s != MLA_OK) return s;
  if (!di.gfx950) return MLA_ERR_NOT_SUPPORTED;
  const int32_t eb = p->kv_dtype == MLA_KV_FP8_E4M3FN ? 1 : 2;
  if (mla_launch_gather(kv_pool, block_table, seq_lens, p->block_table_stride, p->page_size, p->num_pages,
                        p->max_seq_len, b, eb, dst, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_plan_host(const mla_decode_params* p, const int32_t* seq_lens_host, int32_t* pieces,
                         int32_t max_pieces, int32_t* n_pieces, int32_t* grid) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (n_pieces == nullptr || grid == nullptr || (p->batch > 0 && seq_lens_host == nullptr)) return MLA_ERR_INVALID_VALUE;
  if (max_pieces > 0 && pieces == nullptr) return MLA_ERR_INVALID_VALUE;
  Layout lay;
  s = layout_of(p, &lay);
  if (s != MLA_OK) return s;
  const int32_t B = p->batch, nrb = mla::row_blocks(p->q_len, p->num_heads);
  const int64_t NG = lay.groups;
  int64_t n = 0;
  auto emit = [&](const mla::Piece& pc, int64_t wg) {
    if (n < max_pieces) {
      int32_t* o = pieces + n * 6;
      o[0] = (int32_t)wg; o[1] = pc.b; o[2] = pc.rb; o[3] = pc.tile0; o[4] = pc.tile1; o[5] = pc.slot;
    }
    n++;
  };
  if (p->num_splits > 0) {
    for (int64_t g = 0; g < NG; g++)
      for (int32_t rb = 0; rb < nrb; rb++) {
        const int32_t b = (int32_t)(g / p->num_splits);
        mla::Piece pc;
        if (mla::forced_piece(g, rb, nrb, p->num_splits,
                              mla::units_of(mla::clamp_len(seq_lens_host[b], p->max_seq_len)), &pc))
          emit(pc, g * nrb + rb);
      }
  } else {
    std::vector<int64_t> off((size_t)B + 1, 0);
    for (int32_t b = 0; b < B; b++)
      off[b + 1] = off[b] + mla::positions_of(mla::clamp_len(seq_lens_host[b], p->max_seq_len));
    auto fr = [&](int64_t u) -> int32_t {   // largest b with off[b] <= u
      int32_t lo = 0, hi = B - 1;
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (off[(size_t)mid] <= u) lo = mid; else hi = mid - 1;
      }
      return lo;
    };
    auto units = [&](int32_t b) -> int32_t { return mla::units_of(mla::clamp_len(seq_lens_host[b], p->max_seq_len)); };
    const int64_t total = off[(size_t)B];
    // The groups are walked as a folded launch on num_cus CUs (256 when
    // unset) walks them, several per workgroup; the pieces do not depend on
    // it.  They are listed by plan workgroup.
    const int32_t vg = mla::fold_factor(NG, nrb, 0, p->num_cus > 0 ? p->num_cus : 256);
    std::vector<std::pair<int64_t, mla::Piece>> got;
    for (int64_t g0 = 0; g0 < NG; g0 += vg) {
      const int64_t g1 = std::min<int64_t>(g0 + vg, NG);
      const int64_t v_begin = mla::wg_start(g0, total, NG);
      const int32_t b_first = v_begin < total ? fr(v_begin) : 0;
      for (int32_t rb = 0; rb < nrb; rb++)
        mla::folded_balanced_pieces(g0, g1, NG, rb, nrb, total, b_first, off[(size_t)b_first], units,
                                    [&](const mla::Piece& pc, int64_t g) { got.emplace_back(g * nrb + rb, pc); });
    }
    std::stable_sort(got.begin(), got.end(), [](const auto& x, const auto& y) { return x.first < y.first; });
    for (const auto& e : got) emit(e.second, e.first);
  }
  *n_pieces = (int32_t)n;
  *grid = (int32_t)lay.wgs;
  return n > max_pieces ? MLA_ERR_INVALID_VALUE : MLA_OK;
}

mla_status mla_plan_host_ragged(const mla_decode_params* p, const int32_t* seq_lens_host,
                                const int32_t* qo_indptr_host, int32_t total_q_tokens, int32_t* pieces,
                                int32_t max_pieces, int32_t* n_pieces, int32_t* grid, int32_t* class_plan_used) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (n_pieces == nullptr || grid == nullptr || class_plan_used == nullptr) return MLA_ERR_INVALID_VALUE;
  if (p->batch > 0 && (seq_lens_host == nullptr || qo_indptr_host == nullptr)) return MLA_ERR_INVALID_VALUE;
  if (max_pieces > 0 && pieces == nullptr) return MLA_ERR_INVALID_VALUE;
  if (total_q_tokens < 0) return MLA_ERR_INVALID_VALUE;
  Layout lay;
  s = layout_of(p, &lay);
  if (s != MLA_OK) return s;
  const int32_t B = p->batch, nrb = mla::row_blocks(p->q_len, p->num_heads);
  const int64_t NG = lay.groups;
  // the query tokens of request b as the kernel takes them from the offsets
  auto q_b = [&](int32_t b) -> int32_t {
    const int32_t st = qo_indptr_host[b], en = qo_indptr_host[b + 1];
    if (st < 0 || en < st || en > total_q_tokens) return 0;
    return std::min(en - st, p->q_len);
  };
  auto units = [&](int32_t b) -> int32_t { return mla::units_of(mla::clamp_len(seq_lens_host[b], p->max_seq_len)); };
  auto pos = [&](int32_t b) -> int64_t { return mla::positions_of(mla::clamp_len(seq_lens_host[b], p->max_seq_len)); };
  std::vector<std::pair<int64_t, mla::Piece>> got;   // (plan workgroup, piece)
  *class_plan_used = 0;
  if (p->num_splits > 0) {
    for (int64_t g = 0; g < NG; g++)
      for (int32_t rb = 0; rb < nrb; rb++) {
        const int32_t b = (int32_t)(g / p->num_splits);
        mla::Piece pc;
        if (mla::forced_piece(g, rb, nrb, p->num_splits, units(b), &pc)) got.emplace_back(g * nrb + rb, pc);
      }
  } else {
    const int32_t cus = p->num_cus > 0 ? p->num_cus : 256;
    const int32_t vg = mla::fold_factor(NG, nrb, 0, cus);
    // the class plan's slots: the launch's, at most the CUs (as the kernel is given them)
    const int32_t class_S = (int32_t)std::min<int64_t>(NG * nrb, cus);
    const int32_t class_C = (int32_t)std::min<int64_t>(mla::launch_grid(NG, nrb) / mla::kXcds, cus / mla::kXcds);
    mla::ClassPlan cp;
    cp.ok = false;
    if (vg == 1 && nrb <= mla::kMaxClasses) {
      int32_t T[mla::kMaxClasses + 1] = {0};
      for (int32_t b = 0; b < B; b++) {
        const int32_t n = mla::row_blocks(q_b(b), p->num_heads);
        if (n >= 1) T[n] += (int32_t)pos(b);
      }
      cp = mla::make_class_plan(T, nrb, class_S, class_C);
    }
    if (cp.ok) {
      *class_plan_used = 1;
      const int32_t C = class_C;
      for (int32_t x = 0; x < mla::kXcds; x++)
        for (int32_t sl = 0; sl < C; sl++) {
          int32_t g = 0, rb = 0;
          const int32_t n = mla::class_slot(cp, nrb, C, x, sl, &g, &rb);
          if (n == 0) continue;
          auto member = [&](int32_t b) { return mla::row_blocks(q_b(b), p->num_heads) == n; };
          // offsets on the class's line; the request holding the group's first position
          const int64_t v_begin = mla::wg_start(g, cp.T[n], cp.G[n]);
          int64_t off = 0, off_first = 0;
          int32_t b_first = 0;
          for (int32_t b = 0; b < B; b++) {
            if (!member(b)) continue;
            if (off <= v_begin) {
              b_first = b;
              off_first = off;
            }
            off += pos(b);
          }
          auto succ = [&](int32_t b) {
            for (b++; b < B && !member(b); b++) {
            }
            return b;
          };
          mla::BalancedWalk w;
          w.init(g, cp.G[n], rb, n, cp.T[n], b_first, off_first, cp.base[n]);
          mla::Piece pc;
          while (w.next(units, &pc, succ)) got.emplace_back(cp.base[n] + (int64_t)g * n + rb, pc);
        }
    } else {
      std::vector<int64_t> off((size_t)B + 1, 0);
      for (int32_t b = 0; b < B; b++) off[b + 1] = off[b] + pos(b);
      const int64_t total = off[(size_t)B];
      for (int64_t g0 = 0; g0 < NG; g0 += vg) {
        const int64_t g1 = std::min<int64_t>(g0 + vg, NG);
        const int64_t v_begin = mla::wg_start(g0, total, NG);
        int32_t b_first = 0;
        for (int32_t b = 0; b < B; b++)
          if (off[b] <= v_begin) b_first = b;
        for (int32_t rb = 0; rb < nrb; rb++)
          mla::folded_balanced_pieces(g0, g1, NG, rb, nrb, total, b_first, off[(size_t)b_first], units,
                                      [&](const mla::Piece& pc, int64_t g) { got.emplace_back(g * nrb + rb, pc); });
      }
    }
  }
  std::stable_sort(got.begin(), got.end(), [](const auto& x, const auto& y) { return x.first < y.first; });
  int64_t n = 0;
  for (const auto& e : got) {
    const mla::Piece& pc = e.second;
    if ((int64_t)pc.rb * mla::kRowsPerBlock >= (int64_t)q_b(pc.b) * p->num_heads) continue;   // no rows here
    if (n < max_pieces) {
      int32_t* o = pieces + n * 6;
      o[0] = (int32_t)e.first; o[1] = pc.b; o[2] = pc.rb; o[3] = pc.tile0; o[4] = pc.tile1; o[5] = pc.slot;
    }
    n++;
  }
  *n_pieces = (int32_t)n;
  *grid = (int32_t)lay.wgs;
  return n > max_pieces ? MLA_ERR_INVALID_VALUE : MLA_OK;
}

mla_status mla_plan_device(const mla_decode_params* p, const int32_t* seq_lens, int32_t* pieces, int32_t max_per_wg,
                           int32_t* counts, int32_t grid, void* stream) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (seq_lens == nullptr || pieces == nullptr || counts == nullptr || max_per_wg < 1) return MLA_ERR_INVALID_VALUE;
  Layout lay;
  s = layout_of(p, &lay);
  if (s != MLA_OK) return s;
  if (grid != lay.wgs || grid < 1) return MLA_ERR_INVALID_VALUE;
  DeviceInfo di;
  s = device_info(&di);
  if (s != MLA_OK) return s;
  if (!di.gfx950) return MLA_ERR_NOT_SUPPORTED;
  const int32_t nrb = mla::row_blocks(p->q_len, p->num_heads);
  if (mla_launch_plan(seq_lens, p->batch, p->max_seq_len, nrb, p->num_splits, lay.groups,
                      mla::fold_factor(lay.groups, nrb, p->num_splits, di.cus), max_per_wg, pieces, counts,
                      (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

static mla_status kv_append_impl(const mla_kv_append_params* p, const void* k_nope, const void* k_rope,
                                 const int64_t* out_cache_loc, const mla_rope* rope, void* kv_pool, void* stream) {
  if (p == nullptr) return MLA_ERR_INVALID_VALUE;
  if (p->kv_lora_rank != mla::kLatentDim || p->qk_rope_head_dim != mla::kRowDim - mla::kLatentDim)
    return MLA_ERR_NOT_SUPPORTED;
  if (p->num_tokens < 0 || p->num_pages < 1) return MLA_ERR_INVALID_VALUE;
  if (p->page_size != 32 && p->page_size != 64) return MLA_ERR_INVALID_VALUE;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_VALUE;
  if (p->kv_dtype == MLA_KV_FP8_E4M3FN && !finite_pos(p->k_scale)) return MLA_ERR_INVALID_VALUE;
  if (p->nope_stride < mla::kLatentDim || p->rope_stride < mla::kRowDim - mla::kLatentDim ||
      (p->nope_stride & 7) != 0 || (p->rope_stride & 7) != 0)
    return MLA_ERR_INVALID_VALUE;
  if (p->num_tokens == 0) return MLA_OK;
  if (k_nope == nullptr || k_rope == nullptr || out_cache_loc == nullptr || kv_pool == nullptr)
    return MLA_ERR_INVALID_VALUE;
  if (((uintptr_t)k_nope | (uintptr_t)k_rope | (uintptr_t)kv_pool) & 15) return MLA_ERR_INVALID_VALUE;
  if (((uintptr_t)out_cache_loc & 7) != 0) return MLA_ERR_INVALID_VALUE;
  DeviceInfo di;
  mla_status s = device_info(&di);
  if (s != MLA_OK) return s;
  if (!di.gfx950) return MLA_ERR_NOT_SUPPORTED;
  mla::AppendArgs a;
  a.nope = (const uint16_t*)k_nope;
  a.rope = (const uint16_t*)k_rope;
  a.loc = out_cache_loc;
  a.pool = kv_pool;
  a.nope_stride = p->nope_stride;
  a.rope_stride = p->rope_stride;
  a.slots = (int64_t)p->num_pages * p->page_size;
  a.T = p->num_tokens;
  a.fp8 = p->kv_dtype == MLA_KV_FP8_E4M3FN ? 1 : 0;
  a.k_scale = a.fp8 ? p->k_scale : 1.f;
  a.positions = rope != nullptr ? rope->positions : nullptr;
  a.rope_cs = rope != nullptr ? rope->cos_sin_cache : nullptr;
  a.rope_max_pos = rope != nullptr ? rope->max_position : 0;
  a.rope_neox = rope != nullptr ? rope->is_neox : 0;
  if (mla_launch_append(&a, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status mla_kv_append(const mla_kv_append_params* p, const void* k_nope, const void* k_rope,
                         const int64_t* out_cache_loc, void* kv_pool, void* stream) {
  return kv_append_impl(p, k_nope, k_rope, out_cache_loc, nullptr, kv_pool, stream);
}

mla_status mla_kv_append_rope(const mla_kv_append_params* p, const void* k_nope, const void* k_rope,
                              const int64_t* out_cache_loc, const mla_rope* rope, void* kv_pool, void* stream) {
  mla_status s = check_rope(rope);
  if (s != MLA_OK) return s;
  return kv_append_impl(p, k_nope, k_rope, out_cache_loc, rope, kv_pool, stream);
}

mla_status mla_check_inputs_host(const mla_decode_params* p, const int32_t* block_table_host,
                                 const int32_t* seq_lens_host) {
  mla_status s = check_params(p);
  if (s != MLA_OK) return s;
  if (p->batch > 0 && (block_table_host == nullptr || seq_lens_host == nullptr)) return MLA_ERR_INVALID_VALUE;
  for (int32_t b = 0; b < p->batch; b++) {
    const int32_t L = seq_lens_host[b];
    if (L < 0 || L > p->max_seq_len) return MLA_ERR_INVALID_VALUE;
    const int32_t n = (L + p->page_size - 1) / p->page_size;
    for (int32_t i = 0; i < n; i++) {
      const int32_t pg = block_table_host[(int64_t)b * p->block_table_stride + i];
      if (pg < 0 || pg >= p->num_pages) return MLA_ERR_INVALID_VALUE;
    }
  }
  return MLA_OK;
}

}  // extern "C"
