/*
 * libmla.h -- C ABI of libmla: batched paged Multi-head Latent Attention
 * (MLA) decode over a compressed latent KV cache, for AMD MI355X (gfx950).
 *
 * The operation is the decode call of the attention backends of
 * "sglang trtllm_mla_backend.py" (TRTLLMMLABackend._run_decode_kernel and
 * forward_decode) and "tokenspeed flashmla.py" (FlashMLABackend.forward_decode,
 * and forward_extend with causal=True for several query tokens):
 *
 *   For request b (L = seq_lens[b] cached tokens, the q_len new ones
 *   included), query token j < q_len and head h, the visible tokens are
 *   t < L - q_len + 1 + j (bottom-right causal alignment).  Token t's row is
 *   pool[block_table[b][t / page_size]][t % page_size][0:576]: the 512-wide
 *   latent c_kv followed by the 64-wide rope key.  One latent row serves all
 *   heads (one KV head).
 *
 *     s_t = softmax_scale * k_scale * (q[b,j,h,0:576] . row_t)
 *     out[b,j,h,c] = sum_t softmax(s)_t * k_scale * row_t[c],  c < 512
 *     lse[b,j,h]   = ln sum_t exp(s_t)
 *
 *   k_scale applies only to an fp8 pool (the bmm1 scale rule of
 *   _compute_decode_bmm1_scale); a bf16 pool ignores it.  A query row with no
 *   visible token gets out = 0 and lse = -inf (the zero-KV row convention of
 *   the sglang backend).
 *
 * Conventions for every entry point:
 *  - All pointers marked "device" are HIP device pointers; the library never
 *    allocates, frees or synchronises, and enqueues all work on `stream`
 *    (a hipStream_t; NULL = the null stream).  The caller owns every buffer.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    error status means nothing was enqueued.
 *  - Device data are trusted the way the pages trust them: seq_lens[b] must
 *    lie in [0, max_seq_len] (values outside are clamped), and every
 *    block-table entry a request reads (index < ceil(seq_lens[b] /
 *    page_size)) must lie in [0, num_pages).  An entry outside that range is
 *    never dereferenced: a bf16 pool reads page 0 in its place, an fp8 pool
 *    reads zeros, and the result is undefined.  Entries past a request's
 *    last page are never read and may hold anything (-1, 0, ...).
 *    mla_check_inputs_host() checks all of this on host copies.
 *  - A workspace must not be shared by calls that may run concurrently.
 */
#ifndef LIBMLA_H
#define LIBMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: adds mla_decode_qparts(_rope), mla_decode_ragged, mla_check_qo_indptr_host,
 * mla_kv_append(_rope); version 1 entry points and structs are unchanged. */
#define MLA_ABI_VERSION 3

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_VALUE = 1,       /* a bad argument (cf. the ValueError for page sizes other than 32/64) */
  MLA_ERR_NOT_SUPPORTED = 2,       /* valid but unsupported (dims other than 512+64, not a gfx950 device) */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below mla_decode_workspace_size() */
  MLA_ERR_HIP = 4                  /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum {
  MLA_KV_BF16 = 0,        /* pool elements are bfloat16 */
  MLA_KV_FP8_E4M3FN = 1   /* pool elements are OCP float8_e4m3fn codes, dequantised as code * k_scale */
} mla_kv_dtype;

typedef struct {
  int32_t batch;              /* B >= 0 requests; B = 0 enqueues nothing. At most 8192. */
  int32_t q_len;              /* query tokens per request, 1..64 (q_len > 1: causal, bottom-right aligned) */
  int32_t num_heads;          /* H query heads per request (this GPU's share), 1..256; q_len*H <= 4096 */
  int32_t kv_lora_rank;       /* must be 512 (latent width = output width per head) */
  int32_t qk_rope_head_dim;   /* must be 64 */
  int32_t page_size;          /* tokens per page: 32 or 64 */
  int32_t num_pages;          /* pages in the pool, >= 1 */
  int32_t block_table_stride; /* W: int32 elements between block-table rows, >= ceil(max_seq_len/page_size) */
  int32_t max_seq_len;        /* upper bound of seq_lens, 0 <= max_seq_len <= W*page_size */
  int32_t kv_dtype;           /* an mla_kv_dtype */
  float softmax_scale;        /* finite, > 0 (1/sqrt(qk_nope_head_dim + qk_rope_head_dim)) */
  float k_scale;              /* fp8 pool: finite, > 0; bf16 pool: ignored */
  int32_t num_splits;         /* 0: the balanced planner; n > 0: split every request's token range into
                                 min(n, its 32-token tiles) pieces, one workgroup each (at most 1024) */
  int32_t min_work_units;     /* balanced planner: 0 = one workgroup per compute unit; n > 0 = n workgroups
                                 (one decode workgroup fits a compute unit at a time, so a target above the
                                 CU count runs in several rounds and is slower; it is there to force many
                                 split pieces) */
  int32_t num_cus;            /* 0: read the compute-unit count of the current device; n > 0: use n
                                 (lets host-only planning calls run without a device) */
  int32_t quantize_q_fp8;     /* 0: the query stays bf16 and every score is the exact product of bf16 values
                                 and dequantised codes (fp32 sums).  1 (an fp8 pool only, else
                                 MLA_ERR_INVALID_VALUE): the fp8 decode of the pages, which cast the query to
                                 float8_e4m3fn with q_scale 1 before their fp8 kernel ("tokenspeed
                                 trtllm_mla.py", TRTLLMMLABackend.forward_decode; "sglang
                                 trtllm_mla_backend.py", forward_decode and _compute_decode_bmm1_scale): each
                                 query element, after the rotary embedding when one is applied and rounded to
                                 bf16, becomes its e4m3fn code (round to nearest even, saturated at +-448,
                                 NaN stays NaN) and the scores are fp8 x fp8 products summed in fp32.  The
                                 softmax weights and the output product stay bf16.  A query that already
                                 holds e4m3fn values (passed as their exact bf16 values) is left unchanged. */
} mla_decode_params;

/* MLA_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

/* Static, human-readable name of a status code. */
const char* mla_status_str(int32_t status);

/* Bytes of device workspace mla_decode() needs for these parameters (split-KV
 * partial results and planning scratch).  This is the split-KV workspace the
 * pages hand their decode kernel: the zeroed buffer of
 * get_trtllm_workspace_buffer on "tokenspeed trtllm_mla.py" and of
 * TRTLLMMLABackend.__init__ on "sglang trtllm_mla_backend.py"
 * (workspace_buffer).  Unlike theirs it is sized per call and needs no
 * initialisation: it holds no counters, and every byte a call reads it has
 * written first.  No device memory is touched; with num_cus == 0 and
 * min_work_units == 0 and num_splits == 0 it queries the current device's
 * compute-unit count.  Errors: MLA_ERR_INVALID_VALUE / MLA_ERR_NOT_SUPPORTED
 * as mla_decode() for bad parameters, MLA_ERR_HIP if the device query fails. */
mla_status mla_decode_workspace_size(const mla_decode_params* p, size_t* bytes);

/* The decode.  Layouts (all row-major, contiguous):
 *   q           device, bf16  [B][q_len][H][576]  absorbed query: latent 512 then rope 64
 *   kv_pool     device, bf16 or e4m3fn [num_pages][page_size][576]
 *   block_table device, int32 [B][block_table_stride]
 *   seq_lens    device, int32 [B]  cached tokens per request, the q_len new tokens included
 *   out         device, bf16  [B][q_len][H][512]   (written)
 *   lse         device, fp32  [B][q_len][H] natural-log LSE of the scaled scores, or NULL
 *   workspace   device, >= mla_decode_workspace_size() bytes, 256-byte aligned
 * Enqueues up to two kernels on `stream` (split-KV decode, then the LSE
 * combine of split pieces) and returns without waiting. */
mla_status mla_decode(const mla_decode_params* p, const void* q, const void* kv_pool, const int32_t* block_table,
                      const int32_t* seq_lens, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Where the two parts of the query live when they are not one [.., 576]
 * row: query row (b, j, h), with token = b * q_len + j, has its 512-wide
 * absorbed latent part at q_nope + token * nope_token_stride +
 * h * nope_head_stride and its 64-wide rope part at q_rope +
 * token * rope_token_stride + h * rope_head_stride (strides in bf16
 * elements, each a multiple of 8, >= 0).  This is the pair the pages
 * concatenate before the decode kernel (concat_mla_absorb_q_general(q_nope,
 * q_rope) in TRTLLMMLABackend.forward_decode on "sglang
 * trtllm_mla_backend.py"); for example the head-major output of the
 * absorbed-query product viewed token-major has nope_token_stride = 512 and
 * nope_head_stride = tokens * 512. */
typedef struct {
  int64_t nope_token_stride;
  int64_t nope_head_stride;
  int64_t rope_token_stride;
  int64_t rope_head_stride;
} mla_query_layout;

/* mla_decode() with the query given as its two parts (see mla_query_layout)
 * instead of one [B][q_len][H][576] tensor: the decode reads them in place,
 * so no concatenated copy is made.  q_nope and q_rope: device, bf16, 16-byte
 * aligned.  Results are bit-identical to mla_decode() on the concatenated
 * query.  Other arguments, layouts and errors as mla_decode(); a stride that
 * is negative or not a multiple of 8 is MLA_ERR_INVALID_VALUE. */
mla_status mla_decode_qparts(const mla_decode_params* p, const void* q_nope, const void* q_rope,
                             const mla_query_layout* layout, const void* kv_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Ragged multi-token decode: request b has its own number of query tokens
 * q_b = qo_indptr[b+1] - qo_indptr[b] (0 <= q_b <= p->q_len), stored as rows
 * qo_indptr[b] .. qo_indptr[b+1]-1 of a packed query, with no padding -- the
 * cu_seqlens_q form of the draft-extend batches of "tokenspeed
 * trtllm_mla.py" (TRTLLMMLABackend.init_forward_metadata builds
 * cu_seqlens_q from extend_seq_lens; the pages then pad every request to
 * max_seq_len_q and unpad the output).  seq_lens[b] counts request b's q_b
 * new tokens, and query token j of request b sees the tokens
 * t < seq_lens[b] - q_b + 1 + j (the bottom-right alignment of mla_decode,
 * per request).  p->q_len is the largest q_b (it sizes the plan and the
 * workspace: mla_decode_workspace_size(p) applies unchanged).
 *   q          device, bf16  [total_q_tokens][H][576]
 *   qo_indptr  device, int32 [B+1], nondecreasing, qo_indptr[0] = 0,
 *              qo_indptr[B] = total_q_tokens.  The offsets are trusted on
 *              the device, never followed out of the tensors: a request whose
 *              offsets fall outside [0, total_q_tokens] or run backwards is
 *              treated as having no query tokens, and a request with more
 *              than p->q_len tokens as having its first p->q_len; nothing is
 *              read or written for the tokens left out, so their out and lse
 *              rows keep whatever they held.  mla_check_qo_indptr_host()
 *              checks the offsets on a host copy.
 *   out        device, bf16  [total_q_tokens][H][512]   (written)
 *   lse        device, fp32  [total_q_tokens][H], or NULL
 * total_q_tokens = 0 (every request without a query token) checks the
 * parameters and enqueues nothing; q, out and lse may then be NULL.
 * Other arguments, layouts and errors as mla_decode().  With every q_b equal
 * to p->q_len the results are bit-identical to mla_decode(). */
mla_status mla_decode_ragged(const mla_decode_params* p, const void* q, const int32_t* qo_indptr,
                             int32_t total_q_tokens, const void* kv_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Host-side check (CPU only) of a ragged batch's offsets: qo_indptr[0] = 0,
 * 0 <= q_b <= p->q_len for every request, qo_indptr[B] = total_q_tokens.
 * MLA_ERR_INVALID_VALUE on the first violation. */
mla_status mla_check_qo_indptr_host(const mla_decode_params* p, const int32_t* qo_indptr_host,
                                    int32_t total_q_tokens);

/* Rotary embedding of the 64-wide rope parts, the one the pages hand to
 * their rope kernel with the token positions (forward_decode of
 * TRTLLMMLABackend on "sglang trtllm_mla_backend.py": forward_batch.positions,
 * cos_sin_cache and is_neox).  Token t's rope part is turned pair by pair:
 * pair i = (x1, x2) is (dim i, dim i+32) when is_neox, else (dim 2i, dim
 * 2i+1), and becomes (x1 c - x2 s, x2 c + x1 s) with c, s = columns i and
 * 32+i of cache row clamp(positions[t], 0, max_position-1).  Each product and
 * the difference or sum is an fp32 operation (no fused multiply-add), and the
 * result is rounded to bf16 (nearest even). */
typedef struct {
  const int64_t* positions;     /* device, int64 [tokens], 8-byte aligned */
  const float* cos_sin_cache;   /* device, fp32 [max_position][64]: cos in 0..31, sin in 32..63; 16-byte aligned */
  int32_t max_position;         /* rows of the cache, >= 1 */
  int32_t is_neox;              /* 1: pairs (i, i+32); 0: pairs (2i, 2i+1) */
} mla_rope;

/* mla_decode_qparts() that first turns every query row's rope part by the
 * rotary embedding at its token's position (token = b * q_len + j indexes
 * rope->positions): the rotation the pages apply to q_rope before the decode
 * kernel, done here on the fragments in registers, so the rotated query is
 * never written out.  Errors as mla_decode_qparts(); an invalid rope
 * description (null pointers, max_position < 1, is_neox not 0 or 1, a
 * misaligned cache or positions array) is MLA_ERR_INVALID_VALUE. */
mla_status mla_decode_qparts_rope(const mla_decode_params* p, const void* q_nope, const void* q_rope,
                                  const mla_query_layout* layout, const mla_rope* rope, const void* kv_pool,
                                  const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mla_decode() with its workspace in a device array the library holds
 * itself, MLA_NOALLOC_SCRATCH_BYTES (64 MiB) per device, alive until the
 * process ends.  The caller passes inputs and outputs as for mla_decode()
 * (same layouts and errors); the call allocates nothing and frees nothing.
 * Parameters whose workspace (mla_decode_workspace_size) exceeds the array
 * return MLA_ERR_WORKSPACE_TOO_SMALL and enqueue nothing; every balanced plan
 * sized to the compute-unit count fits (about 42 MB at most on 256 CUs).
 * Every call on one device shares that device's array, so calls that may
 * overlap on one device (two streams, two threads) race: serialise them.
 * The array needs no clearing between calls: a call writes every byte of it
 * it reads.  Results are bit-identical to mla_decode(). */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_noalloc(const mla_decode_params* p, const void* q, const void* kv_pool,
                              const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                              void* stream);

/* mla_decode() that also records three caller-created HIP events (hipEvent_t,
 * each may be NULL) on `stream`: before the split-KV kernel, between it and
 * the combine kernel, and after the combine, so that a benchmark can time the
 * two kernels separately.  Same arguments, layouts and errors as mla_decode(). */
mla_status mla_decode_timed(const mla_decode_params* p, const void* q, const void* kv_pool,
                            const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_split_done,
                            void* ev_end);

/* Debug/test: copy the stored rows of request b's first min(seq_lens[b],
 * max_seq_len) tokens, byte for byte, into dst [.. ][576] (device, pool
 * element type) through the same page addressing the decode uses.  Rows
 * past that count are not written. */
mla_status mla_gather_kv(const mla_decode_params* p, const void* kv_pool, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t b, void* dst, void* stream);

/* Host mirror of the work plan (CPU only, no device access when p->num_cus >
 * 0 or p->min_work_units > 0 or p->num_splits > 0).  The plan plays the part
 * of the tile-scheduler metadata and split counts the pages obtain from
 * get_mla_metadata(seq_lens, heads, 1) in FlashMLABackend._init_decode_metadata
 * on "tokenspeed flashmla.py"; here it is recomputed inside the decode kernel
 * from the device seq_lens, and this call returns the same plan on the host
 * for tests.  It lists pieces rather than the pages' per-request split
 * pointer, because one workgroup may take pieces of two requests.  A plan assigns each
 * workgroup g < grid a list of pieces (g, b, row_block, tile_begin,
 * tile_end, slot): rows [64*row_block, 64*row_block+64) of request b's
 * q_len*H query rows (row = j*H + h) over 32-token tiles [tile_begin,
 * tile_end) of its tokens; slot < 0
 * means the piece covers the whole request and writes the output directly,
 * otherwise it writes a partial result to that workspace slot for the
 * combine.  pieces: host, int32 [max_pieces][6].  Returns
 * MLA_ERR_INVALID_VALUE if more than max_pieces pieces exist (*n_pieces then
 * holds the count needed). */
mla_status mla_plan_host(const mla_decode_params* p, const int32_t* seq_lens_host, int32_t* pieces,
                         int32_t max_pieces, int32_t* n_pieces, int32_t* grid);

/* Debug/test: the plan of a ragged batch (mla_decode_ragged) on the host,
 * with the query token offsets qo_indptr_host [B+1] (taken as the kernel
 * takes them: offsets outside [0, total_q_tokens] or running backwards
 * give no query token, more than p->q_len tokens give p->q_len).  In
 * balanced mode, unfolded, with at most 8 row blocks per request, the
 * requests are planned in row-block classes: request b has n_b row blocks
 * (rows q_b*H), the requests with n_b = n share groups of n workgroups, and
 * each class's groups take equal shares of that class's cost positions
 * (*class_plan_used = 1).  Otherwise, and when every request has all its
 * row blocks, the plan is mla_plan_host()'s (*class_plan_used = 0).
 * Pieces as for mla_plan_host(), with the first column the workgroup's
 * number in the plan (the class plan numbers its workgroups class by class
 * in descending n); pieces of row blocks without rows are left out. */
mla_status mla_plan_host_ragged(const mla_decode_params* p, const int32_t* seq_lens_host,
                                const int32_t* qo_indptr_host, int32_t total_q_tokens, int32_t* pieces,
                                int32_t max_pieces, int32_t* n_pieces, int32_t* grid, int32_t* class_plan_used);

/* Debug/test: the same plan computed on the device by the code the decode
 * kernel runs.  pieces: device int32 [grid][max_per_wg][6]; counts: device
 * int32 [grid] (pieces of each workgroup, possibly above max_per_wg, in
 * which case only the first max_per_wg are written).  grid is what
 * mla_plan_host() reports for the same parameters. */
mla_status mla_plan_device(const mla_decode_params* p, const int32_t* seq_lens, int32_t* pieces,
                           int32_t max_per_wg, int32_t* counts, int32_t grid, void* stream);

/* Host-side input check (CPU only): every seq_lens[b] in [0, max_seq_len]
 * and every block-table entry a request reads in [0, num_pages).
 * MLA_ERR_INVALID_VALUE on the first violation. */
mla_status mla_check_inputs_host(const mla_decode_params* p, const int32_t* block_table_host,
                                 const int32_t* seq_lens_host);

/* ---- KV-cache append: the cache write that precedes each decode step,
 * set_mla_kv_buffer(layer, out_cache_loc, k_nope, k_rope) in
 * TRTLLMMLABackend.forward_decode on "sglang trtllm_mla_backend.py" and on
 * "tokenspeed trtllm_mla.py".  Row i = [k_nope[i][0:512] | k_rope[i][0:64]]
 * is stored in flat slot out_cache_loc[i] of the pool, that is page
 * loc / page_size, slot loc % page_size (the token -> row map the decode
 * reads through).  A bf16 pool stores the bf16 bits unchanged.  An fp8 pool
 * stores the OCP float8_e4m3fn code of x / k_scale, computed as an fp32
 * quotient, saturated to +-448 and rounded to nearest with ties to even
 * (the per-tensor scale convention of scaled_fp8_quant in
 * _quantize_fp8_qkv on "sglang trtllm_mla_backend.py"); a NaN stores 0x7F,
 * an infinity saturates. */
typedef struct {
  int64_t nope_stride;        /* elements between rows of k_nope: >= 512, a multiple of 8 */
  int64_t rope_stride;        /* elements between rows of k_rope: >= 64, a multiple of 8 */
  int32_t num_tokens;         /* T >= 0 rows; T = 0 enqueues nothing */
  int32_t kv_lora_rank;       /* must be 512 */
  int32_t qk_rope_head_dim;   /* must be 64 */
  int32_t page_size;          /* 32 or 64 */
  int32_t num_pages;          /* pages in the pool, >= 1 */
  int32_t kv_dtype;           /* an mla_kv_dtype: the pool's element type */
  float k_scale;              /* fp8 pool: finite, > 0; bf16 pool: ignored */
} mla_kv_append_params;

/* Layouts:
 *   k_nope        device, bf16  [T][nope_stride], 16-byte aligned (e.g. k[..., :512] of a [T][576] tensor)
 *   k_rope        device, bf16  [T][rope_stride], 16-byte aligned (e.g. k[..., 512:])
 *   out_cache_loc device, int64 [T] flat slots; a location outside
 *                 [0, num_pages * page_size) is skipped (nothing is written for
 *                 that row).  Locations should be distinct: with repeats, one of
 *                 the rows is stored, which one is unspecified.
 *   kv_pool       device, bf16 or e4m3fn [num_pages][page_size][576], 16-byte aligned (written)
 * Enqueues one kernel on `stream` and returns without waiting.  Argument
 * errors (MLA_ERR_INVALID_VALUE / MLA_ERR_NOT_SUPPORTED) enqueue nothing. */
mla_status mla_kv_append(const mla_kv_append_params* p, const void* k_nope, const void* k_rope,
                         const int64_t* out_cache_loc, void* kv_pool, void* stream);

/* mla_kv_append() that turns each new row's rope part by the rotary
 * embedding at its position (rope->positions indexed by row i) before it is
 * stored: the key half of the pages' rope-then-write sequence (the rotated
 * rope part is rounded to bf16 first, then stored or quantised as by
 * mla_kv_append()).  Errors as mla_kv_append() and mla_decode_qparts_rope(). */
mla_status mla_kv_append_rope(const mla_kv_append_params* p, const void* k_nope, const void* k_rope,
                              const int64_t* out_cache_loc, const mla_rope* rope, void* kv_pool, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBMLA_H */
