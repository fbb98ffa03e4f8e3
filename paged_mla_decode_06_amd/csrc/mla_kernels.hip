// mla_kernels.hip -- gfx950 kernels of libmla: split-KV paged MLA decode,
// LSE combine, debug gather and debug plan.
//
// The decode is the one of "sglang trtllm_mla_backend.py"
// (TRTLLMMLABackend._run_decode_kernel) and "tokenspeed flashmla.py"
// (FlashMLABackend.forward_decode / forward_extend, causal=True): every
// query row (j, h) of request b attends over the request's paged 576-wide
// latent rows; all rows share the one latent KV head, so a KV tile staged
// once in LDS serves 128 query rows.
//
// Split kernel, one workgroup = 64 query rows (a row block) of one request,
// 16 waves in three roles (below): QK wave w owns rows 16w..16w+15 of the
// row block, lane l owns row l%16 throughout.  Per 32-token KV tile staged
// in LDS:
//   S^T[32 tok x 16 rows]  = K_tile[32 x 576] . Q^T[576 x 16]   (36 MFMA 16x16x32 bf16)
//   P^T = exp2(S^T*scale*log2e - m)  (online softmax, lazily rescaled)
//   O^T[512 x 16 rows]    += V^T[512 x 32 tok] . P^T[32 x 16]  (32 MFMA 16x16x32 bf16)
// With K as the A operand and Q^T as B, the S^T accumulator leaves each lane
// holding 8 tokens of its own row, which is exactly the lane's B-operand
// layout of P^T in the second product: the QK wave stores P as that 16-byte
// operand in LDS and a P.V wave reads it back unchanged, and the row max
// needs two lane exchanges.  V^T comes from the same LDS tile through the
// gfx950 transposing LDS read (ds_read_b64_tr_b16; fp8 tiles: ds_read_b64_tr_b8
// and an exact conversion of the codes to bf16).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_args.h"
#include "mla_fp8.h"
#include "mla_plan.h"
#include "mla_rope.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;                      // combine / gather / plan kernels
// Read-ahead depths and accumulation chains of the tile loops (bf16 and fp8
// tiles): K reads ahead of their MFMAs, Vt reads ahead, score chains.
#ifndef MLA_KA
#define MLA_KA 3
#endif
#ifndef MLA_VA
#define MLA_VA 1
#endif
#ifndef MLA_SC
#define MLA_SC 2
#endif
#ifndef MLA_F8_KA
#define MLA_F8_KA 3
#endif
#ifndef MLA_F8_VA
#define MLA_F8_VA 1
#endif
#ifndef MLA_F8_SC
#define MLA_F8_SC 2
#endif
constexpr int kRowsPerWave = 16;   // one 16-row MFMA block per QK wave
// A split workgroup runs three kinds of wave in a pipeline over the KV tiles
// of a piece (waves are spread evenly over the four SIMDs: one QK wave, two
// PV waves and one loader wave on each, 128 registers per wave):
//   QK waves      (kRowGroups = 4) S = Q.K^T for their 16 rows on tile j+1,
//                 online softmax, P (bf16) and the rows' rescale factors out
//                 to LDS;
//   PV waves      (kPVWaves = 8) O = alpha*O + P.V on tile j, each for a
//                 share of the (row group, output dims) grid: two row groups
//                 times 128 output dims, 64 accumulator registers;
//   loader waves  (kLoaderWaves = 4) tile j+3 into the LDS ring.
// Splitting the two products over different waves gives each one its
// registers (Q and O no longer share a wave), and the softmax of one wave
// runs while the others keep the matrix unit busy; two PV waves per SIMD
// overlap each other's LDS reads.  A tile load can stall its wave at issue
// for hundreds of cycles while the memory queue is full; the loader waves
// take those stalls.
constexpr int kRowGroups = kRowsPerBlock / kRowsPerWave;
#ifndef MLA_PV_WAVES
#define MLA_PV_WAVES 8
#endif
constexpr int kPVWaves = MLA_PV_WAVES;
constexpr int kQKWave0 = 0, kPVWave0 = kRowGroups, kLoaderWave0 = kRowGroups + kPVWaves;
constexpr int kLoaderWaves = 4;
constexpr int kSplitWaves = kRowGroups + kPVWaves + kLoaderWaves;
static_assert(kSplitWaves % 4 == 0 && kSplitWaves <= 16, "whole waves per SIMD, at most 1024 threads");
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kRowBytes = kRowDim * 2;             // 1152: one bf16 row in LDS
constexpr int kTileBytes = kTile * kRowBytes;      // 36864
constexpr int kChunks = kTile * kRowDim * 2 / 16;  // 2304 16-byte chunks per bf16 tile
constexpr int kTileLoads = kChunks / 64;           // 36 wave-wide 1 KB loads per tile
constexpr int kLoadsPerWave = kTileLoads / kLoaderWaves;   // 9 per loader wave and tile
constexpr int kQSteps = kRowDim / 32;              // 18 k-steps of 32 over the 576 dims
constexpr int kVBlocks = kLatentDim / 16;          // 32 blocks of 16 latent dims
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;
// A row's running maximum is raised only when a tile's maximum exceeds it by
// more than this (log2 units); exponentials stay <= 2^8, exact math unchanged.
constexpr float kRescaleSlack = 8.0f;
// How the pool's elements reach the matrix unit (the KV template parameter
// of the split kernel):
//   kKvBf16  bf16 pool: bf16 tiles in LDS, bf16 products.
//   kKvFp8   e4m3fn pool: the codes are staged in LDS as they are, and K and
//            V^T are converted to bf16 (exactly) as their MFMA fragments are
//            read; bf16 products.
//   kKvFp8Q  e4m3fn pool, codes staged as they are; the query rows are
//            quantised to e4m3fn and the scores are fp8 products; V^T is
//            converted to bf16 at its fragment read.
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvFp8Q = 2;
constexpr bool fp8_tile(int kv) { return kv != kKvBf16; }

static_assert(kChunks % 64 == 0, "tile must be a whole number of wave-wide loads");
static_assert(kTileLoads % kLoaderWaves == 0, "every loader wave issues the same number of tile loads");
// KV tile buffers in LDS: in each interval the P.V waves read one tile, the QK
// waves the next, and the two after those are in flight.
constexpr int kTileBufs = 4;
// LDS of a split workgroup: the tile ring; two sets (by tile parity) of the
// softmax weights P (one 1 KB block per row group: its lanes' MFMA operands)
// and of the per-row rescale factors; the final row statistics.  The kernel
// has no static LDS.
constexpr int kPBufOff = kTileBufs * kTileBytes;
constexpr int kABufOff = kPBufOff + 2 * kRowGroups * 1024;
constexpr int kStatsOff = kABufOff + 2 * kRowsPerBlock * 4;
constexpr int kSplitLdsBytes = kStatsOff + kRowsPerBlock * 8;
static_assert(kSplitLdsBytes <= 160 * 1024, "split workgroup LDS");
static_assert((kMaxBatch + 1 + 1024) * 4 <= kTileBufs * kTileBytes, "planning scan scratch fits the tile buffers");
static_assert(kTile == 32, "the MFMA layout below assumes 32-token tiles");

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
// Pointers into LDS carry the LDS address space, so that address arithmetic
// stays 32-bit and constant offsets fold into the DS instructions.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const char lds_cchar;

// Swizzle of LDS tile row r: the logical 16-byte chunk c of the row is stored
// at physical chunk c ^ swz(r) (only the low three bits of c change, so a
// chunk stays inside its 128-byte group).  With the 1152-byte row pitch
// (odd and even rows half a bank period apart), swz(r) = r mod 8 leaves both
// reads of the tile free of bank conflicts: the K reads (one chunk of 16
// consecutive rows per 16 lanes) and the transposing V reads (two adjacent
// chunks of 4 consecutive rows per 16 lanes); the LDS bank-conflict counter
// reads zero for the split kernel with it.  swz(r + 16) == swz(r), so the two
// 16-row halves of a tile share lane offsets.
__device__ __forceinline__ int swz(int r) { return r & 7; }

// Byte offset of logical 16-byte chunk c of LDS row r.
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowBytes + (((c & ~7) | ((c & 7) ^ swz(r))) << 4);
}

// The query tokens of request b: the index of the first one and their
// number q_b.  A uniform batch has q_b = q_len at b*q_len; a ragged batch
// reads them from its offsets, and a request whose offsets fall outside
// [0, total_q] or run backwards gets none (so a bad offset never moves a read
// or a write out of the query and output tensors).  q_b is at most q_len, the
// bound the plan was sized for.
struct QExtent {
  int64_t tok0;
  int32_t qb;
};
template <bool RAGGED, class Args>
__device__ __forceinline__ QExtent q_extent(const Args& a, int32_t b) {
  if (!RAGGED || a.qo_indptr == nullptr) return QExtent{(int64_t)b * a.q_len, a.q_len};
  const int32_t s = a.qo_indptr[b], e = a.qo_indptr[b + 1];
  if (s < 0 || e < s || e > a.total_q) return QExtent{0, 0};
  return QExtent{(int64_t)s, e - s < a.q_len ? e - s : a.q_len};
}

// The 18 16-byte query fragments of one lane (dims 32k + 8(l/16) .. +8 of its
// row, k < 18): the 16 of the latent part at byte offsets 64k from pn, the
// two of the rope part at 0 and 64 from pr.  One asm statement also waits
// for them: nothing the compiler emits can touch the registers before the
// data is there, and the compiler keeps no record of these loads, so it
// never waits for them inside the tile loop.  The wait covers every vector
// memory operation the wave issued before; the QK waves that call this issue
// no tile loads (the loader waves do), so it waits for the query alone.
#define MLA_Q_OUT(k) "=&v"(q[k])
__device__ __forceinline__ void load_q_fragments(u32x4_t (&q)[18], const void* pn, const void* pr) {
  asm volatile(
      "global_load_dwordx4 %0, %18, off\n\t"
      "global_load_dwordx4 %1, %18, off offset:64\n\t"
      "global_load_dwordx4 %2, %18, off offset:128\n\t"
      "global_load_dwordx4 %3, %18, off offset:192\n\t"
      "global_load_dwordx4 %4, %18, off offset:256\n\t"
      "global_load_dwordx4 %5, %18, off offset:320\n\t"
      "global_load_dwordx4 %6, %18, off offset:384\n\t"
      "global_load_dwordx4 %7, %18, off offset:448\n\t"
      "global_load_dwordx4 %8, %18, off offset:512\n\t"
      "global_load_dwordx4 %9, %18, off offset:576\n\t"
      "global_load_dwordx4 %10, %18, off offset:640\n\t"
      "global_load_dwordx4 %11, %18, off offset:704\n\t"
      "global_load_dwordx4 %12, %18, off offset:768\n\t"
      "global_load_dwordx4 %13, %18, off offset:832\n\t"
      "global_load_dwordx4 %14, %18, off offset:896\n\t"
      "global_load_dwordx4 %15, %18, off offset:960\n\t"
      "global_load_dwordx4 %16, %19, off\n\t"
      "global_load_dwordx4 %17, %19, off offset:64\n\t"
      "s_waitcnt vmcnt(0)"
      : MLA_Q_OUT(0), MLA_Q_OUT(1), MLA_Q_OUT(2), MLA_Q_OUT(3), MLA_Q_OUT(4), MLA_Q_OUT(5), MLA_Q_OUT(6),
        MLA_Q_OUT(7), MLA_Q_OUT(8), MLA_Q_OUT(9), MLA_Q_OUT(10), MLA_Q_OUT(11), MLA_Q_OUT(12), MLA_Q_OUT(13),
        MLA_Q_OUT(14), MLA_Q_OUT(15), MLA_Q_OUT(16), MLA_Q_OUT(17)
      : "v"(pn), "v"(pr)
      : "memory");
}
#undef MLA_Q_OUT

// Workgroup barrier ordering LDS only.  The tile loop's waves exchange data
// through LDS alone (tile loads are awaited explicitly with vmcnt before the
// barrier), so the barrier must not wait for the global loads in flight: a
// full __syncthreads would drain the tile prefetches at every tile.
// The explicit lgkmcnt(0) makes this wave's own LDS writes complete before it
// arrives: the workgroup fence restricted to LDS emits no wait on gfx950, and
// without one a write issued just before the barrier (the softmax weights, a
// staged output row) could still be in flight when a wave on another SIMD
// passes the barrier and reads it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wave-wide 16-byte-per-lane load from global memory straight into LDS:
// lane l's 16 bytes at gbase + voff land at LDS address lds_addr + 16*l.
// Issued from asm so that the compiler does not see an LDS write in flight:
// it would otherwise wait for every outstanding global load before each
// transposing LDS read.  The caller orders the data with an explicit vmcnt
// wait and an LDS barrier.  M0 is written here; no compiler-generated code in
// the tile loop keeps a value in M0.
__device__ __forceinline__ void dma16(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(lds_addr), "s"(gbase)
               : "memory");
}

// Address of the first element of token t of request b, or null when the
// block-table entry for t is outside [0, N).  The same addressing serves the
// decode and the debug gather.
__device__ __forceinline__ const char* token_row(const void* pool, const int32_t* bt, int32_t W, int32_t P,
                                                 int32_t N, int32_t b, int32_t t, int32_t elem_bytes) {
  const int32_t page = bt[(int64_t)b * W + t / P];
  if ((uint32_t)page >= (uint32_t)N) return nullptr;
  return (const char*)pool + ((int64_t)page * P + (t % P)) * (int64_t)(kRowDim * elem_bytes);
}

// Block-table entries of one request, 64 at a time in one vector register
// (lane l holds entry first + l), so a tile's page id is a lane read rather
// than a memory load whose wait would also drain the tile loads in flight.
// Only entries of pages the piece reads are loaded.
// The window is loaded from asm with its own vmcnt(0): a compiler-visible
// load here would make the compiler wait for every global load in flight
// (the tile prefetches included) before each tile's page lookup.  Lanes past
// the piece's last entry load that last entry again, so every address read is
// one the piece uses.
struct PageWindow {
  int32_t vec = -1;
  int32_t first = 0;
  int32_t end = 0;     // one past the last entry the piece reads
  __device__ __forceinline__ void load(const SplitArgs& a, int b, int first_entry) {
    first = first_entry;
    if (first >= end) {
      vec = -1;
      return;
    }
    const int lane = threadIdx.x & 63;
    const int32_t* ptr = a.bt + (int64_t)b * a.W + min(first + lane, end - 1);
    asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(vec) : "v"(ptr) : "memory");
  }
  __device__ __forceinline__ void init(const SplitArgs& a, int b, int first_entry, int end_entry) {
    end = end_entry;
    load(a, b, first_entry);
  }
  // page id of block-table entry idx (first <= idx < end), uniform across the wave
  __device__ __forceinline__ int32_t page(const SplitArgs& a, int b, int idx) {
    if (idx - first >= 64) load(a, b, idx);
    return __builtin_amdgcn_readlane(vec, idx - first);
  }
};

// ---- KV tile staging.  The 32 rows of a tile are consecutive slots of one
// page (tiles are 32-token aligned and the page size is 32 or 64), so a tile
// is one contiguous run of global memory.
//
// Loader waves issue wave-wide 16-byte loads that write LDS directly
// (global_load_lds_dwordx4: lane l lands at the wave's LDS base + 16*l); a
// lane picks the global chunk whose swizzled LDS position is its own.  Lanes
// of rows past the piece's last token re-read a chunk of the tile's first
// row, so every LDS row holds finite values; their scores are masked.
template <int KV>
struct Stage;

template <>
struct Stage<kKvBf16> {
  // Load i of loader wave w fills the 64 physical LDS chunks starting at
  // P = 64*(w + kLoaderWaves*i).  The chunk p = P + l of lane l holds logical
  // chunk (p mod 72) ^ z(r) of row r = p / 72, z(r) = swz(r), so its
  // source offset inside the tile is 16*(p ^ z(r)) = 16*P + 16*(l ^ z(r))
  // (P is a multiple of 8 and z only flips the low three bits).  The lane
  // part 16*(l ^ z) < 1024 takes 10 bits: three loads share a register.
  static constexpr int kPacked = (kLoadsPerWave + 2) / 3;
  uint32_t xoff[kPacked];
  __device__ __forceinline__ static int first_chunk(int wave, int i) { return 64 * (wave + kLoaderWaves * i); }
  // lw: this wave's index among the loader waves
  __device__ __forceinline__ void init(int lw) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kPacked; j++) xoff[j] = 0;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; i++) {
      const int r = (first_chunk(lw, i) + lane) / 72;
      xoff[i / 3] |= (uint32_t)(16 * (lane ^ swz(r))) << (10 * (i % 3));
    }
  }
  __device__ __forceinline__ uint32_t lane_off(int i) const { return (xoff[i / 3] >> (10 * (i % 3))) & 1023u; }
  // Issues exactly kLoadsPerWave loads per loader wave for a tile that holds
  // at least one valid token (the waits below count on it); rows past the
  // last valid token re-read the same chunk of the tile's first row, so every
  // LDS row stays finite.  A block-table entry outside [0, N) reads page 0 in
  // its place (the result is undefined then, but the count holds).  A tile
  // with no valid token (only a request with no token at all) issues no load
  // and is filled with zeros.
  // Called by loader wave lw; returns the number of loads it issued (0 or kLoadsPerWave).
  __device__ __forceinline__ int issue(const SplitArgs& a, lds_char* buf, PageWindow& pw, int b, int ts,
                                       int tok_end, int lw) const {
    // wave-uniform by construction; said so, so that the tile base lands in
    // scalar registers as the DMA instruction requires
    b = __builtin_amdgcn_readfirstlane(b);
    ts = __builtin_amdgcn_readfirstlane(ts);
    tok_end = __builtin_amdgcn_readfirstlane(tok_end);
    const int wave = lw;
    if (ts >= tok_end) {
      // no valid token (a request with no token at all): zeros instead, so
      // that the masked scores meet finite values
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; i++)
        *(__attribute__((address_space(3))) u32x4_t*)(buf + wave * 1024 + kLoaderWaves * 1024 * i + 16 * lane) =
            u32x4_t{0u, 0u, 0u, 0u};
      return 0;
    }
    const int32_t page = pw.page(a, b, ts >> a.p_shift);
    const int32_t pg = (uint32_t)page < (uint32_t)a.N ? page : 0;
    const char* base = (const char*)a.pool + (((int64_t)pg << a.p_shift) + (ts & (a.P - 1))) * (int64_t)kRowBytes;
    const uint32_t dst = (uint32_t)(uintptr_t)(buf + wave * 1024);
    // Opaque copies: the offsets are unpacked here, once per tile, instead of
    // being hoisted out of the tile loop as nine live registers.
    Stage<kKvBf16> o = *this;
#pragma unroll
    for (int j = 0; j < kPacked; j++) asm("" : "+v"(o.xoff[j]));
    if (ts + kTile <= tok_end) {
      // whole tile: uniform base + 10-bit lane offset
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; i++)
        dma16(base + 16 * first_chunk(wave, i), o.lane_off(i), dst + kLoaderWaves * 1024 * i);
    } else {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; i++) {
        const int P = first_chunk(wave, i);
        const int r = (P + lane) / 72;
        const uint32_t off = (uint32_t)(16 * P) + o.lane_off(i) - (ts + r < tok_end ? 0u : (uint32_t)(r * kRowBytes));
        dma16(base, off, dst + kLoaderWaves * 1024 * i);
      }
    }
    return kLoadsPerWave;
  }
  // Wait until this tile's loads have landed while the loads of `later`
  // tiles issued after it may stay in flight (loads complete in issue order).
  __device__ __forceinline__ void wait(int later) const {
    static_assert(kLoadsPerWave == 9, "the vmcnt immediates assume 9 loads per loader wave and tile");
    if (later >= 2) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t word) {
  // Two e4m3fn codes (the low or the high half of the word) straight to a
  // bf16 pair by the gfx950 scaled conversion with scale 1: every e4m3fn
  // value is a bf16 value, so the conversion is exact.
  typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, (bf16x2_cvt_t)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI));
}

// fp8 pool: the codes are staged as they are.  A tile is 32
// rows of 576 bytes (36 16-byte chunks) in the first half of its ring buffer.
// Logical chunk c of row r sits at physical chunk c ^ swz8(r): only the low
// two bits change, so a chunk stays inside its aligned group of four (36 is
// a multiple of four).  The compute waves read the tile in 8-byte pieces: the
// K fragments (8 bytes of 16 consecutive rows per 16 lanes) and the 8-bit
// transposing V reads (8 bytes of 8 rows per 16 lanes, two lanes to a row).
// With the 576-byte pitch and swz8(r) = (r/4) mod 4, and the second 16-token
// block of K taken in the row order 16 + (i ^ 8), both read at the rate of
// conflict-free linear 8-byte reads (measured on gfx950 against other
// swizzles and row orders, which ran 20-130 % slower).
__device__ __forceinline__ int swz8(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int lds_off8(int r, int c) { return r * kRowDim + ((c ^ swz8(r)) << 4); }
constexpr int kTile8Bytes = kTile * kRowDim;                    // 18432
constexpr int kLoaders8 = 2;                                    // loader waves issuing fp8 tile loads
constexpr int kLoads8 = kTile8Bytes / 1024 / kLoaders8;         // 9 wave-wide 1 KB loads each
static_assert(kLoads8 == kLoadsPerWave, "the fp8 tile loads share the bf16 tile's wait counts");
static_assert(kTile8Bytes % (1024 * kLoaders8) == 0 && (kRowDim / 16) % 4 == 0, "fp8 tile staging");

// Loader wave lw < kLoaders8, load i fills the 64 physical chunks starting at
// 64*(lw + kLoaders8*i): lane l's chunk p holds logical chunk
// (p mod 36) ^ swz8(r) of row r = p / 36, at byte 576r + 16c of the tile's
// contiguous run in the pool (< 2^16: two offsets to a register).  The other
// loader waves issue nothing for an fp8 tile.
struct Stage8 {
  static constexpr int kPacked = (kLoads8 + 1) / 2;
  uint32_t xoff[kPacked];
  __device__ __forceinline__ static int first_chunk(int lw, int i) { return 64 * (lw + kLoaders8 * i); }
  __device__ __forceinline__ void init(int lw) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kPacked; j++) xoff[j] = 0;
    if (lw >= kLoaders8) return;
#pragma unroll
    for (int i = 0; i < kLoads8; i++) {
      const int p = first_chunk(lw, i) + lane;
      const int r = p / 36;
      const int c = (p - 36 * r) ^ swz8(r);
      xoff[i / 2] |= (uint32_t)(r * kRowDim + 16 * c) << (16 * (i % 2));
    }
  }
  __device__ __forceinline__ uint32_t lane_off(int i) const { return (xoff[i / 2] >> (16 * (i % 2))) & 0xFFFFu; }
  // As Stage<0>::issue: kLoads8 loads per issuing wave for a tile with a
  // valid token (rows past the last one re-read the same chunk of row 0; a
  // block-table entry outside [0, N) reads page 0), zeros for a tile
  // without one.
  __device__ __forceinline__ int issue(const SplitArgs& a, lds_char* buf, PageWindow& pw, int b, int ts, int tok_end,
                                       int lw) const {
    if (lw >= kLoaders8) return 0;
    b = __builtin_amdgcn_readfirstlane(b);
    ts = __builtin_amdgcn_readfirstlane(ts);
    tok_end = __builtin_amdgcn_readfirstlane(tok_end);
    const int lane = threadIdx.x & 63;
    if (ts >= tok_end) {
#pragma unroll
      for (int i = 0; i < kLoads8; i++)
        *(__attribute__((address_space(3))) u32x4_t*)(buf + 1024 * (lw + kLoaders8 * i) + 16 * lane) =
            u32x4_t{0u, 0u, 0u, 0u};
      return 0;
    }
    const int32_t page = pw.page(a, b, ts >> a.p_shift);
    const int32_t pg = (uint32_t)page < (uint32_t)a.N ? page : 0;
    const char* base = (const char*)a.pool + (((int64_t)pg << a.p_shift) + (ts & (a.P - 1))) * (int64_t)kRowDim;
    const uint32_t dst = (uint32_t)(uintptr_t)(buf + 1024 * lw);
    Stage8 o = *this;
#pragma unroll
    for (int j = 0; j < kPacked; j++) asm("" : "+v"(o.xoff[j]));
    if (ts + kTile <= tok_end) {
#pragma unroll
      for (int i = 0; i < kLoads8; i++) dma16(base, o.lane_off(i), dst + 1024 * kLoaders8 * i);
    } else {
#pragma unroll
      for (int i = 0; i < kLoads8; i++) {
        const int r = (first_chunk(lw, i) + lane) / 36;
        const uint32_t off = o.lane_off(i) - (ts + r < tok_end ? 0u : (uint32_t)(r * kRowDim));
        dma16(base, off, dst + 1024 * kLoaders8 * i);
      }
    }
    return kLoads8;
  }
  __device__ __forceinline__ void wait(int later) const {
    if (later >= 2) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};
template <>
struct Stage<kKvFp8> : Stage8 {};
template <>
struct Stage<kKvFp8Q> : Stage8 {};

#ifndef MLA_PERMLANE
#define MLA_PERMLANE 1
#endif
// Reductions over the four lanes l, l^16, l^32, l^48 that hold one query row.
// The gfx950 lane swaps are plain VALU operations; each returns the two
// swapped registers, and combining both gives the partner's value in every
// lane.
__device__ __forceinline__ float row_max4(float x) {
#if MLA_PERMLANE
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
#else
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
#endif
}
__device__ __forceinline__ float row_sum4(float x) {
#if MLA_PERMLANE
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  const uint32_t v = __builtin_bit_cast(uint32_t, x);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
#else
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
#endif
}

// An LDS address the optimiser cannot look into: per-read constant offsets
// then fold into the DS instructions instead of being re-added to the tile
// buffer arithmetic for every read.
__device__ __forceinline__ lds_cchar* opaque_lds(lds_cchar* p) {
  uint32_t v = (uint32_t)(uintptr_t)p;
  asm("" : "+v"(v));
  return (lds_cchar*)(uintptr_t)v;
}

#ifndef MLA_PIN_ORDER
#define MLA_PIN_ORDER 1
#endif
// Issue priorities of the QK and loader waves (the PV waves keep 0).
#ifndef MLA_PRIO_QK
#define MLA_PRIO_QK 1
#endif
#ifndef MLA_PRIO_LD
#define MLA_PRIO_LD 3
#endif
// Row groups per PV wave.  The kPVWaves PV waves split the (row group,
// 16-dim block) grid: kPVRowGroups row groups times 1/kPVDimParts of the 32
// dim blocks each, so a V^T fragment read from LDS feeds kPVRowGroups MFMAs.
#ifndef MLA_PV_RG
#define MLA_PV_RG 2
#endif
constexpr int kPVRowGroups = MLA_PV_RG;
constexpr int kPVDimParts = kPVWaves * kPVRowGroups / kRowGroups;   // dim ranges per row group
static_assert(kPVDimParts * kRowGroups == kPVWaves * kPVRowGroups, "PV waves cover the grid exactly");
constexpr int kPVBlocks = kVBlocks / kPVDimParts;   // 16-dim blocks of one PV wave
static_assert(kRowGroups % kPVRowGroups == 0 && kPVBlocks % 4 == 0, "PV work split");
__device__ __forceinline__ s16x4_t lds_read_tr16(lds_cchar* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
}

// Two floats to a bf16 pair (lo, hi), round to nearest even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){lo, hi}, bf16x2_t));
}

constexpr int kQKSteps = 2 * kQSteps;   // (token block, k-step) pairs of S^T = K . Q^T

// Lane-dependent parts of the LDS addresses a wave reads, fixed for the
// whole kernel; every per-read remainder is a compile-time offset.
//  K fragment of step s = 2k + tb: token 16tb + l%16, dims 32k + 8(l/16)..+8,
//    at kbase[k&1] + 18432*tb + 128*(k>>1).
//  V^T block mb (two transposing reads): lane i of 16-lane group g reads
//    4 dims of token 4g + i/4 (and of token 16 + 4g + i/4); the hardware hands
//    lane i dim 16mb + i of the group's 4 tokens.  At vbase[mb&3] +
//    18432*second + 128*(mb>>2).
struct LaneOffsets {
  int kbase[2];
  int vbase[4];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i16 = lane & 15;
    const int zk = swz(i16);                             // swizzle of rows i16 and 16 + i16
#pragma unroll
    for (int p = 0; p < 2; p++) kbase[p] = i16 * kRowBytes + 16 * ((g + 4 * p) ^ zk);
    const int vr = 4 * g + (i16 >> 2);                   // tokens vr and vr + 16 share a swizzle
    const int zv = swz(vr);
    const int bit = (i16 >> 1) & 1;
#pragma unroll
    for (int m4 = 0; m4 < 4; m4++) vbase[m4] = vr * kRowBytes + 16 * ((2 * m4 + bit) ^ zv) + 8 * (i16 & 1);
  }
};

// The same for a tile of fp8 codes (lds_off8).
//  K fragment of step k (dims 32k + 8g .. +8 of the lane's token, 8 codes):
//    token i16 of the first 16-token block and 16 + (i16 ^ 8) of the second
//    (tb), at kbase[tb][k&1] + 64*(k>>1).
//  V^T block mb (one 8-bit transposing read): lane 16G + 2m + h reads 8
//    codes of token tok(G, m), dims 16mb + 8h .. +8, where tok(G, m) is
//    4G + m for m < 4 and 16 + ((4G + m - 4) ^ 8) otherwise: the order of
//    the lane's eight scores.  The hardware hands lane j of the group dim
//    16mb + j of the group's 8 tokens.  At vbase[mb&3] + 64*(mb>>2).
struct LaneOffsets8 {
  int kbase[2][2];
  int vbase[4];
  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int tb = 0; tb < 2; tb++) {
      const int r = tb ? 16 + (i16 ^ 8) : i16;
#pragma unroll
      for (int e = 0; e < 2; e++) kbase[tb][e] = r * kRowDim + 16 * ((2 * e + (g >> 1)) ^ swz8(r)) + 8 * (g & 1);
    }
    const int h = i16 & 1, m = i16 >> 1;
    const int r = m < 4 ? 4 * g + m : 16 + ((4 * g + m - 4) ^ 8);
#pragma unroll
    for (int m4 = 0; m4 < 4; m4++) vbase[m4] = r * kRowDim + 16 * (m4 ^ swz8(r)) + 8 * h;
  }
};
template <int KV>
struct LaneOffsetsSel {
  typedef LaneOffsets type;
};
template <>
struct LaneOffsetsSel<kKvFp8> {
  typedef LaneOffsets8 type;
};
template <>
struct LaneOffsetsSel<kKvFp8Q> {
  typedef LaneOffsets8 type;
};
template <int KV>
using LaneOffsetsOf = typename LaneOffsetsSel<KV>::type;

// Eight e4m3fn codes (two words, code e in byte e%4 of word e/4) to the
// bf16x8 fragment of their values.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(u32x2_t w) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                                              fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])});
}

// QK wave, one tile: S^T[32 tokens x 16 rows] = K_tile . Q^T (36 MFMA), the
// K reads kKAhead steps ahead of their MFMA.  Lane l ends with the scores of
// row l%16 for tokens 4g + r (s0[r]) and 16 + 4g + r (s1[r]), g = l/16.
template <int kKAhead, int kSChains>
__device__ __forceinline__ void qk_tile(const bf16x8_t (&qf)[kQSteps], lds_cchar* cur, const LaneOffsets& lo_,
                                        f32x4v_t& s0, f32x4v_t& s1) {
  static_assert(kSChains == 2 || kSChains == 4, "one or two accumulation chains per token block");
  constexpr int kCh = kSChains / 2;
  lds_cchar* kp[2] = {opaque_lds(cur + lo_.kbase[0]), opaque_lds(cur + lo_.kbase[1])};
  auto kread = [&](int s) -> bf16x8_t {
    const int k = s >> 1, tb = s & 1;
    return *(__attribute__((address_space(3))) const bf16x8_t*)(kp[k & 1] + 18432 * tb + 128 * (k >> 1));
  };
  bf16x8_t kb[kKAhead];
#pragma unroll
  for (int s = 0; s < kKAhead; s++) kb[s] = kread(s);
  f32x4v_t sp[2][kCh];
#pragma unroll
  for (int tb = 0; tb < 2; tb++)
#pragma unroll
    for (int c = 0; c < kCh; c++) sp[tb][c] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kQKSteps; s++) {
    const bf16x8_t kf = kb[s % kKAhead];
    if (s + kKAhead < kQKSteps) kb[s % kKAhead] = kread(s + kKAhead);
    const int k = s >> 1, tb = s & 1;
    sp[tb][k % kCh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[k], sp[tb][k % kCh], 0, 0, 0);
    // keep each step's read kKAhead steps ahead of its MFMA: left alone, the
    // scheduler sinks the reads next to their use and exposes the LDS latency
    if (MLA_PIN_ORDER) __builtin_amdgcn_sched_barrier(0);
  }
  s0 = sp[0][0];
  s1 = sp[1][0];
  if constexpr (kCh == 2) {
    s0 += sp[0][1];
    s1 += sp[1][1];
  }
}

// QK wave, one tile of fp8 codes, bf16 products: as qk_tile, each K
// fragment read as 8 codes and converted to bf16 (exactly) before its MFMA.
// s1[r] is the score of token 16 + ((4g + r) ^ 8).
template <int kKAhead, int kSChains>
__device__ __forceinline__ void qk_tile_cvt(const bf16x8_t (&qf)[kQSteps], lds_cchar* cur, const LaneOffsets8& lo_,
                                            f32x4v_t& s0, f32x4v_t& s1) {
  static_assert(kSChains == 2 || kSChains == 4, "one or two accumulation chains per token block");
  constexpr int kCh = kSChains / 2;
  lds_cchar* kp[2][2] = {{opaque_lds(cur + lo_.kbase[0][0]), opaque_lds(cur + lo_.kbase[0][1])},
                         {opaque_lds(cur + lo_.kbase[1][0]), opaque_lds(cur + lo_.kbase[1][1])}};
  auto kread = [&](int s) -> u32x2_t {
    const int k = s >> 1, tb = s & 1;
    return *(__attribute__((address_space(3))) const u32x2_t*)(kp[tb][k & 1] + 64 * (k >> 1));
  };
  u32x2_t kb[kKAhead];
#pragma unroll
  for (int s = 0; s < kKAhead; s++) kb[s] = kread(s);
  f32x4v_t sp[2][kCh];
#pragma unroll
  for (int tb = 0; tb < 2; tb++)
#pragma unroll
    for (int c = 0; c < kCh; c++) sp[tb][c] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kQKSteps; s++) {
    const bf16x8_t kf = fp8x8_to_bf16x8(kb[s % kKAhead]);
    if (s + kKAhead < kQKSteps) kb[s % kKAhead] = kread(s + kKAhead);
    const int k = s >> 1, tb = s & 1;
    sp[tb][k % kCh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[k], sp[tb][k % kCh], 0, 0, 0);
    if (MLA_PIN_ORDER) __builtin_amdgcn_sched_barrier(0);
  }
  s0 = sp[0][0];
  s1 = sp[1][0];
  if constexpr (kCh == 2) {
    s0 += sp[0][1];
    s1 += sp[1][1];
  }
}

// The query rows of a QK wave as e4m3fn codes, in the k order of the fp8
// MFMAs: main[kb] is the B operand of 16x16x128 step kb (dims 128kb ..
// +128): lane l (row l%16, g = l/16) holds in bytes 8j .. 8j+7 dims
// 32(4kb + j) + 8g .. +8, the dims its K fragment of step 4kb + j holds, so
// the k order inside the MFMA is the same for both operands.  rope[s] is the
// B operand of 16x16x32 step s over the rope dims 512 + 32s .. +32 (lane
// bytes = dims 512 + 32s + 8g .. +8).
typedef int i32x8_t __attribute__((ext_vector_type(8)));
struct QCodes {
  i32x8_t main[4];
  u32x2_t rope[2];
};

// Eight bf16 query values to their e4m3fn codes (two words).
__device__ __forceinline__ u32x2_t bf16x8_to_e4m3(u32x4_t v) {
  auto lo = [](uint32_t w) { return __builtin_bit_cast(float, w << 16); };
  auto hi = [](uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); };
  return u32x2_t{e4m3fn_x4(lo(v[0]), hi(v[0]), lo(v[1]), hi(v[1])), e4m3fn_x4(lo(v[2]), hi(v[2]), lo(v[3]), hi(v[3]))};
}

// QK wave, one tile of fp8 codes, fp8 products: per 16-token block four
// 16x16x128 MFMAs over the 512 latent dims (each fed by four 8-byte K
// fragment reads) and two 16x16x32 ones over the 64 rope dims, the two
// blocks' accumulations alternating, operands read two MFMAs ahead.
// s1[r] is the score of token 16 + ((4g + r) ^ 8).
__device__ __forceinline__ void qk_tile_q8(const QCodes& q8, lds_cchar* cur, const LaneOffsets8& lo_, f32x4v_t& s0,
                                           f32x4v_t& s1) {
  typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
  lds_cchar* kp[2][2] = {{cur + lo_.kbase[0][0], cur + lo_.kbase[0][1]}, {cur + lo_.kbase[1][0], cur + lo_.kbase[1][1]}};
  // Each read's address is opaque: left alone, the compiler pairs the reads
  // 64 bytes apart into one two-address read, which the LDS serves with bank
  // conflicts (measured: 19.5 M conflict cycles per fp8 dispatch instead of
  // 0.5 M).
  auto kread = [&](int tb, int k) -> u32x2_t {
    return *(__attribute__((address_space(3))) const u32x2_t*)opaque_lds(kp[tb][k & 1] + 64 * (k >> 1));
  };
  // MFMAs i = 0..7: 16x16x128 step kb = i/2 of block tb = i%2; i = 8..11:
  // 16x16x32 rope step s = (i-8)/2 of block tb = i%2
  constexpr int kOps = 12, kAhead = 2;
  i32x8_t A[kAhead + 1];
  u32x2_t R[2][2];
  auto fetch = [&](int i) {
    const int tb = i & 1;
    if (i < 8) {
      const int kb = i >> 1;
      const u32x2_t r0 = kread(tb, 4 * kb), r1 = kread(tb, 4 * kb + 1), r2 = kread(tb, 4 * kb + 2),
                    r3 = kread(tb, 4 * kb + 3);
      A[i % (kAhead + 1)] = __builtin_bit_cast(i32x8_t, u32x8_t{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]});
    } else {
      R[tb][(i - 8) >> 1] = kread(tb, 16 + ((i - 8) >> 1));
    }
  };
#pragma unroll
  for (int i = 0; i < kAhead; i++) fetch(i);
  f32x4v_t sp[2] = {f32x4v_t{0.f, 0.f, 0.f, 0.f}, f32x4v_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < kOps; i++) {
    if (i + kAhead < kOps) fetch(i + kAhead);
    const int tb = i & 1;
    if (i < 8) {
      // e4m3 operands (format 0 for both), unit scales (E8M0 127)
      sp[tb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[i % (kAhead + 1)], q8.main[i >> 1], sp[tb], 0, 0,
                                                                 0, 127, 0, 127);
    } else {
      const int st = (i - 8) >> 1;
      sp[tb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, R[tb][st]),
                                                          __builtin_bit_cast(long, q8.rope[st]), sp[tb], 0, 0, 0);
    }
    if (MLA_PIN_ORDER) __builtin_amdgcn_sched_barrier(0);
  }
  s0 = sp[0];
  s1 = sp[1];
}

// QK wave, one tile: the online softmax of the lane's 8 scores of its row.
// The bf16 weights go to LDS as the lane's 16-byte B operand of the PV MFMA
// (tokens in the order of the scores: the V^T reads follow the same order),
// and the factor by which the row's running output is to be rescaled.
// kTb1Perm: s1[r] holds token 16 + ((4g + r) ^ 8) (fp8 tiles), else 16 + 4g + r.
template <bool kTb1Perm>
__device__ __forceinline__ void softmax_tile(f32x4v_t s0, f32x4v_t s1, float& m_run, float& l_run, int ts, int limit,
                                             int lim_min, float scale_log2, lds_char* pout, lds_char* aout) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  // raw scores of the lane's 8 tokens; masked tokens become -inf (a tile
  // below lim_min is visible to every row of the wave)
  float sv[8];
#pragma unroll
  for (int e = 0; e < 8; e++) sv[e] = e < 4 ? s0[e & 3] : s1[e & 3];
  if (ts + kTile > lim_min) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int t = e < 4 ? ts + 4 * g + e : ts + 16 + (kTb1Perm ? ((4 * g + (e & 3)) ^ 8) : 4 * g + (e & 3));
      sv[e] = t < limit ? sv[e] : kNegInf;
    }
  }
  // row maximum in log2 units: the scale is positive, so it is taken on the
  // raw scores and scaled once.  The running maximum is raised only when a
  // tile's maximum exceeds it by more than kRescaleSlack.
  float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  mx = row_max4(mx) * scale_log2;
  const bool need = mx > m_run + kRescaleSlack;
  float alpha = 1.f;
  if (__any(need)) {
    const float m_new = need ? mx : m_run;
    alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // m_run = -inf gives 0
    l_run *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run == kNegInf ? 0.f : m_run;
  float psum = 0.f;
  u32x4_t pk;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * e], scale_log2, -m_use));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * e + 1], scale_log2, -m_use));
    psum += p0 + p1;
    pk[e] = pack_bf16x2(p0, p1);
  }
  l_run += psum;
  *(__attribute__((address_space(3))) u32x4_t*)(pout + 16 * lane) = pk;
  if (g == 0) *(__attribute__((address_space(3))) float*)aout = alpha;
}

// PV wave, one tile: for its kPVRowGroups row groups and kPVBlocks dim
// blocks, O^T = alpha * O^T + V^T[16 dims x 32] . P^T (kPVRowGroups MFMA per
// block), V^T from the LDS tile through the transposing read, kVAhead blocks
// ahead of their MFMAs.  vcur is the tile plus the wave's first dim block.
template <int kVAhead>
__device__ __forceinline__ void pv_tile(f32x4v_t (&acc)[kPVRowGroups][kPVBlocks], lds_cchar* vcur,
                                        const LaneOffsets& lo_, lds_cchar* pin, lds_cchar* ain) {
  const int lane = threadIdx.x & 63;
  lds_cchar* vp[4] = {opaque_lds(vcur + lo_.vbase[0]), opaque_lds(vcur + lo_.vbase[1]),
                      opaque_lds(vcur + lo_.vbase[2]), opaque_lds(vcur + lo_.vbase[3])};
  auto vread = [&](int mb, int second) -> u32x2_t {
    return __builtin_bit_cast(u32x2_t, lds_read_tr16(vp[mb & 3] + 18432 * second + 128 * (mb >> 2)));
  };
  u32x2_t vb[kVAhead][2];
#pragma unroll
  for (int m = 0; m < kVAhead; m++) {
    vb[m][0] = vread(m, 0);
    vb[m][1] = vread(m, 1);
  }
  bf16x8_t pf[kPVRowGroups];
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++)
    pf[r] = *(__attribute__((address_space(3))) const bf16x8_t*)(pin + 1024 * r + 16 * lane);
  float alpha[kPVRowGroups];
  if constexpr (kPVRowGroups == 4) {
    const f32x4v_t a4 = *(__attribute__((address_space(3))) const f32x4v_t*)ain;
#pragma unroll
    for (int r = 0; r < 4; r++) alpha[r] = a4[r];
  } else {
#pragma unroll
    for (int r = 0; r < kPVRowGroups; r++) alpha[r] = ((__attribute__((address_space(3))) const float*)ain)[r];
  }
  bool any = false;
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++) any |= alpha[r] != 1.f;
  if (__any(any)) {
#pragma unroll
    for (int r = 0; r < kPVRowGroups; r++)
#pragma unroll
      for (int mb = 0; mb < kPVBlocks; mb++) acc[r][mb] *= alpha[r];
  }
#pragma unroll
  for (int mb = 0; mb < kPVBlocks; mb++) {
    const u32x2_t lo = vb[mb % kVAhead][0], hi = vb[mb % kVAhead][1];
    if (mb + kVAhead < kPVBlocks) {
      vb[mb % kVAhead][0] = vread(mb + kVAhead, 0);
      vb[mb % kVAhead][1] = vread(mb + kVAhead, 1);
    }
    const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
    for (int r = 0; r < kPVRowGroups; r++)
      acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r], acc[r][mb], 0, 0, 0);
    if (MLA_PIN_ORDER) __builtin_amdgcn_sched_barrier(0);
  }
}

// PV wave, one tile of fp8 codes: as pv_tile, each V^T block one 8-bit
// transposing read of 8 codes per lane, converted to bf16 (exactly) before
// its MFMAs.
template <int kVAhead>
__device__ __forceinline__ void pv_tile8(f32x4v_t (&acc)[kPVRowGroups][kPVBlocks], lds_cchar* vcur,
                                         const LaneOffsets8& lo_, lds_cchar* pin, lds_cchar* ain) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  lds_cchar* vp[4] = {opaque_lds(vcur + lo_.vbase[0]), opaque_lds(vcur + lo_.vbase[1]),
                      opaque_lds(vcur + lo_.vbase[2]), opaque_lds(vcur + lo_.vbase[3])};
  auto vread = [&](int mb) -> u32x2_t {
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                           (__attribute__((address_space(3))) i32x2_t*)(vp[mb & 3] + 64 * (mb >> 2))));
  };
  u32x2_t vb[kVAhead];
#pragma unroll
  for (int m = 0; m < kVAhead; m++) vb[m] = vread(m);
  bf16x8_t pf[kPVRowGroups];
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++)
    pf[r] = *(__attribute__((address_space(3))) const bf16x8_t*)(pin + 1024 * r + 16 * lane);
  float alpha[kPVRowGroups];
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++) alpha[r] = ((__attribute__((address_space(3))) const float*)ain)[r];
  bool any = false;
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++) any |= alpha[r] != 1.f;
  if (__any(any)) {
#pragma unroll
    for (int r = 0; r < kPVRowGroups; r++)
#pragma unroll
      for (int mb = 0; mb < kPVBlocks; mb++) acc[r][mb] *= alpha[r];
  }
#pragma unroll
  for (int mb = 0; mb < kPVBlocks; mb++) {
    const bf16x8_t vf = fp8x8_to_bf16x8(vb[mb % kVAhead]);
    if (mb + kVAhead < kPVBlocks) vb[mb % kVAhead] = vread(mb + kVAhead);
#pragma unroll
    for (int r = 0; r < kPVRowGroups; r++)
      acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[r], acc[r][mb], 0, 0, 0);
    if (MLA_PIN_ORDER) __builtin_amdgcn_sched_barrier(0);
  }
}

// The pipeline of one piece runs in intervals j = -1 .. nt-1, each opened by
// a workgroup barrier; in interval j the QK waves take tile j+1, the PV waves
// tile j, and the loaders issue tile j+3 into the buffer of tile j-1 (free:
// the PV waves finished it in interval j-1, the QK waves in j-2).  Three
// more barriers close the piece: after the first every tile is done and the
// QK waves' final row max and sum are in LDS; after the second the PV waves
// have staged the output rows in the tile buffers; after the third those
// rows have been copied out.
__device__ __forceinline__ int tile_buf(int t) { return t & (kTileBufs - 1); }
static_assert((kTileBufs & (kTileBufs - 1)) == 0, "tile_buf masks the tile index");

template <int KV>
__device__ void load_piece(const SplitArgs& a, lds_char* lds, Stage<KV>& stg, const Piece& pc, int lw) {
  const int b = pc.b;
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int tok_end = min(pc.tile1 * kTile, L);
  const int nt = pc.tile1 - pc.tile0;
  PageWindow pw;
  pw.init(a, b, (pc.tile0 * kTile) >> a.p_shift, (tok_end + a.P - 1) >> a.p_shift);
  auto put = [&](int t) {   // tile t of the piece into its ring buffer
    stg.issue(a, lds + tile_buf(t) * kTileBytes, pw, b, (pc.tile0 + t) * kTile, tok_end, lw);
  };
  for (int t = 0; t < 2 && t < nt; t++) put(t);
  for (int j = -1; j < nt; j++) {
    // tile j+1 is in LDS before barrier j; tile j+2 may still be in flight
    stg.wait(j + 2 < nt ? 1 : 0);
    lds_barrier();
    if (j + 3 < nt) put(j + 3);
  }
  lds_barrier();
  lds_barrier();
  lds_barrier();
}

// The QK waves' side of one piece: the scores and the online softmax of the
// wave's 16 rows.
template <int KV, bool RAGGED>
__device__ void qk_piece(const SplitArgs& a, lds_char* lds, const LaneOffsetsOf<KV>& lo_, const Piece& pc, int w) {
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int b = pc.b;
  const int L = clamp_len(a.seq_lens[b], a.max_seq_len);
  const int tok_end = min(pc.tile1 * kTile, L);
  const int nt = pc.tile1 - pc.tile0;
  const int rib = 16 * w + i16;   // this lane's row in the block
  const int row = pc.rb * kRowsPerBlock + rib;
  const QExtent qe = q_extent<RAGGED>(a, b);
  const bool row_ok = row < qe.qb * a.H;
  const int jrow = row_ok ? row / a.H : 0, hrow = row_ok ? row - jrow * a.H : 0;
  const int limit = min(tok_end, L - qe.qb + 1 + jrow);   // tokens t < limit are visible to this row
  // smallest limit over the wave's rows: tiles below it need no mask
  int lim_min = limit;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, d));
  lim_min = __builtin_amdgcn_readfirstlane(lim_min);
  // Q^T B-operand fragments: lane holds row i16, dims 32k + 8g .. +8; rows
  // past the request's last query row load its first row and are zeroed.
  static_assert(kQSteps == 18, "load_q_fragments loads 18 fragments");
  bf16x8_t qf[kQSteps];
  {
    // query token b*q_len + j, head h: the latent part and the rope part
    // each through its own token and head strides
    const int64_t tok = qe.tok0 + (row_ok ? jrow : 0);
    const int64_t h = row_ok ? hrow : 0;
    u32x4_t qv[kQSteps];
    load_q_fragments(qv, a.q + tok * a.qn_tok + h * a.qn_head + 8 * g, a.q_rope + tok * a.qr_tok + h * a.qr_head + 8 * g);
    if (a.rope_cs != nullptr && row_ok) {
      // rotary embedding of the rope part at the token's position: lane g
      // holds rope dims 8g..8g+7 (fragment 16) and 32+8g..32+8g+7 (17)
      const float* cs = rope_row(a.rope_cs, a.positions, tok, a.rope_max_pos);
      if (a.rope_neox) {
        rope_rotate_halves(qv[16], qv[17], cs, 8 * g);
      } else {
        rope_rotate_interleaved(qv[16], cs, 8 * g);
        rope_rotate_interleaved(qv[17], cs, 32 + 8 * g);
      }
    }
#pragma unroll
    for (int k = 0; k < kQSteps; k++) qf[k] = __builtin_bit_cast(bf16x8_t, row_ok ? qv[k] : u32x4_t{0u, 0u, 0u, 0u});
  }
  // fp8 products: the rows (rotated, when a rotary embedding applies) as
  // e4m3fn codes of their bf16 values, scale 1
  QCodes q8;
  if constexpr (KV == kKvFp8Q) {
    typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
    u32x2_t c[kQSteps];
#pragma unroll
    for (int k = 0; k < kQSteps; k++) c[k] = bf16x8_to_e4m3(__builtin_bit_cast(u32x4_t, qf[k]));
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
      q8.main[kb] = __builtin_bit_cast(i32x8_t, u32x8_t{c[4 * kb][0], c[4 * kb][1], c[4 * kb + 1][0], c[4 * kb + 1][1],
                                                        c[4 * kb + 2][0], c[4 * kb + 2][1], c[4 * kb + 3][0],
                                                        c[4 * kb + 3][1]});
    q8.rope[0] = c[16];
    q8.rope[1] = c[17];
  }
  float m_run = kNegInf, l_run = 0.f;
  for (int j = -1; j < nt; j++) {
    lds_barrier();
    const int t = j + 1;
    if (t < nt) {
      f32x4v_t s0, s1;
      lds_cchar* cur = lds + tile_buf(t) * kTileBytes;
      if constexpr (KV == kKvFp8Q)
        qk_tile_q8(q8, cur, lo_, s0, s1);
      else if constexpr (KV == kKvFp8)
        qk_tile_cvt<MLA_F8_KA, MLA_F8_SC>(qf, cur, lo_, s0, s1);
      else
        qk_tile<MLA_KA, MLA_SC>(qf, cur, lo_, s0, s1);
      softmax_tile<fp8_tile(KV)>(s0, s1, m_run, l_run, (pc.tile0 + t) * kTile, limit, lim_min, a.scale_log2,
                   lds + kPBufOff + ((t & 1) * kRowGroups + w) * 1024,
                   lds + kABufOff + (t & 1) * (kRowsPerBlock * 4) + 16 * i16 + 4 * w);
    }
  }
  const float l_tot = row_sum4(l_run);
  if (g == 0) {
    float* stats = (float*)(lds + kStatsOff);
    stats[2 * rib] = m_run;
    stats[2 * rib + 1] = l_tot;
  }
  lds_barrier();
  lds_barrier();
  lds_barrier();
}

// The PV waves' side of one piece: the output rows, written with the LSE (or
// as a partial result).
template <int KV, bool RAGGED>
__device__ void pv_piece(const SplitArgs& a, lds_char* lds, const LaneOffsetsOf<KV>& lo_, const Piece& pc, int v) {
  const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
  const int b = pc.b;
  const int nt = pc.tile1 - pc.tile0;
  const int rg0 = kPVRowGroups * (v / kPVDimParts);   // first row group of this wave
  const int mb0 = kPVBlocks * (v % kPVDimParts);      // first 16-dim block of this wave
  f32x4v_t acc[kPVRowGroups][kPVBlocks];
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++)
#pragma unroll
    for (int mb = 0; mb < kPVBlocks; mb++) acc[r][mb] = f32x4v_t{0.f, 0.f, 0.f, 0.f};
  for (int j = -1; j < nt; j++) {
    lds_barrier();
    if (j >= 0) {
      lds_cchar* vcur = lds + tile_buf(j) * kTileBytes + (fp8_tile(KV) ? 16 : 32) * mb0;
      lds_cchar* pin = lds + kPBufOff + ((j & 1) * kRowGroups + rg0) * 1024;
      lds_cchar* ain = lds + kABufOff + (j & 1) * (kRowsPerBlock * 4) + 16 * i16 + 4 * rg0;
      if constexpr (fp8_tile(KV))
        pv_tile8<MLA_F8_VA>(acc, vcur, lo_, pin, ain);
      else
        pv_tile<MLA_VA>(acc, vcur, lo_, pin, ain);
    }
  }
  lds_barrier();   // every tile is done; the QK waves' row statistics are in LDS

  // ---- epilogue.  The bf16 rows are staged in LDS (the tile buffers) so
  // that every output row leaves as one contiguous 1 KB store of a wave
  // instead of 16 rows x 32 bytes per store.
  constexpr int kStagePitch = kLatentDim * 2 + 16;   // rows 16 bytes apart in the banks
  static_assert(kRowsPerBlock * kStagePitch <= kTileBufs * kTileBytes, "staged rows fit the tile buffers");
  const float* stats = (const float*)(lds + kStatsOff);
#pragma unroll
  for (int r = 0; r < kPVRowGroups; r++) {
    const int rib = 16 * (rg0 + r) + i16;
    const float l_tot = stats[2 * rib + 1];
    const float inv = l_tot > 0.f ? a.out_scale / l_tot : 0.f;
    lds_char* srow = lds + rib * kStagePitch + 32 * mb0 + 8 * g;
#pragma unroll
    for (int mb = 0; mb < kPVBlocks; mb++) {
      const f32x4v_t o = acc[r][mb] * inv;
      u32x2_t wv;
      wv[0] = pack_bf16x2(o[0], o[1]);
      wv[1] = pack_bf16x2(o[2], o[3]);
      *(__attribute__((address_space(3))) u32x2_t*)(srow + 32 * mb) = wv;
    }
  }
  lds_barrier();   // every row is staged
  // Wave v copies out rows kCopyRows*v .. +kCopyRows and their LSEs: lane l
  // carries bytes 16l .. 16l+15 of a row.
  constexpr int kCopyRows = kRowsPerBlock / kPVWaves;
  const QExtent qe = q_extent<RAGGED>(a, b);
  const int R_b = qe.qb * a.H;
  {
    const int rib = kCopyRows * v + i16;
    const int row = pc.rb * kRowsPerBlock + rib;
    if (row < R_b && g == 0 && i16 < kCopyRows) {
      const float m_run = stats[2 * rib], l_tot = stats[2 * rib + 1];
      const float lse_nat = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : kNegInf;
      if (pc.slot < 0) {
        if (a.lse != nullptr) {
          const int jq = row / a.H;
          a.lse[(qe.tok0 + jq) * a.H + (row - jq * a.H)] = lse_nat;
        }
      } else {
        a.part_lse[(int64_t)pc.slot * kRowsPerBlock + rib] = lse_nat;
      }
    }
  }
  for (int rr = 0; rr < kCopyRows; rr++) {
    const int r_in = kCopyRows * v + rr;
    const int r = pc.rb * kRowsPerBlock + r_in;
    if (r >= R_b) break;
    const u32x4_t o = *(__attribute__((address_space(3))) const u32x4_t*)(lds + r_in * kStagePitch + 16 * lane);
    uint16_t* dst;
    if (pc.slot < 0) {
      const int jq = r / a.H;
      dst = a.out + ((qe.tok0 + jq) * a.H + (r - jq * a.H)) * kLatentDim;
    } else {
      dst = a.part_o + ((int64_t)pc.slot * kRowsPerBlock + r_in) * kLatentDim;
    }
    *(u32x4_t*)(dst + 8 * lane) = o;
  }
  lds_barrier();   // every wave has read its rows before the next piece's tile loads land there
}

// Block-wide prefix sums off[0..B] of per-request cost positions pos(b)
// into LDS.  part: NT ints of LDS scratch.
template <int NT, class Pos>
__device__ void build_offsets(int32_t B, const Pos& pos, int32_t* off, int32_t* part) {
  const int tid = threadIdx.x;
  const int per = (B + NT - 1) / NT;
  const int b0 = tid * per, b1 = min(B, b0 + per);
  int32_t sum = 0;
  for (int b = b0; b < b1; b++) sum += pos(b);
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of part[] (Hillis-Steele)
  for (int d = 1; d < NT; d <<= 1) {
    const int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid == 0 ? 0 : part[tid - 1];
  for (int b = b0; b < b1; b++) {
    off[b] = run;
    run += pos(b);
  }
  if (tid == NT - 1) off[B] = part[NT - 1];
  __syncthreads();
}

// The balanced plan's cost-position offsets off[0..B] (all requests).
template <int NT>
__device__ void build_pos_offsets(const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t* off,
                                   int32_t* part) {
  build_offsets<NT>(B, [&](int b) { return positions_of(clamp_len(seq_lens[b], max_seq_len)); }, off, part);
}

// Balanced mode with B <= 64 * kWaveScanPer: the same offsets computed by one
// wave alone, with no LDS and no barrier: lane l sums the cost positions of
// requests l*per .. l*per+per-1, a prefix over the lanes places them, and the
// lane whose range holds position start(g) names the first request of the
// workgroup.  With publish, the wave also writes off[0..B] for the combine.
constexpr int kWaveScanPer = 16;
struct ShareStart {
  int32_t total, b_first, off_first;
};
__device__ ShareStart wave_share_start(const SplitArgs& a, int64_t grp, bool publish) {
  const int lane = threadIdx.x & 63;
  const int per = (a.B + 63) / 64;
  const int b0 = lane * per;
  int32_t u[kWaveScanPer];
  int32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kWaveScanPer; i++) {
    const int b = b0 + i;
    u[i] = i < per && b < a.B ? positions_of(clamp_len(a.seq_lens[b], a.max_seq_len)) : 0;
    sum += u[i];
  }
  int32_t incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  ShareStart r;
  r.total = __builtin_amdgcn_readlane(incl, 63);
  const int64_t v_begin = wg_start(grp, r.total, a.NG);
  int32_t run = incl - sum, found_b = -1, found_off = 0;
#pragma unroll
  for (int i = 0; i < kWaveScanPer; i++) {
    const int b = b0 + i;
    if (i < per && b < a.B) {
      if (publish) a.pos_off_ws[b] = run;
      if (run <= v_begin && v_begin < run + u[i]) {
        found_b = b;
        found_off = run;
      }
    }
    run += u[i];
  }
  if (publish && lane == 63) a.pos_off_ws[a.B] = r.total;
  const uint64_t hit = __ballot(found_b >= 0);
  r.b_first = 0;
  r.off_first = 0;
  if (hit != 0) {
    const int src = __builtin_ctzll(hit);
    r.b_first = __builtin_amdgcn_readlane(found_b, src);
    r.off_first = __builtin_amdgcn_readlane(found_off, src);
  }
  return r;
}

__device__ __forceinline__ int32_t find_request(const int32_t* off, int32_t B, int64_t u) {
  int lo = 0, hi = B - 1;   // largest b with off[b] <= u
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Row blocks of request b of a ragged batch: its class in the class plan.
__device__ __forceinline__ int32_t class_of(const SplitArgs& a, int32_t b) {
  return row_blocks(q_extent<true>(a, b).qb, a.H);
}
// The same where b is wave-uniform (the walks): the result is too, and is
// said so, so that the walk's state stays in scalar registers.
__device__ __forceinline__ int32_t class_of_uniform(const SplitArgs& a, int32_t b) {
  return __builtin_amdgcn_readfirstlane(class_of(a, b));
}

// Where a workgroup's walk starts.  Uniform plan: the first plan group grp
// and its row block rb, with b_first / off_first locating the group's share
// on the line of all requests (cls = 0).  Class plan: group grp of class
// cls (cls_G groups, dense base cls_base), on the line of that class's
// requests only.
struct WalkStart {
  int64_t grp;
  int32_t rb, total, b_first, off_first;
  int32_t cls, cls_G, cls_base;
};

// Class plan of a ragged batch (every thread of the workgroup): the class
// totals, the plan, this workgroup's group, and where its share starts.
// Returns false when the class plan does not apply (the uniform plan
// does); *none is set when the class plan leaves this workgroup without a
// group.  Block 0 publishes the plan, and the first workgroup of each class
// its requests' offsets, for the combine.
__device__ __forceinline__ bool class_start(const SplitArgs& a, char* smem, WalkStart* ws, bool* none) {
  constexpr int NT = kSplitThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* red = (int32_t*)smem;   // [NT / 64][kMaxClasses]
  int32_t t[kMaxClasses + 1];
#pragma unroll
  for (int k = 0; k <= kMaxClasses; k++) t[k] = 0;
  for (int b = tid; b < a.B; b += NT) {
    const int32_t nb = class_of(a, b);
    const int32_t p = positions_of(clamp_len(a.seq_lens[b], a.max_seq_len));
#pragma unroll
    for (int k = 1; k <= kMaxClasses; k++) t[k] += nb == k ? p : 0;
  }
#pragma unroll
  for (int k = 1; k <= kMaxClasses; k++) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t[k] += __shfl_xor(t[k], d);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 1; k <= kMaxClasses; k++) red[wave * kMaxClasses + k - 1] = t[k];
  }
  __syncthreads();
  int32_t T[kMaxClasses + 1];
  T[0] = 0;
#pragma unroll
  for (int k = 1; k <= kMaxClasses; k++) {
    int32_t sum = 0;
    for (int w = 0; w < NT / 64; w++) sum += red[w * kMaxClasses + k - 1];
    T[k] = __builtin_amdgcn_readfirstlane(sum);
  }
  __syncthreads();   // red is overwritten below
  const ClassPlan cp = make_class_plan(T, a.nrb, a.class_S, a.class_C);
  if (blockIdx.x == 0 && tid == 0) {
    a.class_tab[0] = cp.ok ? 1 : 0;
#pragma unroll
    for (int n = 0; n <= kMaxClasses; n++) {
      a.class_tab[kTabT + n] = cp.T[n];
      a.class_tab[kTabG + n] = cp.G[n];
      a.class_tab[kTabBase + n] = cp.base[n];
    }
  }
  *none = false;
  if (!cp.ok) return false;
  int32_t g = 0, rb = 0;
  const int32_t n = class_slot(cp, a.nrb, a.class_C, (int32_t)(blockIdx.x % kXcds), (int32_t)(blockIdx.x / kXcds),
                               &g, &rb);
  if (n == 0) {
    *none = true;
    return true;
  }
  int32_t total = 0, G = 0, base = 0;
#pragma unroll
  for (int k = 1; k <= kMaxClasses; k++) {
    if (n == k) {
      total = cp.T[k];
      G = cp.G[k];
      base = cp.base[k];
    }
  }
  // offsets on the class's line: requests of other classes take no positions
  int32_t* off = (int32_t*)smem;
  build_offsets<NT>(
      a.B, [&](int b) { return class_of(a, b) == n ? positions_of(clamp_len(a.seq_lens[b], a.max_seq_len)) : 0; },
      off, off + kMaxBatch + 1);
  const int64_t v_begin = wg_start(g, total, G);
  ws->grp = g;
  ws->rb = rb;
  ws->total = total;
  ws->b_first = __builtin_amdgcn_readfirstlane(find_request(off, a.B, v_begin));
  ws->off_first = __builtin_amdgcn_readfirstlane(off[ws->b_first]);
  ws->cls = n;
  ws->cls_G = G;
  ws->cls_base = base;
  if (g == 0 && rb == 0)
    for (int b = tid; b < a.B; b += NT)
      if (class_of(a, b) == n) a.pos_off_ws[b] = off[b];
  __syncthreads();   // every wave has read the offsets before tiles land there
  return true;
}

// Every wave of a workgroup walks the same pieces: the loader waves fill the
// tile ring, the compute waves consume it; their barriers pair up one to one.
// ws.grp: the first plan group of the launched group (forced mode: its only one).
template <bool RAGGED, class PieceFn>
__device__ __forceinline__ void for_each_piece(const SplitArgs& a, const WalkStart& ws, PieceFn&& fn_all) {
  // A ragged batch's request with fewer query rows than this row block's
  // first has nothing here: every wave of the workgroup skips the piece.
  auto fn = [&](const Piece& pc) {
    if (RAGGED && pc.rb * kRowsPerBlock >= q_extent<RAGGED>(a, pc.b).qb * a.H) return;
    fn_all(pc);
  };
  auto units = [&](int32_t b) -> int32_t { return units_of(clamp_len(a.seq_lens[b], a.max_seq_len)); };
  if (a.num_splits > 0) {
    const int32_t b = (int32_t)(ws.grp / a.num_splits);
    Piece pc;
    if (forced_piece(ws.grp, ws.rb, a.nrb, a.num_splits, units(b), &pc)) fn(pc);
    return;
  }
  // Balanced: the uniform plan's groups grp .. grp+vg_per-1 on the line of
  // all requests, or the class plan's group grp on the line of its class
  // (after request b comes the next request of the class).  One walk for
  // both, so that the piece body is emitted once more only.
  const bool by_class = RAGGED && ws.cls > 0;
  auto succ = [&](int32_t b) {
    if (!by_class) return b + 1;
    for (b++; b < a.B && class_of_uniform(a, b) != ws.cls; b++) {
    }
    return b;
  };
  const int64_t G = by_class ? (int64_t)ws.cls_G : a.NG;
  const int64_t g1 = by_class ? ws.grp + 1 : min(ws.grp + a.vg_per, a.NG);
  folded_balanced_pieces(ws.grp, g1, G, ws.rb, by_class ? ws.cls : a.nrb, ws.total, ws.b_first, ws.off_first, units,
                         [&](const Piece& pc, int64_t) { fn(pc); }, succ, by_class ? (int64_t)ws.cls_base : 0);
}

// RAGGED: per-request query lengths from a.qo_indptr (a separate
// instantiation, so the uniform batch's code is what it was without them).
template <int KV, bool RAGGED>
__global__ __launch_bounds__(kSplitThreads, 1) void mla_split_kernel(SplitArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  lds_char* tiles = (lds_char*)smem;
  int64_t lgrp;
  WalkStart ws;
  group_of_block(blockIdx.x, a.nrb, &lgrp, &ws.rb);
  ws.grp = lgrp * a.vg_per;   // the first plan group this workgroup walks
  ws.total = ws.b_first = ws.off_first = 0;
  ws.cls = ws.cls_G = ws.cls_base = 0;
  // A ragged batch in balanced mode: the row-block class plan when it applies.
  bool planned = false;
  if constexpr (RAGGED) {
    if (a.class_plan) {
      bool none = false;
      planned = class_start(a, smem, &ws, &none);
      if (none) return;
    }
  }
  // Balanced mode: the cost-position offsets of all requests, of which this workgroup
  // keeps only where its share starts; block 0 publishes them for the
  // combine.  Up to 64 * kWaveScanPer requests every wave computes them on its
  // own; larger batches build them block-wide in the tile buffers' LDS
  // (before any tile is loaded).  Every LDS byte a wave reads later is written
  // first in the pipeline (tiles by loads or zero fills), so nothing is
  // cleared here.
  if (!planned && a.num_splits == 0) {
    if (a.B <= 64 * kWaveScanPer) {
      const ShareStart st = wave_share_start(a, ws.grp, blockIdx.x == 0 && threadIdx.x < 64);
      ws.total = __builtin_amdgcn_readfirstlane(st.total);
      ws.b_first = __builtin_amdgcn_readfirstlane(st.b_first);
      ws.off_first = __builtin_amdgcn_readfirstlane(st.off_first);
    } else {
      int32_t* off = (int32_t*)smem;
      build_pos_offsets<kSplitThreads>(a.seq_lens, a.B, a.max_seq_len, off, off + kMaxBatch + 1);
      if (blockIdx.x == 0)
        for (int b = threadIdx.x; b <= a.B; b += kSplitThreads) a.pos_off_ws[b] = off[b];
      ws.total = __builtin_amdgcn_readfirstlane(off[a.B]);
      const int64_t v_begin = wg_start(ws.grp, ws.total, a.NG);
      if (v_begin < ws.total) {
        ws.b_first = __builtin_amdgcn_readfirstlane(find_request(off, a.B, v_begin));
        ws.off_first = __builtin_amdgcn_readfirstlane(off[ws.b_first]);
      }
      __syncthreads();   // every wave has read the offsets before tiles land there
    }
  }
  if (!planned && lgrp >= a.NGL) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= kLoaderWave0) {
    if (MLA_PRIO_LD) __builtin_amdgcn_s_setprio(MLA_PRIO_LD);
    const int lw = wave - kLoaderWave0;
    Stage<KV> stg;
    stg.init(lw);
    for_each_piece<RAGGED>(a, ws, [&](const Piece& pc) { load_piece<KV>(a, tiles, stg, pc, lw); });
  } else if (wave >= kPVWave0) {
    LaneOffsetsOf<KV> lo_;
    lo_.init();
    for_each_piece<RAGGED>(a, ws, [&](const Piece& pc) { pv_piece<KV, RAGGED>(a, tiles, lo_, pc, wave - kPVWave0); });
  } else {
    if (MLA_PRIO_QK) __builtin_amdgcn_s_setprio(MLA_PRIO_QK);
    LaneOffsetsOf<KV> lo_;
    lo_.init();
    for_each_piece<RAGGED>(a, ws, [&](const Piece& pc) { qk_piece<KV, RAGGED>(a, tiles, lo_, pc, wave - kQKWave0); });
  }
}

// ---- combine: merge the partial results of each split row block by LSE
// Lanes load the pieces' LSEs in parallel, then the 512-wide bf16 partials
// are summed with weights exp(lse_s - LSE).  kWaves = 1: one wave per query
// row, four rows per workgroup (few pieces per row).  kWaves = 4: the four
// waves of a workgroup share one row, each summing every fourth group of
// eight pieces, and add up through LDS -- four times the loads in flight per
// row when rows have many pieces (long requests split over many workgroups).
template <int kWaves>
struct CombineShape {
  static constexpr int kRowsPerWg = kWaves == 1 ? kThreads / 64 : 1;
};

// One row per wave: at most 64 VGPRs, eight workgroups per CU, so the grid of
// a full-size decode (up to 2048 workgroups) runs in one round.  One row per
// workgroup: fewer, wider workgroups, up to 128 VGPRs.
//
// kByGroup (balanced plans with B <= kByGroupMaxB, when the groups are fewer
// than the requests or the batch is ragged): the grid covers the split
// kernel's workgroups instead of the requests, NG * nrb * 16 workgroups.  A
// split request's last tile lies in the share of exactly one group g1, and
// that share starts inside the request (its first tile lies in an earlier
// group), so the request holding position start(g) is the only one the
// workgroups of group g may have to merge: they merge it when it is split
// and ends in g's share.  Unsplit requests, and row blocks a short request
// of a ragged batch does not have, then cost no workgroup.  Under a
// row-block class plan the same holds on each class's own line of positions
// and groups.
constexpr int kByGroupMaxB = 4 * kThreads;   // offsets found with one load round per thread
template <int kWaves, bool kByGroup>
__global__ __launch_bounds__(kThreads, kWaves == 1 ? 8 : 4) void mla_combine_kernel(CombineArgs a) {
  static_assert(kWaves == 1 || kWaves == kThreads / 64, "one wave per row, or the whole workgroup");
  static_assert(!kByGroup || kWaves == 1, "the group grid uses one wave per row");
  constexpr int kRowsPerWg = CombineShape<kWaves>::kRowsPerWg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ws = kWaves == 1 ? 0 : wave;       // this wave's share of the pieces
  const int chunks = kRowsPerBlock / kRowsPerWg;
  const int64_t blk = blockIdx.x / chunks;     // b * nrb + rb, or g * nrb + rb with kByGroup
  const int row_in_blk = (int)(blockIdx.x - blk * chunks) * kRowsPerWg + (kWaves == 1 ? wave : 0);
  int32_t b, rb;
  int64_t g0, g1, first_pos = 0, total = 0;
  int64_t NGc = a.NG, slot_base = 0;   // the plan's groups (of the request's class) and its first slot
  int32_t nrbc = a.nrb;                // workgroups per group
  if constexpr (kByGroup) {
    // blk is a split workgroup's number: g * nrb + rb in the uniform plan, or
    // the dense number of a workgroup of the row-block class plan (class n's
    // groups take numbers base_n .. base_n + G_n * n - 1, n per group).
    // Every wave of the workgroup takes part before any returns.
    int64_t g = 0;
    int32_t n = 0;   // class of a class plan's group; 0: the uniform plan
    if (a.class_tab != nullptr && a.class_tab[0] == 1) {
#pragma unroll
      for (int k = 1; k <= kMaxClasses; k++) {
        const int64_t base = a.class_tab[kTabBase + k], Gk = a.class_tab[kTabG + k];
        if (blk >= base && blk < base + Gk * k) {
          n = k;
          g = (blk - base) / k;
          rb = (int32_t)(blk - base - g * k);
          total = a.class_tab[kTabT + k];
          NGc = Gk;
          nrbc = k;
          slot_base = 2 * base;
        }
      }
      if (n == 0) return;   // a slot the class plan leaves empty
    } else {
      g = blk / a.nrb;
      rb = (int32_t)(blk - g * a.nrb);
      total = a.pos_off_ws[a.B];
    }
    const int64_t v = wg_start(g, total, NGc);
    __shared__ int32_t found;
    if (threadIdx.x == 0) found = -1;
    __syncthreads();
    // the request holding position v on the group's line: one request does
    // (on a class's line, only that class's requests take positions)
#pragma unroll
    for (int k = 0; k < kByGroupMaxB / kThreads; k++) {
      const int bb = (int)threadIdx.x + kThreads * k;
      if (bb >= a.B) continue;
      const int64_t o = a.pos_off_ws[bb];
      if (n == 0) {
        if (o <= v && v < a.pos_off_ws[bb + 1]) found = bb;
      } else if (row_blocks(q_extent<true>(a, bb).qb, a.H) == n) {
        if (o <= v && v < o + positions_of(clamp_len(a.seq_lens[bb], a.max_seq_len))) found = bb;
      }
    }
    __syncthreads();
    b = found;
    if (b < 0) return;   // an empty share at the end
    first_pos = a.pos_off_ws[b];
    const int32_t U = n == 0 ? a.pos_off_ws[b + 1] - (int32_t)first_pos - kPieceCost
                             : units_of(clamp_len(a.seq_lens[b], a.max_seq_len));
    g0 = first_group(first_pos, total, NGc);
    g1 = last_group(first_pos, U, total, NGc);
    if (g1 != g || g0 == g1) return;   // not a split request that ends in this share
  } else {
    b = (int32_t)(blk / a.nrb);
    rb = (int32_t)(blk - (int64_t)b * a.nrb);
  }
  const int row = rb * kRowsPerBlock + row_in_blk;
  const QExtent qe = q_extent<true>(a, b);
  if (row >= qe.qb * a.H) return;
  // the pieces of this row block: groups [g0, g1]
  if constexpr (kByGroup) {
    // g0, g1, first_pos and total were found above
  } else if (a.num_splits > 0) {
    const int32_t U = units_of(clamp_len(a.seq_lens[b], a.max_seq_len));
    const int32_t Sp = a.num_splits < U ? a.num_splits : U;
    if (Sp <= 1) return;
    g0 = (int64_t)b * a.num_splits;
    g1 = g0 + Sp - 1;
  } else if (a.class_tab != nullptr && a.class_tab[0] == 1) {
    // the row-block class plan of a ragged batch: the request's class n is
    // its row-block count, its offset is on the line of that class
    const int32_t n = row_blocks(qe.qb, a.H);
    total = a.class_tab[kTabT + n];
    NGc = a.class_tab[kTabG + n];
    nrbc = n;
    slot_base = 2 * (int64_t)a.class_tab[kTabBase + n];
    first_pos = a.pos_off_ws[b];
    const int32_t U = units_of(clamp_len(a.seq_lens[b], a.max_seq_len));
    g0 = first_group(first_pos, total, NGc);
    g1 = last_group(first_pos, U, total, NGc);
    if (g0 == g1) return;
  } else {
    // the request's cost positions give its tile count too (positions_of),
    // so the three offsets load together and seq_lens is not read
    total = a.pos_off_ws[a.B];
    first_pos = a.pos_off_ws[b];
    const int32_t U = a.pos_off_ws[b + 1] - (int32_t)first_pos - kPieceCost;
    g0 = first_group(first_pos, total, a.NG);
    g1 = last_group(first_pos, U, total, a.NG);
    if (g0 == g1) return;
  }
  auto slot_of = [&](int64_t g) -> int64_t {
    if (a.num_splits > 0) return g * a.nrb + rb;
    if (wg_start(g, total, NGc) == wg_start(g + 1, total, NGc)) return -1;   // an empty group
    return slot_base + balanced_slot(g, g0, first_pos, total, NGc, rb, nrbc);
  };
  const int64_t n = g1 - g0 + 1;
  // Lane l handles piece c0 + l of each chunk of 64: its slot, its LSE and
  // its weight exp(lse - M).  Partial rows are then loaded eight at a time
  // (lane l owns dims 8l..8l+7) so that their latencies overlap; a missing
  // piece reads slot 0 with weight 0 and is dropped by a select (that slot
  // may hold anything).  With at most 64 pieces the first eight rows are
  // loaded together with the LSEs, before the maximum is known.
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  auto load8 = [&](int32_t s32, int j, u32x4_t (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int32_t sk = __builtin_amdgcn_readlane(s32, min(j + k, 63));
      v[k] = *(const u32x4_t*)(a.part_o + ((int64_t)sk * kRowsPerBlock + row_in_blk) * kLatentDim + 8 * lane);
    }
  };
  auto accum8 = [&](float w, int j, int cnt, const u32x4_t (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const float wk = j + k < cnt ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int32_t, w),
                                                                                          min(j + k, 63)))
                                   : 0.f;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float lo = wk * __builtin_bit_cast(float, v[k][e] << 16);
        const float hi = wk * __builtin_bit_cast(float, v[k][e] & 0xFFFF0000u);
        o[2 * e] += wk != 0.f ? lo : 0.f;
        o[2 * e + 1] += wk != 0.f ? hi : 0.f;
      }
    }
  };
  float M = kNegInf;
  if (n <= 64) {
    const int64_t s = lane < n ? slot_of(g0 + lane) : -1;
    const int32_t s32 = s >= 0 ? (int32_t)s : 0;
    const float ls = s >= 0 ? a.part_lse[s * kRowsPerBlock + row_in_blk] : kNegInf;
    u32x4_t v[8];
    load8(s32, 8 * ws, v);
    M = ls;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
    if (M != kNegInf) {
      const float w = ls == kNegInf ? 0.f : __expf(ls - M);
      den = w;
      const int cnt = (int)n;
      if (8 * ws < cnt) accum8(w, 8 * ws, cnt, v);
      for (int j = 8 * ws + 8 * kWaves; j < cnt; j += 8 * kWaves) {
        load8(s32, j, v);
        accum8(w, j, cnt, v);
      }
    }
  } else {
    // pass 1: maximum LSE over the pieces
    for (int64_t c0 = 0; c0 < n; c0 += 64) {
      const int64_t s = c0 + lane < n ? slot_of(g0 + c0 + lane) : -1;
      const float ls = s >= 0 ? a.part_lse[s * kRowsPerBlock + row_in_blk] : kNegInf;
      M = fmaxf(M, ls);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
    // pass 2: weighted sum
    if (M != kNegInf) {
      for (int64_t c0 = 0; c0 < n; c0 += 64) {
        const int64_t s = c0 + lane < n ? slot_of(g0 + c0 + lane) : -1;
        const int32_t s32 = s >= 0 ? (int32_t)s : 0;
        const float ls = s >= 0 ? a.part_lse[s * kRowsPerBlock + row_in_blk] : kNegInf;
        const float w = ls == kNegInf ? 0.f : __expf(ls - M);
        den += w;
        const int cnt = (int)min((int64_t)64, n - c0);
        for (int j = 8 * ws; j < cnt; j += 8 * kWaves) {
          u32x4_t v[8];
          load8(s32, j, v);
          accum8(w, j, cnt, v);
        }
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d);
  if constexpr (kWaves > 1) {
    // every wave holds the full denominator; wave 0 adds the others' sums
    __shared__ float red[kWaves - 1][kLatentDim];
    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < 8; e++) red[wave - 1][8 * lane + e] = o[e];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int r = 0; r < kWaves - 1; r++)
#pragma unroll
      for (int e = 0; e < 8; e++) o[e] += red[r][8 * lane + e];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int32_t jq = row / a.H, h = row - jq * a.H;
  const int64_t orow = (qe.tok0 + jq) * a.H + h;
  u32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; e++)
    w[e] = pack_bf16x2(o[2 * e] * inv, o[2 * e + 1] * inv);
  *(u32x4_t*)(a.out + orow * kLatentDim + 8 * lane) = w;
  if (a.lse != nullptr && lane == 0) a.lse[orow] = den > 0.f ? M + __logf(den) : kNegInf;
}

// ---- debug: gather one request's stored rows through the block table
__global__ __launch_bounds__(kThreads) void mla_gather_kernel(const void* pool, const int32_t* bt,
                                                               const int32_t* seq_lens, int32_t W, int32_t P,
                                                               int32_t N, int32_t max_seq_len, int32_t b,
                                                               int32_t elem_bytes, char* dst) {
  const int32_t L = clamp_len(seq_lens[b], max_seq_len);
  const int32_t row_bytes = kRowDim * elem_bytes;
  const int32_t chunks_per_row = row_bytes / 16;
  const int64_t n = (int64_t)L * chunks_per_row;
  for (int64_t ci = (int64_t)blockIdx.x * kThreads + threadIdx.x; ci < n; ci += (int64_t)gridDim.x * kThreads) {
    const int32_t t = (int32_t)(ci / chunks_per_row), c = (int32_t)(ci - (int64_t)t * chunks_per_row);
    const char* src = token_row(pool, bt, W, P, N, b, t, elem_bytes);
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (src != nullptr) x = *(const u32x4_t*)(src + c * 16);
    *(u32x4_t*)(dst + (int64_t)t * row_bytes + c * 16) = x;
  }
}

// ---- debug: the plan as the decode kernel computes it
// (launched as the decode is: vg_per plan groups per launched group)
__global__ __launch_bounds__(kThreads) void mla_plan_kernel(const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                                             int32_t nrb, int32_t num_splits, int64_t NG,
                                                             int32_t vg_per, int64_t NGL, int32_t max_per_wg,
                                                             int32_t* pieces, int32_t* counts) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int32_t* off = (int32_t*)smem;
  int64_t lgrp;
  int32_t rb;
  group_of_block(blockIdx.x, nrb, &lgrp, &rb);
  const int64_t grp = lgrp * vg_per;
  // Pieces are counted per plan group: cur is the group being counted (its
  // n pieces so far), every group below it already has its count written.
  int64_t cur = grp;
  int32_t n = 0;
  auto close_until = [&](int64_t g) {   // write the counts of groups cur .. g-1, then count g
    for (; cur < g; cur++, n = 0)
      if (threadIdx.x == 0) counts[cur * nrb + rb] = n;
  };
  auto emit = [&](const Piece& pc, int64_t g) {
    close_until(g);
    if (threadIdx.x == 0 && n < max_per_wg) {
      const int64_t wg = g * nrb + rb;   // logical workgroup index of the plan
      int32_t* o = pieces + (wg * max_per_wg + n) * 6;
      o[0] = (int32_t)wg; o[1] = pc.b; o[2] = pc.rb; o[3] = pc.tile0; o[4] = pc.tile1; o[5] = pc.slot;
    }
    n++;
  };
  __shared__ int32_t part[kThreads];
  if (num_splits == 0) build_pos_offsets<kThreads>(seq_lens, B, max_seq_len, off, part);
  if (lgrp >= NGL) return;
  const int64_t g1 = min(grp + vg_per, NG);
  if (num_splits > 0) {
    const int32_t b = (int32_t)(grp / num_splits);
    Piece pc;
    if (forced_piece(grp, rb, nrb, num_splits, units_of(clamp_len(seq_lens[b], max_seq_len)), &pc)) emit(pc, grp);
  } else {
    const int32_t total = off[B];
    const int64_t v_begin = wg_start(grp, total, NG);
    const int32_t b_first = v_begin < total ? find_request(off, B, v_begin) : 0;
    auto units = [&](int32_t b) -> int32_t { return units_of(clamp_len(seq_lens[b], max_seq_len)); };
    folded_balanced_pieces(grp, g1, NG, rb, nrb, total, b_first, off[b_first], units, emit);
  }
  close_until(g1);
}

}  // namespace mla

// ---- launchers called by the host API
extern "C" {

size_t mla_split_lds_bytes(int32_t B, int32_t num_splits) {
  (void)B;
  (void)num_splits;
  static_assert((mla::kMaxBatch + 1) * 4 <= mla::kTileBufs * mla::kTileBytes,
                "the planning scan keeps B+1 offsets in the tile buffers");
  return (size_t)mla::kSplitLdsBytes;
}

hipError_t mla_launch_split(const mla::SplitArgs* a, int kv_mode, hipStream_t stream) {
  if (kv_mode < 0 || kv_mode > 2) return hipErrorInvalidValue;
  const size_t lds = mla_split_lds_bytes(a->B, a->num_splits);
  const bool ragged = a->qo_indptr != nullptr;
  const int v = kv_mode + (ragged ? 3 : 0);
  void (*const fns[6])(mla::SplitArgs) = {mla::mla_split_kernel<0, false>, mla::mla_split_kernel<1, false>,
                                          mla::mla_split_kernel<2, false>, mla::mla_split_kernel<0, true>,
                                          mla::mla_split_kernel<1, true>,  mla::mla_split_kernel<2, true>};
  static bool attr_set[6] = {false, false, false, false, false, false};
  if (!attr_set[v]) {
    // dynamic LDS above 64 KB: raise the per-kernel limit once to what the
    // kernel uses (static and dynamic LDS together stay within the 160 KB a
    // gfx950 workgroup may have)
    hipError_t e = hipFuncSetAttribute((const void*)fns[v], hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)mla::kSplitLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[v] = true;
  }
  const unsigned grid = (unsigned)mla::launch_grid(a->NGL, a->nrb);
  hipLaunchKernelGGL(fns[v], dim3(grid), dim3(mla::kSplitThreads), lds, stream, *a);
  return hipGetLastError();
}

hipError_t mla_launch_combine(const mla::CombineArgs* a, hipStream_t stream) {
  // a workgroup per row when requests are split into many pieces on average
  const bool wide = a->num_splits > 0 ? a->num_splits >= 8 : a->NG >= 4 * (int64_t)a->B;
  // the grid over the split workgroups when the groups are fewer than the
  // requests, or when the split kernel may plan in row-block classes (its
  // workgroups then take at most NG * nrb dense numbers)
  const bool by_group = !wide && a->num_splits == 0 && a->B <= mla::kByGroupMaxB &&
                        (a->NG < a->B || a->class_tab != nullptr);
  const int rows_per_wg = wide ? mla::CombineShape<4>::kRowsPerWg : mla::CombineShape<1>::kRowsPerWg;
  const int64_t units = by_group ? a->NG : (int64_t)a->B;
  const int64_t blocks = units * a->nrb * (mla::kRowsPerBlock / rows_per_wg);
  if (blocks == 0) return hipSuccess;
  if (wide)
    hipLaunchKernelGGL((mla::mla_combine_kernel<4, false>), dim3((unsigned)blocks), dim3(mla::kThreads), 0, stream,
                       *a);
  else if (by_group)
    hipLaunchKernelGGL((mla::mla_combine_kernel<1, true>), dim3((unsigned)blocks), dim3(mla::kThreads), 0, stream,
                       *a);
  else
    hipLaunchKernelGGL((mla::mla_combine_kernel<1, false>), dim3((unsigned)blocks), dim3(mla::kThreads), 0, stream,
                       *a);
  return hipGetLastError();
}

hipError_t mla_launch_gather(const void* pool, const int32_t* bt, const int32_t* seq_lens, int32_t W, int32_t P,
                             int32_t N, int32_t max_seq_len, int32_t b, int32_t elem_bytes, void* dst,
                             hipStream_t stream) {
  const int64_t chunks = (int64_t)max_seq_len * (mla::kRowDim * elem_bytes / 16);
  int64_t blocks = (chunks + mla::kThreads - 1) / mla::kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(mla::mla_gather_kernel, dim3((unsigned)blocks), dim3(mla::kThreads), 0, stream, pool, bt,
                     seq_lens, W, P, N, max_seq_len, b, elem_bytes, (char*)dst);
  return hipGetLastError();
}

hipError_t mla_launch_plan(const int32_t* seq_lens, int32_t B, int32_t max_seq_len, int32_t nrb, int32_t num_splits,
                           int64_t NG, int32_t vg_per, int32_t max_per_wg, int32_t* pieces, int32_t* counts,
                           hipStream_t stream) {
  const size_t lds = num_splits > 0 ? 16 : ((size_t)B + 1) * 4;
  const int64_t NGL = mla::launched_groups(NG, vg_per);
  hipLaunchKernelGGL(mla::mla_plan_kernel, dim3((unsigned)mla::launch_grid(NGL, nrb)), dim3(mla::kThreads), lds,
                     stream, seq_lens, B, max_seq_len, nrb, num_splits, NG, vg_per, NGL, max_per_wg, pieces, counts);
  return hipGetLastError();
}

}  // extern "C"
