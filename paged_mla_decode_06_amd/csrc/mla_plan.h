// mla_plan.h -- split-KV work planning of libmla, shared by the host mirror
// and the device kernels so that both produce the same plan.
//
// Work unit: one 32-token tile of one request for one block of 64 query
// rows (rows are (j, h) pairs, j-major, j < q_len, h < H).  A request with L
// tokens has U = max(1, ceil(L/32)) units per row block (a request with no
// token still gets one unit, which writes out = 0 and lse = -inf).  Units are
// ordered (request, row block, tile).
//
// Balanced mode (num_splits == 0), in the spirit of the tile-scheduler
// metadata the pages obtain from get_mla_metadata ("tokenspeed flashmla.py",
// FlashMLABackend._init_decode_metadata): G workgroups each take a
// contiguous, equal share [start(g), start(g+1)) of all units, with
// start(g) = floor(g*total/G).  A share is cut into pieces at row-block
// boundaries.  A piece that covers its whole row block writes the output;
// any other piece writes a partial result to slot 2g (the workgroup's first
// piece) or 2g+1 (its last piece), and the combine merges the partials of a
// row block from the workgroups that touch it.
//
// Forced mode (num_splits = S > 0): each row block's U tiles are cut into
// S' = min(S, U) near-equal pieces, one workgroup each; workgroup
// g = (b*nrb + rb)*S + s, slot g when S' > 1.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ inline
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int kRowDim = 576;       // latent 512 + rope 64
constexpr int kLatentDim = 512;
constexpr int kTile = 32;          // tokens per KV tile
constexpr int kRowsPerBlock = 64;  // query rows per workgroup (4 waves x 16)
constexpr int kMaxBatch = 16384;

MLA_HD int32_t clamp_len(int32_t L, int32_t max_seq_len) {
  return L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
}
MLA_HD int32_t units_of(int32_t L) {
  int32_t u = (L + kTile - 1) / kTile;
  return u < 1 ? 1 : u;
}
MLA_HD int32_t row_blocks(int32_t q_len, int32_t heads) {
  return (q_len * heads + kRowsPerBlock - 1) / kRowsPerBlock;
}
// First unit of workgroup g in balanced mode.
MLA_HD int64_t wg_start(int64_t g, int64_t total, int64_t G) { return g * total / G; }
// The workgroup whose share holds unit u (0 <= u < total): the largest g with start(g) <= u.
MLA_HD int64_t wg_of_unit(int64_t u, int64_t total, int64_t G) { return ((u + 1) * G - 1) / total; }

// Workgroups the decode launches.  ub_units = B * nrb * units_of(max_seq_len)
// bounds the true unit count, so a balanced grid never exceeds the work.
MLA_HD int64_t grid_size(int32_t B, int32_t nrb, int32_t max_seq_len, int32_t num_splits, int32_t target) {
  if (B <= 0) return 0;
  if (num_splits > 0) return (int64_t)B * nrb * num_splits;
  int64_t ub = (int64_t)B * nrb * units_of(max_seq_len);
  int64_t t = target < 1 ? 1 : target;
  return ub < t ? ub : t;
}
// Partial-result slots the workspace holds.
MLA_HD int64_t slot_count(int64_t grid, int32_t num_splits) { return num_splits > 0 ? grid : 2 * grid; }

struct Piece {
  int32_t b, rb, tile0, tile1, slot;
};

// Pieces of balanced-mode workgroup g.  unit_off(b) = nrb * sum_{b' < b} U_b'
// for b in [0, B]; `find(u)` returns the request b with unit_off(b) <= u <
// unit_off(b+1).  fn(Piece) is called for each piece in order.
template <class Off, class Find, class Fn>
MLA_HD void balanced_pieces(int64_t g, int64_t G, int32_t nrb, const Off& unit_off, const Find& find, int32_t B,
                            Fn&& fn) {
  const int64_t total = unit_off(B);
  const int64_t u_begin = wg_start(g, total, G), u_end = wg_start(g + 1, total, G);
  if (u_begin >= u_end) return;
  int32_t b = find(u_begin);
  int64_t u = u_begin;
  while (u < u_end) {
    const int64_t ob = unit_off(b);
    const int32_t U = (int32_t)((unit_off(b + 1) - ob) / nrb);
    const int64_t rel = u - ob;
    const int32_t rb = (int32_t)(rel / U);
    const int32_t tile0 = (int32_t)(rel - (int64_t)rb * U);
    const int64_t blk_end = ob + (int64_t)(rb + 1) * U;
    const int64_t pe = blk_end < u_end ? blk_end : u_end;
    const int32_t tile1 = tile0 + (int32_t)(pe - u);
    const bool whole = tile0 == 0 && tile1 == U;
    Piece pc;
    pc.b = b;
    pc.rb = rb;
    pc.tile0 = tile0;
    pc.tile1 = tile1;
    pc.slot = whole ? -1 : (int32_t)(2 * g + (u == u_begin ? 0 : 1));
    fn(pc);
    u = pe;
    if (u == unit_off(b + 1)) b++;
  }
}

// The single piece of forced-mode workgroup g, or false if g has none.
MLA_HD bool forced_piece(int64_t g, int32_t nrb, int32_t S, int32_t U_of_b_known, int32_t b, Piece* pc) {
  const int64_t blk = g / S;
  const int32_t s = (int32_t)(g - blk * S);
  const int32_t U = U_of_b_known;
  const int32_t Sp = S < U ? S : U;
  if (s >= Sp) return false;
  pc->b = b;
  pc->rb = (int32_t)(blk - (int64_t)b * nrb);
  pc->tile0 = (int32_t)((int64_t)s * U / Sp);
  pc->tile1 = (int32_t)((int64_t)(s + 1) * U / Sp);
  pc->slot = Sp > 1 ? (int32_t)g : -1;
  return true;
}

}  // namespace mla
