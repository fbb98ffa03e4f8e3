// mla_plan.h -- split-KV work planning of libmla, shared by the host mirror
// and the device kernels so that both produce the same plan.
//
// Query rows of a request are (j, h) pairs, row = j*H + h, cut into row
// blocks of 64; a request has nrb = ceil(q_len*H / 64) of them.  One
// workgroup handles one row block.  The nrb workgroups of a request form a
// group: they walk the same 32-token KV tiles at the same time, and the
// launch order puts them on the same XCD (workgroup i runs on XCD i mod 8),
// so the second read of each tile is served by that XCD's L2.
//
// Work unit: one 32-token tile of one request.  A request with L tokens has
// U = max(1, ceil(L/32)) units (a request with no token still gets one unit,
// which writes out = 0 and lse = -inf).  Units are ordered (request, tile).
//
// Balanced mode (num_splits == 0), in the spirit of the tile-scheduler
// metadata the pages obtain from get_mla_metadata ("tokenspeed flashmla.py",
// FlashMLABackend._init_decode_metadata), with a fixed start-up cost per
// piece.  The requests are laid out on a line of cost positions: request b
// takes kPieceCost + U_b of them, its start-up cost first (the latency of
// its first tiles, the query load, the epilogue), then one per tile.  NG
// groups each take a contiguous, equal share [start(g), start(g+1)) of all
// positions, start(g) = floor(g*total/NG); the tiles of each request that
// fall in a share form that group's piece of the request, so a group that
// starts more pieces gets fewer tiles.  A piece that covers a whole request
// writes the output; any other piece writes a partial result to slot 2*wg
// (the group's first piece) or 2*wg+1 (its last piece), wg = g*nrb + rb, and
// the combine merges the partials of a row block.
//
// Forced mode (num_splits = S > 0): group g = b*S + s takes piece s of the
// S' = min(S, U) near-equal pieces of request b; slot wg when S' > 1.
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
constexpr int kMaxBatch = 8192;    // the planning scan keeps (B+1) offsets in the tile buffers' LDS
constexpr int kXcds = 8;           // workgroup i is dispatched to XCD i mod 8

MLA_HD int32_t clamp_len(int32_t L, int32_t max_seq_len) {
  return L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
}
MLA_HD int32_t units_of(int32_t L) {
  int32_t u = (L + kTile - 1) / kTile;
  return u < 1 ? 1 : u;
}
// Balanced-mode start-up cost of a piece, in tiles of the steady stream.
#ifndef MLA_PIECE_COST
#define MLA_PIECE_COST 8
#endif
constexpr int kPieceCost = MLA_PIECE_COST;
// Cost positions request b takes in balanced mode.
MLA_HD int32_t positions_of(int32_t L) { return kPieceCost + units_of(L); }
MLA_HD int32_t row_blocks(int32_t q_len, int32_t heads) {
  return (q_len * heads + kRowsPerBlock - 1) / kRowsPerBlock;
}
// First cost position of group g in balanced mode (total positions in all).
MLA_HD int64_t wg_start(int64_t g, int64_t total, int64_t G) { return g * total / G; }
// The group whose share holds position v (0 <= v < total): the largest g with start(g) <= v.
MLA_HD int64_t wg_of_pos(int64_t v, int64_t total, int64_t G) { return ((v + 1) * G - 1) / total; }

// Groups of the plan, never more than B * units_of(max_seq_len) (which
// bounds the true unit count).  Balanced with at_least (a minimum number of
// work units): at least target workgroups.  Balanced otherwise (target =
// the CU count): as many groups as the CUs hold in one round with whole
// groups on each XCD (a group's workgroups share an XCD, and an XCD has
// target / 8 CUs), so that no workgroup waits for a second round.
MLA_HD int64_t group_count(int32_t B, int32_t nrb, int32_t max_seq_len, int32_t num_splits, int32_t target,
                           bool at_least) {
  if (B <= 0) return 0;
  if (num_splits > 0) return (int64_t)B * num_splits;
  const int64_t ub = (int64_t)B * units_of(max_seq_len);
  if (target < 1) target = 1;
  int64_t t;
  if (at_least)
    t = ((int64_t)target + nrb - 1) / nrb;
  else if (target / kXcds >= nrb)
    t = (int64_t)kXcds * ((target / kXcds) / nrb);
  else
    t = target / nrb > 0 ? target / nrb : 1;
  return ub < t ? ub : t;
}
// Workgroups launched: groups padded to a multiple of the XCD count, nrb each.
MLA_HD int64_t launch_grid(int64_t groups, int32_t nrb) {
  return (groups + kXcds - 1) / kXcds * kXcds * nrb;
}
// Partial-result slots the workspace holds.
MLA_HD int64_t slot_count(int64_t groups, int32_t nrb, int32_t num_splits) {
  return (num_splits > 0 ? 1 : 2) * groups * nrb;
}
// Launch index -> (group, row block): all nrb members of a group share an XCD.
MLA_HD void group_of_block(int64_t blk, int32_t nrb, int64_t* group, int32_t* rb) {
  const int64_t xcd = blk % kXcds, q = blk / kXcds;
  *rb = (int32_t)(q % nrb);
  *group = (q / nrb) * kXcds + xcd;
}

struct Piece {
  int32_t b, rb, tile0, tile1, slot;
};

// Pieces of balanced-mode group g for row block rb, one at a time.  total is
// the number of cost positions of all requests; b_first is the request
// holding the group's first position start(g) (off(b_first) <= start(g) <
// off(b_first + 1), off(b) = sum of positions_of(L_b') for b' < b) and
// off_first = off(b_first).  The requests of the share are walked in order,
// so no table of offsets is needed; next(units, &pc) yields the following
// piece (units(b) returns U_b) or false after the last.  A share that ends
// inside a request's start-up positions holds none of its tiles.  Once next()
// has returned false, b and ob locate start(g+1) the same way.
struct BalancedWalk {
  int64_t v, v_end, ob, wg;
  int32_t b, rb;
  bool first;
  MLA_HD void init(int64_t g, int64_t G, int32_t rb_, int32_t nrb, int64_t total, int32_t b_first,
                   int64_t off_first, int64_t wg_base = 0) {
    v = wg_start(g, total, G);
    v_end = wg_start(g + 1, total, G);
    ob = off_first;
    wg = wg_base + g * nrb + rb_;
    b = b_first;
    rb = rb_;
    first = true;
  }
  // succ(b): the request after b on the line of positions (b + 1 unless the
  // line holds only some of the requests)
  template <class Units>
  MLA_HD bool next(const Units& units, Piece* pc) {
    return next(units, pc, [](int32_t b) { return b + 1; });
  }
  template <class Units, class Succ>
  MLA_HD bool next(const Units& units, Piece* pc, const Succ& succ) {
    if (v >= v_end) return false;
    const int32_t U = units(b);
    const int64_t oe = ob + kPieceCost + U;      // end of request b's positions
    const int64_t pe = oe < v_end ? oe : v_end;  // end of this piece's positions
    const int64_t t0 = v - ob - kPieceCost, t1 = pe - ob - kPieceCost;
    if (t1 <= 0) {   // only start-up positions: the share ends here
      v = v_end;
      return false;
    }
    pc->b = b;
    pc->rb = rb;
    pc->tile0 = t0 > 0 ? (int32_t)t0 : 0;
    pc->tile1 = (int32_t)t1;
    const bool whole = pc->tile0 == 0 && pc->tile1 == U;
    pc->slot = whole ? -1 : (int32_t)(2 * wg + (first ? 0 : 1));
    first = false;
    v = pe;
    if (pe == oe) {   // request b ends in this share; otherwise the next share starts inside it
      ob = oe;
      b = succ(b);
    }
    return true;
  }
};

// All pieces of balanced-mode group g for row block rb: fn(Piece) is called
// for each in order.
template <class Units, class Fn>
MLA_HD void balanced_pieces(int64_t g, int64_t G, int32_t rb, int32_t nrb, int64_t total, int32_t b_first,
                            int64_t off_first, const Units& units, Fn&& fn) {
  BalancedWalk w;
  w.init(g, G, rb, nrb, total, b_first, off_first);
  Piece pc;
  while (w.next(units, &pc)) fn(pc);
}

// Launch folding (balanced mode).  A split workgroup holds a whole CU, so a
// plan with more groups than the device holds at once (a minimum of work
// units above the CU count) would otherwise run in rounds, every round's
// workgroups paying their own start-up.  Instead the launch has at most
// resident / nrb groups, and each of its workgroups walks vg_per consecutive
// groups of the plan in order.  The plan itself -- its groups, pieces and
// partial slots -- is unchanged; only the launch index -> group map is.
MLA_HD int32_t fold_factor(int64_t groups, int32_t nrb, int32_t num_splits, int32_t resident) {
  if (num_splits > 0 || groups <= 0) return 1;
  int64_t max_groups = resident / nrb;
  if (max_groups < 1) max_groups = 1;
  return groups <= max_groups ? 1 : (int32_t)((groups + max_groups - 1) / max_groups);
}
// Groups the folded launch covers (launch_grid pads them to whole XCD rounds).
MLA_HD int64_t launched_groups(int64_t groups, int32_t vg_per) { return (groups + vg_per - 1) / vg_per; }

// All pieces of balanced-mode groups g0 .. g1-1 for row block rb, in order:
// fn(Piece, g) for each.  b_first / off_first locate start(g0) as for
// BalancedWalk; where one group's share ends, its walk stands at the request
// holding the next group's start, which seeds the next walk.
// succ and wg_base as for BalancedWalk (defaults: every request, in order,
// and workgroups numbered from 0).
template <class Units, class Fn, class Succ>
MLA_HD void folded_balanced_pieces(int64_t g0, int64_t g1, int64_t G, int32_t rb, int32_t nrb, int64_t total,
                                   int32_t b_first, int64_t off_first, const Units& units, Fn&& fn,
                                   const Succ& succ, int64_t wg_base = 0) {
  int32_t b = b_first;
  int64_t ob = off_first;
  for (int64_t g = g0; g < g1; g++) {
    BalancedWalk w;
    w.init(g, G, rb, nrb, total, b, ob, wg_base);
    Piece pc;
    while (w.next(units, &pc, succ)) fn(pc, g);
    b = w.b;
    ob = w.ob;
  }
}
template <class Units, class Fn>
MLA_HD void folded_balanced_pieces(int64_t g0, int64_t g1, int64_t G, int32_t rb, int32_t nrb, int64_t total,
                                   int32_t b_first, int64_t off_first, const Units& units, Fn&& fn) {
  folded_balanced_pieces(g0, g1, G, rb, nrb, total, b_first, off_first, units, fn, [](int32_t b) { return b + 1; });
}

// ---- Row-block classes: the balanced plan of a ragged batch.
//
// With per-request query lengths q_b, request b has n_b = row_blocks(q_b, H)
// row blocks, between 0 and nrb.  A uniform plan gives every group nrb
// workgroups, so the workgroups of the row blocks a request lacks sit idle
// for its pieces.  The class plan gives the requests of each class n (those
// with n_b = n) groups of n workgroups: class n's requests, in batch order,
// are laid on a line of their own cost positions (total T_n), cut into G_n
// equal shares as in the uniform plan.  The groups' workgroups are numbered
// densely, class by class in descending n (class n starts at base_n), and a
// partial piece of group g, row block rb of class n goes to slot
// 2*(base_n + g*n + rb) (first piece of the group) or that plus one (last).
//
// Placement: the launch has 8 XCDs of C workgroup slots each (workgroup i
// runs on XCD i mod 8 as slot i / 8).  Groups are placed whole on one XCD,
// so that a tile's second and later reads hit that XCD's L2: classes in
// descending n, groups in order, each into the current XCD while it has
// room, else into the next (next fit).  G_n is first set in proportion to
// the class's work n*T_n (at least one group per class with work) within
// S slots in all; then, while next fit cannot place every group, the class
// with the most slots gives up a group.  (Striping each class's groups over
// all XCDs, so that every XCD carries the same mix of classes, measured 2 %
// slower on a draft-extend batch.)
constexpr int kMaxClasses = 8;   // the class plan is used for nrb <= 8
// The plan as published for the combine: [0] 1 when the class plan was
// used, [1 + n] T_n, [10 + n] G_n, [19 + n] base_n for n = 0..8.
constexpr int kClassTabInts = 32;
constexpr int kTabT = 1, kTabG = 10, kTabBase = 19;

struct ClassPlan {
  int32_t T[kMaxClasses + 1];      // cost positions of class n (index n = 1..nrb)
  int32_t G[kMaxClasses + 1];      // groups of class n
  int32_t base[kMaxClasses + 1];   // dense workgroup number of class n's first workgroup
  bool ok;                         // false: the uniform plan applies
};

// Whether next fit places G_n groups of n slots for every class, 8 XCDs of C slots.
MLA_HD bool class_fit(const int32_t* G, int32_t nrb, int32_t C) {
  int32_t x = 0, u = 0;
  for (int n = kMaxClasses; n >= 1; n--) {
    if (n > nrb) continue;
    int32_t left = G[n];
    while (left > 0) {
      const int32_t fit = (C - u) / n;
      if (fit <= 0) {
        if (++x >= kXcds) return false;
        u = 0;
        continue;
      }
      const int32_t k = fit < left ? fit : left;
      u += k * n;
      left -= k;
    }
  }
  return true;
}

// The class plan for class totals T[1..nrb] within S workgroup slots, C per
// XCD.  Not ok when nrb > kMaxClasses, when no class has work, when every
// request has all nrb row blocks (the uniform plan is then the same plan),
// or when the classes do not fit.
MLA_HD ClassPlan make_class_plan(const int32_t* T, int32_t nrb, int32_t S, int32_t C) {
  ClassPlan cp;
  cp.ok = false;
  for (int n = 0; n <= kMaxClasses; n++) {
    cp.T[n] = n >= 1 && n <= nrb ? T[n] : 0;
    cp.G[n] = 0;
    cp.base[n] = 0;
  }
  if (nrb > kMaxClasses) return cp;
  int64_t work = 0;
  int32_t need = 0;
  bool other = false;   // work in a class below nrb
  for (int n = 1; n <= kMaxClasses; n++) {
    if (cp.T[n] <= 0) continue;
    work += (int64_t)n * cp.T[n];
    need += n;
    other = other || n < nrb;
  }
  if (work == 0 || !other || need > S) return cp;
  const int64_t R = S - need;
  for (int n = 1; n <= kMaxClasses; n++)
    cp.G[n] = cp.T[n] > 0 ? 1 + (int32_t)(R * cp.T[n] / work) : 0;
  while (!class_fit(cp.G, nrb, C)) {
    int m = 0;   // the class with the most slots that can give up a group
    for (int n = 1; n <= kMaxClasses; n++)
      if (cp.G[n] >= 2 && (m == 0 || cp.G[n] * n >= cp.G[m] * m)) m = n;
    if (m == 0) return cp;
    cp.G[m]--;
  }
  int32_t dense = 0;
  for (int n = kMaxClasses; n >= 1; n--) {
    cp.base[n] = dense;
    dense += cp.G[n] * n;
  }
  cp.ok = true;
  return cp;
}

// The group at slot s of XCD x under next fit: returns its class n (0 if the
// slot holds none) and sets *g and *rb.
MLA_HD int32_t class_slot(const ClassPlan& cp, int32_t nrb, int32_t C, int32_t x_me, int32_t s_me, int32_t* g,
                          int32_t* rb) {
  int32_t x = 0, u = 0;
  for (int n = kMaxClasses; n >= 1; n--) {
    if (n > nrb) continue;
    int32_t left = cp.G[n], placed = 0;
    while (left > 0) {
      const int32_t fit = (C - u) / n;
      if (fit <= 0) {
        if (++x >= kXcds) return 0;
        u = 0;
        continue;
      }
      const int32_t k = fit < left ? fit : left;
      if (x == x_me && s_me >= u && s_me < u + k * n) {
        *g = placed + (s_me - u) / n;
        *rb = (s_me - u) % n;
        return n;
      }
      u += k * n;
      placed += k;
      left -= k;
    }
  }
  return 0;
}

// The single piece of forced-mode group g for row block rb, or false.  U is
// the unit count of request b = g / S.
MLA_HD bool forced_piece(int64_t g, int32_t rb, int32_t nrb, int32_t S, int32_t U, Piece* pc) {
  const int32_t b = (int32_t)(g / S);
  const int32_t s = (int32_t)(g - (int64_t)b * S);
  const int32_t Sp = S < U ? S : U;
  if (s >= Sp) return false;
  pc->b = b;
  pc->rb = rb;
  pc->tile0 = (int32_t)((int64_t)s * U / Sp);
  pc->tile1 = (int32_t)((int64_t)(s + 1) * U / Sp);
  pc->slot = Sp > 1 ? (int32_t)(g * nrb + rb) : -1;
  return true;
}

// The groups holding pieces of a request whose positions start at first_pos
// and that has U tiles (balanced mode): g0 holds its first tile, g1 its last.
MLA_HD int64_t first_group(int64_t first_pos, int64_t total, int64_t G) {
  return wg_of_pos(first_pos + kPieceCost, total, G);
}
MLA_HD int64_t last_group(int64_t first_pos, int32_t U, int64_t total, int64_t G) {
  return wg_of_pos(first_pos + kPieceCost + U - 1, total, G);
}
// Slot of the piece that group g contributes to row block rb of that request
// (g in [g0, g1], group g's share not empty).  Group g0 holds a piece of an
// earlier request first exactly when its share starts before first_pos.
MLA_HD int64_t balanced_slot(int64_t g, int64_t g0, int64_t first_pos, int64_t total, int64_t G, int32_t rb,
                             int32_t nrb) {
  const bool second = g == g0 && wg_start(g0, total, G) < first_pos;
  return 2 * (g * nrb + rb) + (second ? 1 : 0);
}

}  // namespace mla
