"""The split-KV work plan on the host (no GPU): every (request, row block)
is covered exactly once, partial slots are unique, the balanced grid is
evenly loaded once each piece's start-up cost is counted."""
import math

import numpy as np
import pytest

import paged_mla_decode_06_amd as mla


def params(B, q_len, H, max_len, num_splits=0, min_work_units=0, num_cus=256, P=64):
    W = max(1, -(-max_len // P))
    return mla.make_params(B, q_len, H, P, 1 << 20, W, max_len, mla.MLA_KV_BF16, 0.07, 1.0, num_splits,
                           min_work_units, num_cus)


def check_cover(p, L, pieces, grid):
    B, nrb = p.batch, -(-p.q_len * p.num_heads // mla.ROWS_PER_BLOCK)
    U = np.maximum(1, -(-np.clip(L, 0, p.max_seq_len) // mla.TILE))
    cover = {}
    for g, b, rb, t0, t1, slot in pieces:
        assert 0 <= g < grid and 0 <= b < B and 0 <= rb < nrb and 0 <= t0 < t1 <= U[b]
        cover.setdefault((b, rb), []).append((t0, t1, slot, g))
    assert len(cover) == B * nrb
    used = set()
    for (b, rb), lst in cover.items():
        lst.sort()
        assert lst[0][0] == 0 and lst[-1][1] == U[b]
        for (a0, a1, _, _), (c0, _, _, _) in zip(lst, lst[1:]):
            assert a1 == c0, "pieces must tile the range without gaps or overlap"
        if len(lst) == 1:
            assert lst[0][2] == -1, "a whole row block writes the output directly"
        else:
            for _, _, slot, _ in lst:
                assert slot >= 0 and slot not in used
                used.add(slot)
    return cover


def model_balanced_plan(L, max_len, nrb, NG, c):
    """The balanced plan written out from its definition: request b takes c
    start-up positions and then one position per 32-token tile; group g takes
    positions [g*T//NG, (g+1)*T//NG); the tiles of a request inside a group's
    positions form its piece; a partial piece goes to slot 2*wg if it is the
    group's first piece, else 2*wg+1."""
    U = [max(1, -(-min(max(int(x), 0), max_len) // mla.TILE)) for x in L]
    off = [0]
    for u in U:
        off.append(off[-1] + c + u)
    T = off[-1]
    out = []
    for g in range(NG):
        v0, v1 = g * T // NG, (g + 1) * T // NG
        for rb in range(nrb):
            wg = g * nrb + rb
            first = True
            for b in range(len(U)):
                s = off[b] + c          # position of tile 0
                t0, t1 = max(v0, s) - s, min(v1, off[b + 1]) - s
                if t1 > t0:
                    whole = t0 == 0 and t1 == U[b]
                    out.append((wg, b, rb, t0, t1, -1 if whole else 2 * wg + (0 if first else 1)))
                    first = False
    return sorted(out)


@pytest.mark.parametrize("seed", range(6))
def test_balanced_plan_covers_and_balances(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    q_len = int(rng.choice([1, 2, 4]))
    H = int(rng.choice([16, 64, 128]))
    L = rng.integers(0, 5000, size=B).astype(np.int32)
    if seed == 0:
        L[:] = 0
    p = params(B, q_len, H, int(max(L.max(), 1)), num_cus=int(rng.choice([8, 256, 512])))
    pieces, grid = mla.mla_plan_host(p, L)
    check_cover(p, L, pieces, grid)
    nrb = -(-q_len * H // mla.ROWS_PER_BLOCK)
    assert sorted(map(tuple, np.asarray(pieces).tolist())) == \
        model_balanced_plan(L, p.max_seq_len, nrb, grid // nrb, mla.PIECE_COST)
    # each workgroup's cost, its tiles plus the start-up cost of every request
    # whose first tile it holds, is within the start-up cost of an equal share
    c = mla.PIECE_COST
    cost = np.zeros(grid, dtype=np.int64)
    for g, b, rb, t0, t1, slot in pieces:
        cost[g] += (t1 - t0) + (c if t0 == 0 else 0)
    U = np.maximum(1, -(-np.clip(L, 0, p.max_seq_len) // mla.TILE)).astype(np.int64)
    share = (U.sum() + c * B) / (grid // nrb)
    assert np.all(np.abs(cost - share) <= c + 1)
    # at most two partial pieces per workgroup
    part = np.zeros(grid, dtype=np.int64)
    for g, b, rb, t0, t1, slot in pieces:
        part[g] += slot >= 0
    assert part.max() <= 2


@pytest.mark.parametrize("seed", range(8))
def test_folded_launch_walks_the_same_plan(seed):
    """More groups than the CUs hold (min_work_units above num_cus): each
    launched workgroup walks several consecutive plan groups, every walk
    continuing from where the previous group's share ended -- also inside a
    request, inside its start-up positions, or after an empty share.  The
    pieces are the plan's own: equal to the model written from the plan's
    definition."""
    rng = np.random.default_rng(300 + seed)
    B = int(rng.integers(1, 40))
    q_len, H = int(rng.choice([1, 2, 4])), int(rng.choice([16, 64, 128]))
    L = rng.integers(0, 3000, size=B).astype(np.int32)
    L[rng.random(B) < 0.2] = 0
    L[rng.random(B) < 0.2] = 1
    cus = int(rng.choice([8, 64, 256]))
    p = params(B, q_len, H, int(max(L.max(), 1)), min_work_units=int(rng.integers(cus + 1, 6 * cus + 2)),
               num_cus=cus)
    pieces, grid = mla.mla_plan_host(p, L)
    nrb = -(-q_len * H // mla.ROWS_PER_BLOCK)
    check_cover(p, L, pieces, grid)
    assert sorted(map(tuple, np.asarray(pieces).tolist())) == \
        model_balanced_plan(L, p.max_seq_len, nrb, grid // nrb, mla.PIECE_COST)
    # listed by plan workgroup, as the device plan lists them
    assert np.all(np.diff(np.asarray(pieces)[:, 0]) >= 0)


@pytest.mark.parametrize("seed", range(6))
def test_split_requests_end_in_distinct_group_shares(seed):
    """What the combine's group grid relies on (plans with fewer groups than
    requests): the last piece of every split request lies in a group g whose
    share starts inside that request, after its first tile; so the request
    holding a group's first position, if split and ending in that group, is
    the only one the group's combine workgroups have to merge, and every
    split request is merged by exactly one group."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(20, 1025))
    q_len, H = int(rng.choice([1, 4])), int(rng.choice([16, 128]))
    L = rng.integers(0, 9000, size=B).astype(np.int32)
    L[rng.random(B) < 0.1] = 0
    p = params(B, q_len, H, int(max(L.max(), 1)), num_cus=int(rng.choice([64, 256])))
    pieces, grid = mla.mla_plan_host(p, L)
    nrb = -(-q_len * H // mla.ROWS_PER_BLOCK)
    NG, c = grid // nrb, mla.PIECE_COST
    U = np.maximum(1, -(-np.clip(L, 0, p.max_seq_len) // mla.TILE)).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(U + c)])
    T = int(off[-1])
    start = [g * T // NG for g in range(NG)]
    last_group = {}
    n_pieces = {}
    for wg, b, rb, t0, t1, slot in pieces:
        if rb == 0:
            n_pieces[b] = n_pieces.get(b, 0) + 1
            if t1 == U[b]:
                last_group[b] = wg // nrb
    split = {b for b, n in n_pieces.items() if n > 1}
    merged = []
    for g in range(NG):
        b = int(np.searchsorted(off, start[g], side="right") - 1)   # the request holding start(g)
        if start[g] < T and b in split and last_group[b] == g:
            assert off[b] + c < start[g], "the share starts after the request's first tile"
            merged.append(b)
    assert sorted(merged) == sorted(split)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 64])
def test_forced_plan(S):
    L = np.array([0, 1, 31, 32, 33, 300, 4096], dtype=np.int32)
    p = params(len(L), 1, 128, 4096, num_splits=S)
    pieces, grid = mla.mla_plan_host(p, L)
    nrb = -(-128 // mla.ROWS_PER_BLOCK)
    assert grid == len(L) * nrb * S
    cover = check_cover(p, L, pieces, grid)
    for (b, rb), lst in cover.items():
        U = max(1, -(-int(L[b]) // 32))
        assert len(lst) == min(S, U)


def test_grid_follows_cu_count_and_min_units():
    L = np.full(8, 32768, dtype=np.int32)
    _, grid = mla.mla_plan_host(params(8, 1, 128, 32768, num_cus=256), L)
    assert grid == 256
    _, grid = mla.mla_plan_host(params(8, 1, 128, 32768, min_work_units=512, num_cus=256), L)
    assert grid == 512
    # never more workgroups than units
    _, grid = mla.mla_plan_host(params(2, 1, 16, 100, num_cus=256), np.array([100, 50], dtype=np.int32))
    assert grid == 2 * 1 * 4


def test_long_context_workload_plan():
    """The long-context workload asks for at least 2x the CU count of work units."""
    from mla_synth import WORKLOADS
    from mla_synth.gen import draw_seq_lens
    w = WORKLOADS["long_context"]
    L = draw_seq_lens(w, np.random.default_rng(w.seed))
    p = params(w.batch, 1, w.heads, 32768, min_work_units=w.min_work_units, P=32)
    pieces, grid = mla.mla_plan_host(p, L)
    assert grid >= 512
    check_cover(p, L, pieces, grid)
