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


# ---- ragged batches: the row-block class plan

def model_class_plan(T, nrb, S, C):
    """The class plan from its definition: at least one group per class with
    work, the rest of the S slots in proportion to each class's work n*T_n
    (groups G_n = 1 + floor(R*T_n/work)); while next fit (classes in
    descending n, 8 XCDs of C slots, a group whole on one XCD) cannot place
    every group, the class with the most slots (the larger n on a tie) gives
    up one.  None where the uniform plan applies."""
    if nrb > 8:
        return None
    cls = [n for n in range(1, nrb + 1) if T[n] > 0]
    work = sum(n * T[n] for n in cls)
    if work == 0 or not any(n < nrb for n in cls) or sum(cls) > S:
        return None
    R = S - sum(cls)
    G = {n: (1 + R * T[n] // work if n in cls else 0) for n in range(1, 9)}

    def fits():
        bins = [0] * 8
        x = 0
        for n in range(8, 0, -1):
            for _ in range(G[n]):
                while x < 8 and bins[x] + n > C:
                    x += 1
                if x == 8:
                    return False
                bins[x] += n
        return True

    while not fits():
        m = max((n for n in G if G[n] >= 2), key=lambda n: (G[n] * n, n), default=None)
        if m is None:
            return None
        G[m] -= 1
    base, dense = {}, 0
    for n in range(8, 0, -1):
        base[n] = dense
        dense += G[n] * n
    return G, base


def _ragged_case(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 60))
    H = int(rng.choice([16, 32, 64, 128] if seed % 4 == 0 else [64, 128]))
    q_max = int(rng.integers(1, 5) if seed % 4 == 0 else rng.integers(2, 5))
    while q_max * H > 512:     # at most 8 row blocks, so that the class plan may apply
        q_max -= 1
    L = rng.integers(0, 3000, size=B).astype(np.int32)
    ql = rng.integers(0, q_max + 1, size=B)
    if seed % 3 == 0:
        ql[:] = q_max             # every request with all its row blocks: the uniform plan
    ind = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    cus = int(rng.choice([64, 256]))
    p = params(B, q_max, H, int(max(L.max(), 1)), num_cus=cus)
    return p, L, ql, ind, H, q_max


@pytest.mark.parametrize("seed", range(12))
def test_ragged_class_plan_is_its_definition(seed):
    """The host mirror of the ragged plan against the plan written out from
    its definition: every request's row blocks with rows covered exactly
    once, and with the class plan, each class's pieces those of a balanced
    plan over that class's requests alone, renumbered into the dense slots."""
    p, L, ql, ind, H, q_max = _ragged_case(seed)
    pieces, grid, used = mla.mla_plan_host_ragged(p, L, ind, int(ind[-1]))
    nrb = -(-q_max * H // mla.ROWS_PER_BLOCK)
    NG = grid // nrb
    nb = np.array([-(-int(q) * H // mla.ROWS_PER_BLOCK) for q in ql])
    c = mla.PIECE_COST
    U = np.maximum(1, -(-np.clip(L, 0, p.max_seq_len) // mla.TILE))
    # coverage: (b, rb) for rb < n_b tiled exactly once, nothing for the rest
    cover = {}
    for g, b, rb, t0, t1, slot in pieces:
        assert rb < nb[b]
        cover.setdefault((b, rb), []).append((t0, t1, slot))
    assert set(cover) == {(b, rb) for b in range(len(L)) for rb in range(nb[b])}
    slots = [s for _, _, _, _, _, s in pieces if s >= 0]
    assert len(slots) == len(set(slots)) and all(s < 2 * NG * nrb for s in slots)
    for (b, rb), lst in cover.items():
        lst.sort()
        assert lst[0][0] == 0 and lst[-1][1] == U[b]
        assert all(a[1] == n[0] for a, n in zip(lst, lst[1:]))
        assert (len(lst) == 1) == (lst[0][2] == -1)
    T = {n: int(sum(c + U[b] for b in range(len(L)) if nb[b] == n)) for n in range(0, 9)}
    model = model_class_plan(T, nrb, min(NG * nrb, p.num_cus), min(-(-NG // 8) * nrb, p.num_cus // 8))
    assert used == (model is not None)
    if model is None:
        if (nb == nrb).all():   # the uniform plan: mla_plan_host's
            ref, g2 = mla.mla_plan_host(p, L)
            assert g2 == grid and np.array_equal(np.asarray(pieces), ref)
        return
    G, base = model
    want = []
    for n in range(1, 9):
        members = [b for b in range(len(L)) if nb[b] == n]
        if not members:
            continue
        for wg, bl, rb, t0, t1, slot in model_balanced_plan(L[members], p.max_seq_len, n, G[n], c):
            want.append((base[n] + wg, members[bl], rb, t0, t1, slot + 2 * base[n] if slot >= 0 else -1))
    assert sorted(map(tuple, np.asarray(pieces).tolist())) == sorted(want)


@pytest.mark.parametrize("seed", range(6))
def test_ragged_class_plan_combine_lookup(seed):
    """What the combine computes for a split request of a class plan, from
    its class's groups and the request's offset on the class's line, names
    exactly the slots its pieces wrote, in order."""
    p, L, ql, ind, H, q_max = _ragged_case(3 * seed + 1)
    pieces, grid, used = mla.mla_plan_host_ragged(p, L, ind, int(ind[-1]))
    if not used:
        pytest.skip("the uniform plan applies to this batch")
    nrb = -(-q_max * H // mla.ROWS_PER_BLOCK)
    NG = grid // nrb
    nb = np.array([-(-int(q) * H // mla.ROWS_PER_BLOCK) for q in ql])
    c = mla.PIECE_COST
    U = np.maximum(1, -(-np.clip(L, 0, p.max_seq_len) // mla.TILE))
    T = {n: int(sum(c + U[b] for b in range(len(L)) if nb[b] == n)) for n in range(0, 9)}
    G, base = model_class_plan(T, nrb, min(NG * nrb, p.num_cus), min(-(-NG // 8) * nrb, p.num_cus // 8))
    by_req = {}
    for g, b, rb, t0, t1, slot in pieces:
        by_req.setdefault((b, rb), []).append((t0, slot))
    for (b, rb), lst in by_req.items():
        if len(lst) == 1:
            continue
        n = nb[b]
        first = sum(c + U[x] for x in range(b) if nb[x] == n)
        Tn, Gn = T[n], G[n]
        start = lambda g: g * Tn // Gn
        of = lambda v: ((v + 1) * Gn - 1) // Tn
        g0, g1 = of(first + c), of(first + c + U[b] - 1)
        got = []
        for g in range(g0, g1 + 1):
            if start(g) == start(g + 1):
                continue
            second = g == g0 and start(g0) < first
            got.append(2 * base[n] + 2 * (g * n + rb) + (1 if second else 0))
        assert got == [s for _, s in sorted(lst)]
