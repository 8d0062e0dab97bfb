"""Host check of the GEMM kernels' workgroup -> tile arithmetic (no GPU).

The forward / dgrad kernels map block b to a whole tile, or to one part of a
remainder tile cut along the contraction (`deal_tile_split` in gemm_bf16.hip);
the weight-gradient kernel maps block b to a tile through chunks dealt
round-robin over the 8 XCDs (`k_gemm_wgrad`). Both are restated here in plain
integer arithmetic and checked over a sweep of shapes: every tile (every part of
every cut tile) is reached by exactly one block of the launched grid, the parts
of a tile partition the contraction, share one XCD and use distinct partial-tile
slots below the resident count. The GPU parity tests check the kernels themselves.
"""
import itertools

import numpy as np

SPLIT_MAX = 8
SPLIT_SLOTS = 256


def round_up8(v):
    return (v + 7) // 8 * 8


def deal_split(b, total, n_res, ktiles):
    """-> None (block exits) or (t, part, S, slot, cidx, k0, nk)."""
    full, rem, S, part, slot, cidx = total, 0, 1, 0, 0, 0
    if n_res > 0:
        full = total // n_res * n_res
        rem = total - full
        if rem > 0:
            S = min(n_res // rem, SPLIT_MAX, ktiles)
    if S < 2:
        S = 1
        per = (total + 7) >> 3
        t = (b & 7) * per + (b >> 3)
        if (b >> 3) >= per or t >= total:
            return None
    elif b < full:
        t = (b & 7) * (full >> 3) + (b >> 3)
        S = 1
    else:
        u = b - full
        w = u >> 3
        i = (w // S) * 8 + (u & 7)
        if i >= rem:
            return None
        part = w % S
        t = full + i
        slot = i * S + part
        cidx = i
    k0 = ktiles * part // S
    nk = ktiles * (part + 1) // S - k0
    return t, part, S, slot, cidx, k0, nk


def _check_split(total, n_res, ktiles, bound_extra=0):
    tiles_bound = total + bound_extra       # the launch uses an upper bound on the tiles
    grid = round_up8(tiles_bound + (n_res + 8 * SPLIT_MAX if n_res > 0 else 0))
    seen = {}
    for b in range(grid):
        r = deal_split(b, total, n_res, ktiles)
        if r is None:
            continue
        t, part, S, slot, cidx, k0, nk = r
        assert 0 <= t < total
        assert nk >= 1 and 0 <= k0 and k0 + nk <= ktiles
        seen.setdefault(t, []).append((part, S, slot, cidx, k0, nk, b & 7))
    assert sorted(seen) == list(range(total)), "a tile is missing"
    slots = set()
    for t, parts in seen.items():
        S = parts[0][1]
        assert len(parts) == S and sorted(p[0] for p in parts) == list(range(S))
        assert len({p[6] for p in parts}) == 1, "parts of one tile on different XCDs"
        ranges = sorted((p[4], p[5]) for p in parts)
        assert ranges[0][0] == 0 and sum(n for _, n in ranges) == ktiles
        assert all(a + n == c for (a, n), (c, _) in zip(ranges, ranges[1:]))
        if S > 1:
            assert len({p[3] for p in parts}) == 1
            for p in parts:
                assert p[2] < min(n_res, SPLIT_SLOTS) and p[2] not in slots
                slots.add(p[2])


def test_split_dealing_covers_every_tile_and_part_once():
    rng = np.random.default_rng(0)
    totals = [1, 2, 7, 8, 9, 63, 64, 65, 200, 255, 256, 257, 300, 512, 576, 784, 1000, 4032]
    for total, n_res, ktiles in itertools.product(totals, [0, 8, 64, 248, 256], [1, 2, 3, 7, 64, 896]):
        _check_split(total, n_res, ktiles, bound_extra=int(rng.integers(0, 40)))


def test_split_dealing_mixtral_fc1_dgrad_cut():
    """576 tiles on 256 resident workgroups: 512 whole tiles and 64 tiles cut in 4."""
    cut = [deal_split(b, 576, 256, 896) for b in range(512, 512 + 256)]
    assert all(r is not None and r[2] == 4 for r in cut)
    assert {r[0] for r in cut} == set(range(512, 576))


def deal_wgrad(b, E, n_tiles, k_tiles):
    x, s = b & 7, b >> 3
    t = ((s // k_tiles) * 8 + x) * k_tiles + s % k_tiles
    return t if t < E * n_tiles * k_tiles else None


def test_wgrad_dealing_covers_every_tile_once_and_balances_groups():
    for E, n_tiles, k_tiles in itertools.product([1, 3, 8, 16, 33], [1, 2, 7, 16, 56], [1, 3, 8, 16]):
        grid = 8 * ((E * n_tiles + 7) // 8) * k_tiles
        per_e = n_tiles * k_tiles
        hits = np.zeros(E * per_e, dtype=np.int64)
        share = np.zeros((E, 8), dtype=np.int64)     # tiles of each group per XCD
        for b in range(grid):
            t = deal_wgrad(b, E, n_tiles, k_tiles)
            if t is None:
                continue
            hits[t] += 1
            share[t // per_e, b & 7] += 1
            # a chunk is one output tile row: k_tiles tiles of one group sharing a G slice
            assert (t % per_e) // k_tiles == ((t - t % k_tiles) % per_e) // k_tiles
        assert np.all(hits == 1)
        # every XCD holds an equal share of every group, up to one chunk
        assert np.all(share.max(axis=1) - share.min(axis=1) <= k_tiles)
