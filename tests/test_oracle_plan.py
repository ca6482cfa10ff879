"""Pins of the oracle's placement plan (no GPU).

The plan is pinned to (a) a hand-worked example, (b) an independent brute-force
construction written with plain Python loops on every routing of tiny shapes,
and (c) the invariants of an expert-major, tile-padded pool (StreamEP README,
"How it works": pool-layout dispatch).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_plan(ids, expert_begin, E_local, tile):
    """Placement built one row at a time: experts in ascending order, each expert's
    pairs in ascending pair id, then padding rows until the segment is whole tiles."""
    T = len(ids)
    K = len(ids[0]) if T else 0
    pairs = [(t * K + k, ids[t][k]) for t in range(T) for k in range(K)]
    pos = [-1] * (T * K)
    rows = []            # pair id per pool row, -1 for padding
    tiles = []
    counts = []
    offsets = [0]
    for ex in range(E_local):
        mine = [q for q, i in pairs if i == expert_begin + ex]
        counts.append(len(mine))
        for q in mine:
            pos[q] = len(rows)
            rows.append(q)
        while len(rows) % tile != 0:
            rows.append(-1)
        while len(tiles) * tile < len(rows):
            tiles.append(ex)
        offsets.append(len(rows))
    return counts, offsets, pos, rows, tiles


def check_against_brute(ids, expert_begin, E_local, tile):
    p = oracle.plan(np.array(ids, dtype=np.int32).reshape(len(ids), -1), expert_begin, E_local, tile)
    counts, offsets, pos, rows, tiles = brute_force_plan(ids, expert_begin, E_local, tile)
    assert p.counts.tolist() == counts
    assert p.offsets.tolist() == offsets
    assert p.pos.tolist() == pos
    assert p.P == len(rows) and p.num_tiles == len(tiles)
    assert p.src[: p.P].tolist() == rows
    assert (p.src[p.P:] == -1).all()
    assert p.tile_expert[: p.num_tiles].tolist() == tiles
    assert (p.tile_expert[p.num_tiles:] == -1).all()
    # invariants of the pool
    T, K = len(ids), len(ids[0])
    local = [q for q in range(T * K) if expert_begin <= ids[q // K][q % K] < expert_begin + E_local]
    assert sum(counts) == len(local)
    for q in local:                       # each local pair lands exactly once ...
        assert p.src[p.pos[q]] == q       # ... and src inverts pos
    assert sorted(p.pos[p.pos >= 0].tolist()) == sorted(set(p.pos[p.pos >= 0].tolist()))
    assert all((offsets[e + 1] - offsets[e]) % tile == 0 for e in range(E_local))
    assert p.P <= p.P_cap == oracle.pool_rows_bound(T, K, E_local, tile)
    return p


def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "plan_hand_worked.json")))
    p = oracle.plan(np.array(g["topk_idx"], dtype=np.int32), g["expert_begin"], g["E_local"], g["tile"])
    assert p.counts.tolist() == g["counts"]
    assert p.offsets.tolist() == g["offsets"]
    assert p.pos.tolist() == g["pos"]
    assert p.src.tolist() == g["src"]
    assert p.tile_expert.tolist() == g["tile_expert"]
    assert p.num_tiles == g["num_tiles"]


@pytest.mark.parametrize("T,K", [(1, 1), (1, 2), (2, 2), (3, 1)])
@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_every_routing_small(T, K, tile):
    # ids range over -1, the local experts 0..2 and one id past the local range
    values = [-1, 0, 1, 2, 3]
    n = 0
    for flat in itertools.product(values, repeat=T * K):
        ids = [list(flat[t * K:(t + 1) * K]) for t in range(T)]
        check_against_brute(ids, 0, 3, tile)
        n += 1
    assert n == len(values) ** (T * K)


@pytest.mark.parametrize("tile", [1, 2])
def test_every_routing_three_tokens_two_k(tile):
    values = [-1, 1, 2, 3]          # expert_begin = 1: ids 1, 2 local, 3 and -1 not
    for flat in itertools.product(values, repeat=6):
        ids = [list(flat[0:2]), list(flat[2:4]), list(flat[4:6])]
        check_against_brute(ids, 1, 2, tile)


def test_random_medium_shapes():
    rng = np.random.default_rng(7)
    for _ in range(40):
        T = int(rng.integers(1, 60))
        K = int(rng.integers(1, 5))
        E = int(rng.integers(1, 9))
        tile = int(rng.choice([1, 2, 4, 16]))
        ids = rng.integers(-1, E + 2, size=(T, K)).tolist()
        check_against_brute(ids, 0, E, tile)


def test_tile_one_is_stable_sort():
    # with tile = 1 there is no padding and the pool is the stable sort of pairs by expert
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 5, size=(30, 3))
    p = oracle.plan(ids.astype(np.int32), 0, 5, 1)
    keyed = sorted(range(90), key=lambda q: (ids.reshape(-1)[q], q))
    assert p.src[:90].tolist() == keyed


def test_empty_expert_gets_no_rows():
    ids = np.array([[0, 2], [2, 0]], dtype=np.int32)   # expert 1 empty
    p = oracle.plan(ids, 0, 3, 4)
    assert p.counts.tolist() == [2, 0, 2]
    assert p.offsets.tolist() == [0, 4, 4, 8]
    assert p.tile_expert[:2].tolist() == [0, 2]


def test_no_local_pairs():
    ids = np.full((5, 2), 9, dtype=np.int32)
    p = oracle.plan(ids, 0, 4, 16)
    assert p.P == 0 and p.num_tiles == 0
    assert (p.pos == -1).all() and (p.src == -1).all() and (p.tile_expert == -1).all()
