"""Pins for the oracle's tiling plan, coverage map, w-bar and RoPE tables (CPU)."""
import json
import math
import os
from collections import Counter

import numpy as np
import pytest

from oracle.brute import brute_cover
from oracle.plan import Plan, rope_pairs, rope_tables
from synth import configs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "plan_derived.json")))


def _plan(name):
    c = configs.get(name)
    return Plan(c["grid"], c["tile"], c["stride"])


@pytest.mark.parametrize("name", ["tiny2d", "small_video", "minimax_h3", "vitok4k"])
def test_plan_matches_hand_derivation(name):
    pl = _plan(name)
    gold = GOLD[name]
    assert pl.axis_starts == gold["axis_starts"]
    assert pl.n_tiles == gold["n_tiles"]
    assert pl.tile_tokens == gold["tile_tokens"]
    assert pl.n_union == gold["n_union"]
    assert pl.n_entries == gold["n_entries"]
    hist = Counter(np.diff(pl.cover_ptr).tolist())
    assert {str(k): v for k, v in hist.items()} == gold["cover_hist"]
    # the token histogram is the product of the per-axis histograms
    prod = Counter()
    ah = gold["axis_hist"]
    for a, ca in ah[0].items():
        for b, cb in ah[1].items():
            for c, cc in ah[2].items():
                prod[str(int(a) * int(b) * int(c))] += ca * cb * cc
    assert dict(prod) == gold["cover_hist"]


@pytest.mark.parametrize("name", ["tiny2d", "small_video", "minimax_h3", "vitok4k"])
def test_tile_rows_partition_and_bounds(name):
    pl = _plan(name)
    rows = pl.tile_rows
    assert rows.min() >= 0 and rows.max() < pl.n_union
    for t in range(pl.n_tiles):
        assert len(set(rows[t].tolist())) == pl.tile_tokens
    assert set(rows.ravel().tolist()) == set(range(pl.n_union))
    # CSR entries point back to the same grid row
    for p in range(0, pl.n_union, max(1, pl.n_union // 997)):
        for t, j, _ in pl.cover_of(p):
            assert rows[t, j] == p
        ts = [t for t, _, _ in pl.cover_of(p)]
        assert ts == sorted(ts)


def test_tiny2d_wbar_is_k_over_9():
    pl = _plan("tiny2d")
    g = GOLD["tiny2d_wbar_overlap_columns"]
    W = 24
    for y in range(16):
        for i, c in enumerate(range(8, 16)):
            ent = pl.cover_of(y * W + c)
            assert [t for t, _, _ in ent] == [0, 1]
            assert ent[0][2] == np.float32(g["tile0_numerators"][i] / g["denominator"])
            assert ent[1][2] == np.float32(g["tile1_numerators"][i] / g["denominator"])
        for c in list(range(0, 8)) + list(range(16, 24)):
            ent = pl.cover_of(y * W + c)
            assert len(ent) == 1 and ent[0][2] == 1.0


@pytest.mark.parametrize("name", ["tiny2d", "small_video", "minimax_h3", "vitok4k"])
def test_wbar_sums_to_one(name):
    pl = _plan(name)
    s = np.add.reduceat(pl.cover_w.astype(np.float64), pl.cover_ptr[:-1])
    # each weight is within half an fp32 ulp of a rational; the sum of <= 4 of them
    # is within a few fp32 ulps of 1
    assert np.max(np.abs(s - 1.0)) < 4 * 2.0 ** -24 * 4
    assert np.all(pl.cover_w > 0) and np.all(pl.cover_w <= 1)


SMALL = [
    ((1, 7, 9), (1, 4, 4), (1, 3, 3)),      # 2D, clamped on both axes
    ((3, 5, 6), (2, 3, 4), (1, 2, 3)),      # 3D, clamped, overlap on every axis
    ((2, 6, 6), (2, 6, 3), (2, 6, 3)),      # zero overlap (stride = tile)
    ((1, 5, 11), (1, 5, 5), (1, 5, 2)),     # deep overlap, up to 3 tiles per token
    ((2, 3, 3), (2, 4, 4), (2, 4, 4)),      # tile larger than the grid: one tile
]


@pytest.mark.parametrize("grid,tile,stride", SMALL)
def test_plan_against_brute_force(grid, tile, stride):
    pl = Plan(grid, tile, stride)
    cover, tiles, ext = brute_cover(grid, tile, stride)
    assert pl.tile_start == tiles
    assert pl.extent == ext
    for p in range(pl.n_union):
        got = pl.cover_of(p)
        exp = cover[p]
        assert [(t, j) for t, j, _ in got] == [(t, j) for t, j, _ in exp]
        # exact rational sum 1
        assert sum(w for _, _, w in exp) == 1
        for (_, _, wg), (_, _, we) in zip(got, exp):
            assert abs(wg - float(we)) <= 2.0 ** -24 * float(we) + 1e-12
            assert np.float32(wg) == np.float32(float(we))


def test_rope_pairs_split():
    assert rope_pairs(3, 128) == (22, 21, 21)
    assert rope_pairs(3, 64) == (12, 10, 10)
    assert rope_pairs(3, 32) == (6, 5, 5)
    assert rope_pairs(3, 16) == (4, 2, 2)
    assert rope_pairs(3, 4) == (2, 0, 0)
    assert rope_pairs(2, 128) == (0, 32, 32)
    assert rope_pairs(2, 64) == (0, 16, 16)
    assert rope_pairs(2, 40) == (0, 10, 10)
    assert rope_pairs(2, 32) == (0, 8, 8)
    assert rope_pairs(2, 12) == (0, 3, 3)
    assert rope_pairs(2, 6) == (0, 1, 2)
    for ndim in (2, 3):
        for hd in (6, 32, 40, 64, 128):
            c = rope_pairs(ndim, hd)
            assert sum(c) == hd // 2
            assert max(c[1:]) - min(c[1:]) <= 1      # h and w balanced
            if ndim == 3:
                assert c[0] >= c[1]                  # t takes the remainder


@pytest.mark.parametrize("ndim,grid,tile,stride,hd", [
    (3, (3, 5, 6), (2, 3, 4), (1, 2, 3), 16),
    (2, (1, 7, 9), (1, 4, 4), (1, 3, 3), 32),
])
def test_rope_tables_against_complex_exponential(ndim, grid, tile, stride, hd):
    """cos/sin match e^{i pos f} with f = base**(-i/m) per axis chunk, and the
    rotation is relative: <R(a)q, R(b)k> depends only on b - a."""
    pl = Plan(grid, tile, stride)
    cos, sin = rope_tables(pl, ndim, hd)
    counts = rope_pairs(ndim, hd)
    freqs = np.concatenate([10000.0 ** (-np.arange(m) / m) for m in counts if m])
    axes = np.concatenate([np.full(m, ax) for ax, m in enumerate(counts) if m])
    pos = pl.local_pos[:, axes]                       # [n, P]
    z = np.exp(1j * pos * freqs[None, :])
    assert np.allclose(cos, z.real, atol=1e-7, rtol=0)
    assert np.allclose(sin, z.imag, atol=1e-7, rtol=0)
    # relativity: rotate complex pairs by z and compare dot products
    rng = np.random.default_rng(1)
    q = rng.standard_normal(hd // 2) + 1j * rng.standard_normal(hd // 2)
    k = rng.standard_normal(hd // 2) + 1j * rng.standard_normal(hd // 2)
    zc = cos + 1j * sin
    n = pl.tile_tokens
    for a in range(0, n, 3):
        for b in range(0, n, 5):
            s_ab = np.real(np.vdot(zc[b] * k, zc[a] * q))
            rel = np.exp(1j * (pos[a] - pos[b]) * freqs)
            assert math.isclose(s_ab, np.real(np.vdot(k, rel * q)), rel_tol=0, abs_tol=1e-5)


# --- hard stitching (Table 2 / Table S2 "Hard stitching") --------------------

@pytest.mark.parametrize("grid,tile,stride", SMALL + [((3, 9, 10), (2, 5, 5), (1, 3, 3)),
                                                      ((2, 9, 9), (2, 6, 6), (1, 4, 5))])
def test_hard_stitching_against_brute_force(grid, tile, stride):
    """One-hot w-bar on the tile of largest ramp, ties to the lowest index, in
    exact rational arithmetic; the maps are those of the ramp plan."""
    pl = Plan(grid, tile, stride, blend="hard")
    soft = Plan(grid, tile, stride)
    cover, _, _ = brute_cover(grid, tile, stride, hard=True)
    assert np.array_equal(pl.cover_ptr, soft.cover_ptr)
    assert np.array_equal(pl.cover_tile, soft.cover_tile)
    assert np.array_equal(pl.cover_local, soft.cover_local)
    for p in range(pl.n_union):
        got = pl.cover_of(p)
        exp = cover[p]
        assert [(t, j) for t, j, _ in got] == [(t, j) for t, j, _ in exp]
        assert [w for _, _, w in got] == [float(w) for _, _, w in exp]
        assert sum(w for _, _, w in got) == 1.0


def test_tiny2d_hard_stitching_splits_the_band_in_the_middle():
    """Columns 8..15 are covered by both tiles with ramps (16-c)/9 (tile 0)
    and (c-7)/9 (tile 1): columns 8..11 go to tile 0, 12..15 to tile 1."""
    pl = Plan((1, 16, 24), (1, 16, 16), (1, 8, 8), blend="hard")
    for y in range(16):
        for c in range(24):
            ent = pl.cover_of(y * 24 + c)
            owner = [t for t, _, w in ent if w == 1.0]
            assert len(owner) == 1 and all(w in (0.0, 1.0) for _, _, w in ent)
            assert owner[0] == (0 if c <= 11 else 1)


def test_hard_stitching_tie_goes_to_lowest_tile():
    """An even overlap of 2 columns (tile 4, stride 2): column 2 of the grid has
    ramps 2/3 (tile 0, trailing) and 1/3 (tile 1, leading), column 3 has 1/3 and
    2/3; with overlap 1 (tile 3, stride 2) the shared column has 1/2 and 1/2,
    a tie, and goes to the lower tile."""
    pl = Plan((1, 1, 5), (1, 1, 3), (1, 1, 2), blend="hard")   # starts 0, 2; overlap 1 at column 2
    ent = pl.cover_of(2)
    assert [t for t, _, _ in ent] == [0, 1]
    assert [w for _, _, w in ent] == [1.0, 0.0]
    pl2 = Plan((1, 1, 6), (1, 1, 4), (1, 1, 2), blend="hard")  # starts 0, 2; overlap 2 at columns 2, 3
    assert [w for _, _, w in pl2.cover_of(2)] == [1.0, 0.0]
    assert [w for _, _, w in pl2.cover_of(3)] == [0.0, 1.0]


def test_blend_rule_is_validated():
    with pytest.raises(ValueError):
        Plan((1, 4, 4), (1, 4, 4), (1, 4, 4), blend="soft")
