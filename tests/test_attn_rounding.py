"""The attention rounding model (attn_rounding.py) against the oracle, on the CPU.

1. With its roundings switched off the model is the oracle's definition up to
   fp64 noise: rotating every row by its grid coordinate gives the scores of
   tile-local RoPE, the query blocks' window passes and w-bar sums give the
   oracle's blend, and the global rows are the tiles' own.
2. With them on, it stays within the caps the GPU attention tests use
   (attn_cases.CAP), with a 1.25x margin: those caps are what bf16 q, k,
   softmax weights and outputs produce on the test inputs.
3. Its query blocks follow the rule the plan states (every grid row once,
   rows of a block share their weighted tiles, at most 256 rows per block).
"""
import numpy as np
import pytest

import attn_rounding as AR
from attn_cases import CAP, CASES, QK_SCALES, case_cfg, case_inputs, oracle_attention, rel
from oracle.plan import Plan


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[1]}-hd{c[5]}-qkn{int(c[6])}-{c[7]}")
@pytest.mark.parametrize("shared", [True, False])
def test_model_without_rounding_is_the_oracle(case, shared):
    cfg = case_cfg(*case)
    pl, qkv, qg, kg = case_inputs(cfg, shared, 3.0)
    ref = oracle_attention(qkv, cfg, pl, shared, qg, kg)
    got = AR.attention(AR.qk_prep(qkv, cfg, pl, shared, qg, kg, bf16=False), cfg, pl, shared, bf16=False)
    assert rel(got, ref) < 2e-5


@pytest.mark.parametrize("case", [c for c in CASES if c[7] == "bf16"], ids=lambda c: f"{c[1]}-hd{c[5]}-qkn{int(c[6])}")
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("qk_scale", QK_SCALES)
def test_rounding_points_stay_under_the_caps(case, shared, qk_scale):
    cfg = case_cfg(*case)
    pl, qkv, qg, kg = case_inputs(cfg, shared, qk_scale)
    ref = oracle_attention(qkv, cfg, pl, shared, qg, kg)
    got = AR.attention(AR.qk_prep(qkv, cfg, pl, shared, qg, kg), cfg, pl, shared)
    e = rel(got, ref)
    print(f"  rounding model max|err|/rms {e:.3e} (cap {CAP[qk_scale]})")
    assert e * 1.25 < CAP[qk_scale]
    # and the roundings are not vacuous: the model differs from the exact values
    assert e > 1e-3


@pytest.mark.parametrize("grid,tile,stride,blend", [((2, 12, 20), (2, 8, 8), (2, 6, 6), "ramp"),
                                                     ((1, 20, 36), (1, 16, 16), (1, 12, 12), "hard"),
                                                     ((3, 9, 10), (2, 4, 5), (1, 3, 2), "ramp")])
def test_query_blocks_cover_every_row_once(grid, tile, stride, blend):
    pl = Plan(grid, tile, stride, blend=blend)
    blocks = AR.query_blocks(pl)
    seen = np.concatenate([rows for _, rows in blocks])
    assert np.array_equal(np.sort(seen), np.arange(pl.n_union))
    for tiles, rows in blocks:
        assert 1 <= len(rows) <= AR.QB and list(tiles) == sorted(tiles)
        for r in rows:
            assert tuple(t for t, _, w in pl.cover_of(int(r)) if w != 0.0) == tiles
    sizes = [len(t) for t, _ in blocks]
    assert sizes == sorted(sizes, reverse=True)
    if blend == "hard":
        assert all(len(t) == 1 for t, _ in blocks)
