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
    got = AR.attention(AR.qk_prep(qkv, cfg, pl, shared, qg, kg, bf16=False), cfg, pl, shared, bf16=False,
                       q_g=qg, k_g=kg)
    assert rel(got, ref) < 2e-5


@pytest.mark.parametrize("case", [c for c in CASES if c[7] == "bf16"], ids=lambda c: f"{c[1]}-hd{c[5]}-qkn{int(c[6])}")
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("qk_scale", QK_SCALES)
def test_rounding_points_stay_under_the_caps(case, shared, qk_scale):
    cfg = case_cfg(*case)
    pl, qkv, qg, kg = case_inputs(cfg, shared, qk_scale)
    ref = oracle_attention(qkv, cfg, pl, shared, qg, kg)
    got = AR.attention(AR.qk_prep(qkv, cfg, pl, shared, qg, kg), cfg, pl, shared, q_g=qg, k_g=kg)
    e = rel(got, ref)
    print(f"  rounding model max|err|/rms {e:.3e} (cap {CAP[qk_scale]})")
    assert e * 1.25 < CAP[qk_scale]
    # and the roundings are not vacuous: the model differs from the exact values
    assert e > 1e-3


@pytest.mark.parametrize("gain", [1.0, 1.3, 1.8])
@pytest.mark.parametrize("shared", [True, False])
def test_fixed_offset_bounds_every_score(gain, shared):
    """The premise of the bf16 kernel's fixed softmax offset under QK-RMSNorm:
    on q and k as the library stores them (normalised, gains, RoPE, bf16),
    every score times log2(e)/sqrt(hd) lies within the offset; past the limit
    (gains x1.8) there is no offset and the kernel keeps a running maximum."""
    case = [c for c in CASES if c[6] and c[7] == "bf16"][0]
    cfg = case_cfg(*case)
    pl, qkv, qg, kg = case_inputs(cfg, shared, 3.0)
    qg, kg = (qg * np.float32(gain)).astype(np.float32), (kg * np.float32(gain)).astype(np.float32)
    off = AR.fixed_offset(cfg, qg, kg)
    if gain > 1.5:
        assert off is None
        return
    assert off is not None and off == int(off)
    # bf16: q as stored carries C = log2(e)/sqrt(hd), so q.k is the score times C
    x = AR.qk_prep(qkv, cfg, pl, shared, qg, kg)
    d, hd = cfg["d"], cfg["head_dim"]
    C = 1.0 / np.log(2.0) / np.sqrt(hd)
    worst = 0.0
    for h in range(cfg["n_heads"]):
        q, k = x[:, h * hd:(h + 1) * hd], x[:, d + h * hd:d + (h + 1) * hd]
        worst = max(worst, float(np.max(np.abs(q @ k.T))))
    print(f"  offset {off}, largest |score| x C {worst:.3f}")
    assert worst <= off
    # not vacuous: the scores reach a fair part of the bound
    assert worst > 0.3 * off
    # the row norms the bound rests on: at most sqrt(hd) max|gain| (times C for
    # q), plus bf16 rounding
    qn = np.linalg.norm(x[:, :hd], axis=1)
    kn = np.linalg.norm(x[:, d:d + hd], axis=1)
    assert np.max(qn) <= np.sqrt(hd) * float(np.max(np.abs(qg))) * C * 1.005
    assert np.max(kn) <= np.sqrt(hd) * float(np.max(np.abs(kg))) * 1.005


@pytest.mark.parametrize("qk_scale", [1.0, 3.0, 8.0])
@pytest.mark.parametrize("shared", [True, False])
def test_norm_offset_bounds_every_score(qk_scale, shared):
    """The bf16 kernel's fixed softmax offset without QK-norm: the largest q
    and k head norms as stored bound every score (Cauchy-Schwarz), so every
    score (times C, which q carries) lies within the offset; when the bound
    passes the limit there is no offset and the kernel keeps a running
    maximum."""
    case = [c for c in CASES if not c[6] and c[7] == "bf16"][0]
    cfg = case_cfg(*case)
    pl, qkv, qg, kg = case_inputs(cfg, shared, qk_scale)
    x = AR.qk_prep(qkv, cfg, pl, shared)
    d, hd, H = cfg["d"], cfg["head_dim"], cfg["n_heads"]
    q, k = x[:, :d], x[:, d:2 * d]
    off = AR.norm_offset(q, k, H, hd)
    qm = max(float(np.max(np.linalg.norm(q[:, h * hd:(h + 1) * hd], axis=1))) for h in range(H))
    km = max(float(np.max(np.linalg.norm(k[:, h * hd:(h + 1) * hd], axis=1))) for h in range(H))
    worst = max(float(np.max(np.abs(q[:, h * hd:(h + 1) * hd] @ k[:, h * hd:(h + 1) * hd].T))) for h in range(H))
    print(f"  offset {off}, bound {qm * km:.3f}, largest |score| x C {worst:.3f}")
    assert worst <= qm * km * (1 + 1e-9)
    if qm * km * 1.01 + 1e-3 > AR.FIXED_MAX_LIMIT:
        assert off is None
        return
    assert off is not None and off == int(off) and off >= qm * km * 1.01
    assert worst <= off
    # with the 1 % margin and the rounding up, the offset is the bound's ceiling
    assert off <= qm * km * 1.01 + 1e-3 + 1


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
