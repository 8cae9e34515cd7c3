"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled outputs that the oracle computes one by one.

Each case runs one call of the C ABI over the whole workload (every tile,
every row, the ragged last query and key blocks) and compares a sample of
output rows with the oracle's float64 value of exactly those rows: the
first and last rows, rows on block edges, rows covered by each possible
number of tiles, the global rows, and seeded random rows.
"""
import numpy as np
import pytest
import torch

import shared_token_tiled_amd as ts
from oracle import fp8 as ofp8
from oracle import model as M
from oracle.plan import Plan
from synth import configs, make_inputs, round_bf16

import attn_cases as AC
import attn_rounding as AR
from gpu_helpers import DEV, TOL, Run, max_rel, say

pytestmark = pytest.mark.gpu


def _sample_rows(m, seed, extra=()):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 63, 64, 255, 256, m - 257, m - 256, m - 3, m - 2, m - 1, *extra]
    rand = rng.choice(m, size=24, replace=False).tolist()
    return np.array(sorted({r for r in fixed + rand if 0 <= r < m}), dtype=np.int64)


def _randn(rng, shape, std=1.0):
    return (std * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)


def _union_sample(pl, seed):
    """Rows covered by each possible number of tiles, plus edges and random rows."""
    counts = np.diff(pl.cover_ptr)
    extra = []
    for c in sorted(set(counts.tolist())):
        idx = np.nonzero(counts == c)[0]
        extra += [int(idx[0]), int(idx[len(idx) // 2]), int(idx[-1])]
    return _sample_rows(pl.n_union, seed, extra)


MINIMAX = configs.get("minimax_h3")
_PL = Plan(MINIMAX["grid"], MINIMAX["tile"], MINIMAX["stride"])
M_SHARED = _PL.n_union + _PL.n_tiles                 # rows of a shared-layer GEMM
M_TILED = _PL.n_tiles * (_PL.tile_tokens + 1)        # rows of a per-tile GEMM
D, DM = MINIMAX["d"], MINIMAX["mlp_hidden"]

# (name, M, N, K, epilogue): the GEMMs of one MiniMax-H3-scale layer
GEMMS = [("qkv", M_SHARED, 3 * D, D, ts.TS_EPI_BIAS),
         ("out", M_SHARED, D, D, ts.TS_EPI_RESIDUAL),
         ("fc1", M_SHARED, DM, D, ts.TS_EPI_BIAS_GELU),
         ("fc2", M_SHARED, D, DM, ts.TS_EPI_RESIDUAL),
         ("qkv_per_tile", M_TILED, 3 * D, D, ts.TS_EPI_BIAS)]


@pytest.mark.parametrize("name,M_,N,K,epi", GEMMS)
def test_full_size_gemm_bf16(name, M_, N, K, epi):
    say(f"full-size gemm bf16 {name} M={M_} N={N} K={K} epi={epi}")
    r = np.random.default_rng(M_ + N + K)
    A = round_bf16(_randn(r, (M_, K)))
    B = round_bf16(_randn(r, (N, K), 0.02))
    bias = _randn(r, (N,), 0.02)
    rows = _sample_rows(M_, 1)
    resid = epi == ts.TS_EPI_RESIDUAL
    c = torch.from_numpy(_randn(r, (M_, N))).to(DEV) if resid else \
        torch.empty(M_, N, dtype=torch.bfloat16, device=DEV)
    c0 = c[rows].cpu().numpy().astype(np.float64) if resid else 0.0
    a = torch.from_numpy(A).to(DEV, torch.bfloat16)
    b = torch.from_numpy(B).to(DEV, torch.bfloat16)
    # with the layers' workspace, as the forward calls run it (fc1, fc2 and out
    # split their partial last round of tiles along K)
    ws = torch.empty(ts.TS_GEMM_SPLIT_WS_BYTES, dtype=torch.uint8, device=DEV)
    ts.ts_op_gemm(ts.TS_BF16, epi, a, b, torch.from_numpy(bias).to(DEV), c, ws=ws)
    torch.cuda.synchronize()
    got = c[rows].float().cpu().numpy().astype(np.float64)
    ref = A[rows].astype(np.float64) @ B.astype(np.float64).T + bias
    if epi == ts.TS_EPI_BIAS_GELU:
        ref = M.gelu(ref)
    ref = ref + c0
    rms = np.sqrt(np.mean(ref * ref))
    if resid:
        # fp32 output: K-long fp32 accumulation, relative to the output scale
        bound = 1e-5 * rms
    else:
        # one round to nearest bf16 (half an ulp is at most 2^-8 of the value)
        bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    err = np.abs(got - ref)
    print(f"  max|err|/rms {err.max() / rms:.3e} over {len(rows)} rows x {N} columns")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name,N,K,epi", [("qkv", 3 * D, D, ts.TS_EPI_BIAS),
                                          ("fc2", D, DM, ts.TS_EPI_F32)])
def test_full_size_gemm_fp8(name, N, K, epi):
    """FP8 shared-layer GEMMs at the MiniMax-H3 fp8 shapes.  The per-tensor
    scales are over the whole operands, which the oracle sees whole; only the
    product is sampled."""
    M_ = M_SHARED
    say(f"full-size gemm fp8 {name} M={M_} N={N} K={K}")
    r = np.random.default_rng(N + K)
    A = round_bf16(_randn(r, (M_, K)))
    A[12345, 77] = 9.5                                  # a clear per-tensor maximum
    B = round_bf16(_randn(r, (N, K), 0.02))
    bias = _randn(r, (N,), 0.02)
    rows = _sample_rows(M_, 2, extra=(12345,))
    a = torch.from_numpy(A).to(DEV, torch.bfloat16)
    b = torch.from_numpy(B).to(DEV, torch.bfloat16)
    a8 = torch.empty(M_, K, dtype=torch.uint8, device=DEV)
    b8 = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    sc = torch.empty(2, dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    ts.ts_fp8_quantize(a, a8, sc[0:1], ws)
    ts.ts_fp8_quantize(b, b8, sc[1:2], ws)
    c = torch.empty(M_, N, dtype=torch.float32 if epi == ts.TS_EPI_F32 else torch.bfloat16, device=DEV)
    ts.ts_op_gemm(ts.TS_FP8E4M3, epi, a8, b8, torch.from_numpy(bias).to(DEV), c, sc[0:1], sc[1:2],
                  ws=torch.empty(ts.TS_GEMM_SPLIT_WS_BYTES, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    sa, sb = ofp8.tensor_scale(A), ofp8.tensor_scale(B)
    s_got = sc.cpu().numpy()
    assert s_got[0] == sa and s_got[1] == sb
    qa = ofp8.round_e4m3(A[rows] / sa)
    qb = ofp8.round_e4m3(B / sb)
    ref = (qa @ qb.T) * (np.float64(sa) * np.float64(sb)) + bias
    got = c[rows].float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    # same e4m3 codes on both sides; the MFMA sums the 64 products of one
    # instruction in one step, not with a rounding per add
    bound = (0 if epi == ts.TS_EPI_F32 else 2.0 ** -8 * np.abs(ref)) + 2e-4 * rms
    err = np.abs(got - ref)
    print(f"  max|err|/rms {err.max() / rms:.3e}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name", ["minimax_h3", "vitok4k"])
def test_full_size_attention_step(name):
    """The shared layers' attention step at the full workload size, in the
    launch configuration of a shared layer (qk_prep, the blended window kernel
    over every query block, the split global-row kernels), checked as the
    small cases are (test_gpu_kernels.check_attention) on whole query blocks:
    the first and last block of every window count and the last block."""
    from test_gpu_kernels import check_attention, run_attention_op
    base = configs.get(name)
    cfg = AC.case_cfg(base["ndim"], base["grid"], base["tile"], base["stride"], base["n_heads"],
                      base["head_dim"], base["qk_norm"], "bf16")
    say(f"full-size attention step {name} grid={cfg['grid']} tiles={cfg['tile']}")
    pl, qkv, q_g, k_g = AC.case_inputs(cfg, True, 1.0, seed=21)
    got, qkv_gpu = run_attention_op(cfg, pl, qkv, q_g, k_g, True)
    blocks = AR.query_blocks(pl)
    pick = set()
    for nt in sorted({len(t) for t, _ in blocks}):
        idx = [i for i, (t, _) in enumerate(blocks) if len(t) == nt]
        pick.update((idx[0], idx[-1]))
    pick.add(len(blocks) - 1)
    pick = sorted(pick)
    rows = np.concatenate([blocks[i][1] for i in pick])
    ref_rows = AC.oracle_attention_rows(qkv, cfg, pl, rows, q_g, k_g)
    ref = np.full_like(got, np.nan)
    ref[rows] = ref_rows[:len(rows)]
    ref[pl.n_union:] = ref_rows[len(rows):]
    sel = np.concatenate([rows, pl.n_union + np.arange(pl.n_tiles)])
    e = check_attention(cfg, pl, qkv, q_g, k_g, True, got, qkv_gpu, ref, emu_blocks=pick, rows=sel)
    print(f"  {len(pick)} blocks ({len(rows)} rows) + {pl.n_tiles} global rows: max|gpu-oracle|/rms {e:.3e}")
    assert e < AC.CAP[1.0]


FULL_LAYER = ["minimax_h3", "small_video", "vitok4k"]


def _full_inputs(name):
    cfg = dict(configs.get(name), n_layers=1)
    x, g, layers = make_inputs(cfg, n_layers=1)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    return cfg, x, g, layers, pl


@pytest.mark.parametrize("name", FULL_LAYER)
def test_full_size_shared_layer(name):
    cfg, x, g, layers, pl = _full_inputs(name)
    say(f"full-size shared layer {name} n_union={pl.n_union} tiles={pl.n_tiles}")
    rng = np.random.default_rng(4)
    G = (np.tile(g[None], (pl.n_tiles, 1)) + 0.1 * _randn(rng, (pl.n_tiles, cfg["d"]))).astype(np.float32)
    xa = np.vstack([x, G])
    run = Run(cfg, layers)
    try:
        got = run.shared_layer(xa)
    finally:
        run.close()
    sel = _union_sample(pl, 8)
    rx, rg = M.shared_layer_rows(x.astype(np.float64), G.astype(np.float64), layers[0], cfg, pl,
                                 M.Rope(pl, cfg), sel)
    ex, eg = max_rel(got[sel], rx), max_rel(got[pl.n_union:], rg)
    # the layer's own contribution, without the residual input
    ed = max_rel(got[sel] - x[sel], rx - x[sel])
    print(f"  sampled {len(sel)} rows: out {ex:.3e}, globals {eg:.3e}, layer delta {ed:.3e}")
    tol = TOL[cfg["dtype"]]
    assert ex < tol and eg < tol and ed < tol


@pytest.mark.parametrize("name,per_tile", [("minimax_h3", False), ("minimax_h3", True), ("small_video", False),
                                           ("vitok4k", False)])
def test_full_size_global_rows_attention(name, per_tile):
    """The global-token rows' attention at full size, on its own: with the MLP
    and the out-projection bias zero, a global row's layer delta is its
    attention output (over the n window keys and the global key) times W_o.
    Checked per row against the oracle, to the attention bound."""
    cfg, x, g, layers, pl = _full_inputs(name)
    for k in ("w_1", "b_1", "w_2", "b_2", "b_o"):
        layers[0][k] = np.zeros_like(layers[0][k])
    say(f"full-size global rows {name} per_tile={per_tile} tiles={pl.n_tiles} n={pl.tile_tokens}")
    run = Run(cfg, layers)
    try:
        if per_tile:
            G = np.tile(g[None], (pl.n_tiles, 1)).astype(np.float32)
            _, got = run.stack(x, g, 1)
            _, ref = M.tiled_layer_rows(cfg, pl, x, g, layers[0], [0])
        else:
            rng = np.random.default_rng(6)
            G = (np.tile(g[None], (pl.n_tiles, 1)) + 0.1 * _randn(rng, (pl.n_tiles, cfg["d"]))).astype(np.float32)
            got = run.shared_layer(np.vstack([x, G]))[pl.n_union:]
            _, ref = M.shared_layer_rows(x.astype(np.float64), G.astype(np.float64), layers[0], cfg, pl,
                                         M.Rope(pl, cfg), [0])
    finally:
        run.close()
    dg, dr = got - G, ref - G
    err = np.linalg.norm(dg - dr, axis=1) / np.linalg.norm(dr, axis=1)
    print("  per-row rel-L2 of the global deltas: " + " ".join(f"{v:.1e}" for v in err))
    assert np.all(err < 2e-2)


def test_full_size_tiled_layer_and_merge():
    cfg, x, g, layers, pl = _full_inputs("minimax_h3")
    say(f"full-size per-tile layer + merge minimax_h3 tiles={pl.n_tiles} n={pl.tile_tokens}")
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, 1)
    finally:
        run.close()
    sel = _union_sample(pl, 9)
    rx, rg = M.tiled_layer_rows(cfg, pl, x, g, layers[0], sel)
    ex, eg = max_rel(got[sel], rx), max_rel(ggot, rg)
    ed = max_rel(got[sel] - x[sel], rx - x[sel])
    print(f"  sampled {len(sel)} rows: out {ex:.3e}, globals {eg:.3e}, layer delta {ed:.3e}")
    tol = TOL[cfg["dtype"]]
    assert ex < tol and eg < tol and ed < tol


def test_full_size_stack_is_deterministic_and_finite():
    """TileShare-6 over seven MiniMax-H3-scale layers (six per tile, the merge,
    one shared), twice: results are bit-identical and finite."""
    cfg = dict(MINIMAX, n_layers=7)
    say("full-size stack minimax_h3 L=7 k=6, twice")
    x, g, layers = make_inputs(cfg, n_layers=7)
    run = Run(cfg, layers)
    try:
        a, ga = run.stack(x, g, 6)
        b, gb = run.stack(x, g, 6)
    finally:
        run.close()
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(ga))
    assert np.array_equal(a, b) and np.array_equal(ga, gb)


@pytest.mark.parametrize("name", ["minimax_h3", "small_video"])
@pytest.mark.parametrize("rows_kernel", [True, False])
def test_full_size_layer0_dedup_matches_per_tile_rows(name, rows_kernel, monkeypatch):
    """Table S1, layer 0 at full size: a one-layer tiled decoder with layer 0's
    Norm1, QKV and QK-norm once per token and attention through the tile map
    equals the per-tile layer 0.  Without the ragged-row GEMM the two are
    bit-identical (the same kernels on the same values); with it, the few rows
    it takes differ between the layouts in summation order, so a bf16 q, k or
    v value there can round one unit apart (2^-8 relative), which moves the
    layer output by less than that."""
    if not rows_kernel:
        monkeypatch.setenv("TS_GEMM_ROWS", "never")
    cfg, x, g, layers, pl = _full_inputs(name)
    say(f"full-size layer-0 dedup {name} rows_kernel={rows_kernel} n_union={pl.n_union} tiles={pl.n_tiles}")
    outs = {}
    for dd in (False, True):
        run = Run(dict(cfg, layer0_dedup=dd), layers)
        try:
            outs[dd] = run.stack(x, g, 1)
        finally:
            run.close()
    e = max(max_rel(outs[True][0], outs[False][0]), max_rel(outs[True][1], outs[False][1]))
    print(f"  max|diff|/rms against the per-tile layer 0: {e:.3e}")
    assert np.all(np.isfinite(outs[True][0]))
    if rows_kernel:
        assert e < 2.0 ** -8
    else:
        assert np.array_equal(outs[True][0], outs[False][0]) and np.array_equal(outs[True][1], outs[False][1])
