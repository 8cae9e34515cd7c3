"""Pins for the oracle's block, shared layer and TileShare-k stack (CPU).

Each pin checks the oracle against something other than itself: torch's own
norm / attention / GELU routines, a per-token brute-force formulation, or an
invariant the pages fix (Figure 2 caption: the blend is the only approximate
step; Table 1 caption: identical per-tile states stay identical; abstract:
TileShare-k with every layer per tile is the released tiled decoder).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import model as M
from oracle.brute import brute_per_tile_layer, brute_shared_layer
from oracle.plan import Plan, rope_pairs
from synth import configs, make_inputs

torch.set_default_dtype(torch.float64)


def tiny_cfg(ndim=2, norm="ln", qk=False, grid=(1, 4, 6), tile=(1, 4, 4), stride=(1, 2, 2),
             d=8, heads=2, layers=2, dtype="f32", mlp=16):
    return dict(name="tiny", ndim=ndim, grid=grid, tile=tile, stride=stride, n_layers=layers,
                d=d, n_heads=heads, head_dim=d // heads, mlp_hidden=mlp, norm=norm,
                qk_norm=qk, dtype=dtype, gemm_shared=dtype, seed=3)


# --- library-routine pins ---------------------------------------------------

def test_norms_gelu_attention_against_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 12))
    g = 1 + 0.1 * rng.standard_normal(12)
    b = 0.1 * rng.standard_normal(12)
    tx = torch.from_numpy(x)
    assert np.allclose(M.layer_norm(x, g, b, 1e-6),
                       Fn.layer_norm(tx, (12,), torch.from_numpy(g), torch.from_numpy(b), 1e-6).numpy(),
                       atol=1e-13, rtol=0)
    assert np.allclose(M.rms_norm(x, g, 1e-6),
                       Fn.rms_norm(tx, (12,), torch.from_numpy(g), 1e-6).numpy(), atol=1e-13, rtol=0)
    assert np.allclose(M.gelu(x), Fn.gelu(tx, approximate="none").numpy(), atol=1e-14, rtol=0)
    # exact GELU closed forms
    assert M.gelu(np.array([0.0]))[0] == 0.0
    assert math.isclose(M.gelu(np.array([1.0]))[0], 0.5 * (1 + math.erf(1 / math.sqrt(2))), rel_tol=1e-15)
    q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
    ref = Fn.scaled_dot_product_attention(*(torch.from_numpy(a)[None, None] for a in (q, k, v)))[0, 0]
    assert np.allclose(M.softmax_attention(q, k, v, 0.5), ref.numpy(), atol=1e-13, rtol=0)


def _torch_rope(x, pos, counts, base):
    """RoPE through complex multiplication (torch), independent of the oracle's pair loop."""
    n, hd = x.shape
    freqs = torch.cat([base ** (-torch.arange(m, dtype=torch.float64) / m) for m in counts if m])
    axes = torch.cat([torch.full((m,), ax, dtype=torch.long) for ax, m in enumerate(counts) if m])
    ang = pos[:, axes].to(torch.float64) * freqs[None, :]
    # the oracle stores cos/sin rounded to fp32; do the same
    c = torch.cos(ang).to(torch.float32).to(torch.float64)
    s = torch.sin(ang).to(torch.float32).to(torch.float64)
    z = torch.complex(c, s)
    xc = torch.view_as_complex(x.reshape(n, hd // 2, 2).contiguous())
    return torch.view_as_real(xc * z).reshape(n, hd)


def _torch_vit(cfg, X, layers, pos):
    """Textbook pre-norm ViT on one window with torch ops; last row is the global token."""
    d, H, hd = cfg["d"], cfg["n_heads"], cfg["head_dim"]
    counts = rope_pairs(cfg["ndim"], hd)
    X = torch.from_numpy(X)
    pos = torch.from_numpy(pos)
    n = X.shape[0]
    for p in layers:
        tp = {k: torch.from_numpy(v.astype(np.float64)) for k, v in p.items()}

        def nrm(x, w):
            if cfg["norm"] == "ln":
                return Fn.layer_norm(x, (d,), tp[w + "_g"], tp[w + "_b"], 1e-6)
            return Fn.rms_norm(x, (d,), tp[w + "_g"], 1e-6)
        h = nrm(X, "norm1")
        qkv = Fn.linear(h, tp["w_qkv"], tp["b_qkv"])
        q, k, v = qkv.split(d, dim=1)
        q = q.reshape(n, H, hd)
        k = k.reshape(n, H, hd)
        if cfg["qk_norm"]:
            q = Fn.rms_norm(q, (hd,), tp["q_g"], 1e-6)
            k = Fn.rms_norm(k, (hd,), tp["k_g"], 1e-6)
        qs, ks = [], []
        for hh in range(H):
            qh = torch.cat([_torch_rope(q[:-1, hh], pos, counts, 10000.0), q[-1:, hh]])
            kh = torch.cat([_torch_rope(k[:-1, hh], pos, counts, 10000.0), k[-1:, hh]])
            qs.append(qh)
            ks.append(kh)
        qh = torch.stack(qs)[None]
        kh = torch.stack(ks)[None]
        vh = v.reshape(n, H, hd).transpose(0, 1).contiguous()[None]
        o = Fn.scaled_dot_product_attention(qh, kh, vh)[0].transpose(0, 1).reshape(n, d)
        X = X + Fn.linear(o, tp["w_o"], tp["b_o"])
        u = Fn.gelu(Fn.linear(nrm(X, "norm2"), tp["w_1"], tp["b_1"]), approximate="none")
        X = X + Fn.linear(u, tp["w_2"], tp["b_2"])
    return X.numpy()


@pytest.mark.parametrize("ndim,norm,qk", [(2, "ln", False), (3, "rms", True), (3, "ln", False)])
def test_single_tile_equals_textbook_vit(ndim, norm, qk):
    grid = (1, 4, 6) if ndim == 2 else (2, 3, 4)
    cfg = tiny_cfg(ndim=ndim, norm=norm, qk=qk, grid=grid, tile=grid, stride=grid, d=16, heads=2)
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    assert pl.n_tiles == 1
    X = np.vstack([x[pl.tile_rows[0]], g[None]]).astype(np.float64)
    ref = _torch_vit(cfg, X, layers, pl.local_pos)
    for k in (0, 1, 2):
        out, G = M.stack_forward(cfg, pl, x, g, layers, k)
        back = np.empty_like(out)
        back[pl.tile_rows[0]] = out[pl.tile_rows[0]]
        assert np.allclose(out[pl.tile_rows[0]], ref[:-1], atol=1e-11, rtol=0)
        assert np.allclose(G[0], ref[-1], atol=1e-11, rtol=0)


# --- invariants the pages fix ---------------------------------------------

@pytest.mark.parametrize("ndim,norm,qk", [(2, "ln", False), (3, "rms", True)])
def test_k_equals_L_is_tiled_baseline(ndim, norm, qk):
    grid, tile, stride = ((1, 6, 9), (1, 4, 4), (1, 2, 3)) if ndim == 2 else ((2, 5, 6), (2, 3, 4), (1, 2, 2))
    cfg = tiny_cfg(ndim=ndim, norm=norm, qk=qk, grid=grid, tile=tile, stride=stride)
    x, g, layers = make_inputs(cfg)
    pl = Plan(grid, tile, stride)
    a, ga = M.stack_forward(cfg, pl, x, g, layers, len(layers))
    b, gb = M.tiled_forward(cfg, pl, x, g, layers)
    assert np.array_equal(a, b) and np.array_equal(ga, gb)


@pytest.mark.parametrize("ndim", [2, 3])
def test_zero_overlap_every_k_equals_baseline(ndim):
    grid, tile = ((1, 4, 8), (1, 4, 4)) if ndim == 2 else ((2, 4, 6), (2, 2, 3))
    cfg = tiny_cfg(ndim=ndim, norm="rms" if ndim == 3 else "ln", qk=ndim == 3,
                   grid=grid, tile=tile, stride=tile, layers=3)
    x, g, layers = make_inputs(cfg)
    pl = Plan(grid, tile, tile)
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    for k in range(4):
        out, _ = M.stack_forward(cfg, pl, x, g, layers, k)
        assert M.rel_err(out, base) < 1e-12
    # but the global tokens differ per tile, so they are not merged
    _, G = M.stack_forward(cfg, pl, x, g, layers, 0)
    assert not np.allclose(G[0], G[1])


def test_identical_per_tile_states_stay_identical():
    """With W_v = 0 and b_v = 0 attention adds only b_o, so a token's state is the
    same in every tile; TileShare-0 then equals the tiled baseline to rounding."""
    cfg = tiny_cfg(ndim=2, grid=(1, 5, 9), tile=(1, 4, 5), stride=(1, 1, 2), layers=3)
    x, g, layers = make_inputs(cfg)
    d = cfg["d"]
    for p in layers:
        p["w_qkv"][2 * d:] = 0
        p["b_qkv"][2 * d:] = 0
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    for k in range(4):
        out, _ = M.stack_forward(cfg, pl, x, g, layers, k)
        assert M.rel_err(out, base) < 1e-6     # fp32-rounded w-bar sums to 1 within ~1e-7


def test_overlap_makes_tileshare_differ():
    """Control for the two pins above: with overlap and W_v != 0 the blend is approximate."""
    cfg = tiny_cfg(ndim=2, grid=(1, 5, 9), tile=(1, 4, 5), stride=(1, 1, 2), layers=2)
    x, g, layers = make_inputs(cfg, qk_scale=4.0)
    for p in layers:     # N(0, 0.02) at d = 8 leaves the attention branch tiny
        for key in ("w_qkv", "w_o"):
            p[key] *= 20
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    out, _ = M.stack_forward(cfg, pl, x, g, layers, 0)
    assert M.rel_err(out, base) > 1e-2


def test_blend_before_or_after_out_projection():
    cfg = tiny_cfg(ndim=3, norm="rms", qk=True, grid=(2, 5, 6), tile=(2, 3, 4), stride=(1, 2, 2))
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rope = M.Rope(pl, cfg)
    G = np.tile(g[None].astype(np.float64), (pl.n_tiles, 1))
    a, ga = M.shared_layer(x.astype(np.float64), G, layers[0], cfg, pl, rope)
    b, gb = M.shared_layer(x.astype(np.float64), G, layers[0], cfg, pl, rope, blend_after_out=True)
    # equal up to the fp32 rounding of w-bar (sum 1 within a few 1e-8)
    assert M.rel_err(b, a) < 1e-6 and M.rel_err(gb, ga) < 1e-6


def test_rope_relativity_in_shared_layer():
    """In a shared layer q and k are per token, so a pair of non-global tokens that
    sits in two tiles gets the same score in both (RoPE depends on differences)."""
    cfg = tiny_cfg(ndim=3, norm="rms", qk=True, grid=(2, 5, 6), tile=(2, 3, 4), stride=(1, 2, 2))
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rope = M.Rope(pl, cfg)
    h = M.norm(x.astype(np.float64), layers[0], "norm1", cfg)
    q, k, _ = M.qkv_heads(h, layers[0], cfg)
    hd = cfg["head_dim"]
    checked = 0
    for t1 in range(pl.n_tiles):
        for t2 in range(t1 + 1, pl.n_tiles):
            common = sorted(set(pl.tile_rows[t1].tolist()) & set(pl.tile_rows[t2].tolist()))
            if len(common) < 2:
                continue
            j1 = {int(p): j for j, p in enumerate(pl.tile_rows[t1])}
            j2 = {int(p): j for j, p in enumerate(pl.tile_rows[t2])}
            for a in common[:4]:
                for b in common[-4:]:
                    for hh in range(cfg["n_heads"]):
                        cs = slice(hh * hd, (hh + 1) * hd)
                        s = []
                        for jj in (j1, j2):
                            qa = M.rope_rotate(q[[a], cs], rope.cos[[jj[a]]], rope.sin[[jj[a]]])
                            kb = M.rope_rotate(k[[b], cs], rope.cos[[jj[b]]], rope.sin[[jj[b]]])
                            s.append((qa @ kb.T).item())
                        assert math.isclose(s[0], s[1], rel_tol=0, abs_tol=1e-5)
                        checked += 1
    assert checked > 0


# --- brute-force per-token loops --------------------------------------------

BRUTE = [
    dict(ndim=2, norm="ln", qk=False, grid=(1, 4, 6), tile=(1, 4, 4), stride=(1, 2, 2)),
    dict(ndim=3, norm="rms", qk=True, grid=(2, 3, 4), tile=(2, 2, 3), stride=(1, 1, 1)),
    dict(ndim=3, norm="ln", qk=False, grid=(3, 4, 4), tile=(2, 3, 3), stride=(1, 2, 2)),
]


@pytest.mark.parametrize("c", BRUTE)
def test_shared_layer_against_brute_force(c):
    cfg = tiny_cfg(ndim=c["ndim"], norm=c["norm"], qk=c["qk"], grid=c["grid"], tile=c["tile"],
                   stride=c["stride"], layers=1)
    x, g, layers = make_inputs(cfg, qk_scale=3.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rope = M.Rope(pl, cfg)
    G = np.tile(g[None].astype(np.float64), (pl.n_tiles, 1))
    G[0] += 0.5   # per-tile global rows that differ
    a, ga = M.shared_layer(x.astype(np.float64), G, layers[0], cfg, pl, rope)
    bx, bg = brute_shared_layer(x.astype(np.float64).tolist(), G.tolist(), layers[0], cfg,
                                cfg["grid"], cfg["tile"], cfg["stride"])
    assert np.allclose(a, np.array(bx), atol=1e-10, rtol=0)
    assert np.allclose(ga, np.array(bg), atol=1e-10, rtol=0)


@pytest.mark.parametrize("c", BRUTE)
def test_per_tile_layer_against_brute_force(c):
    cfg = tiny_cfg(ndim=c["ndim"], norm=c["norm"], qk=c["qk"], grid=c["grid"], tile=c["tile"],
                   stride=c["stride"], layers=1)
    x, g, layers = make_inputs(cfg, qk_scale=3.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rope = M.Rope(pl, cfg)
    X = M.gather_tiles(pl, x, g)
    for t in range(pl.n_tiles):
        a = M.per_tile_layer(X[t], layers[0], cfg, rope)
        b = brute_per_tile_layer(X[t].tolist(), layers[0], cfg, pl.extent)
        assert np.allclose(a, np.array(b), atol=1e-10, rtol=0)


def test_tiny2d_config_runs_and_differs_from_baseline():
    cfg = configs.get("tiny2d")
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, _ = M.stack_forward(cfg, pl, x, g, layers, 1)
    ts0, _ = M.stack_forward(cfg, pl, x, g, layers, 0)
    e = M.rel_err(ts0, base)
    assert np.all(np.isfinite(ts0)) and 0 < e < 1.0


# --- row-restricted evaluation (used for checks at the full workload sizes) --

ROWS_CASES = [
    dict(ndim=3, norm="rms", qk=True, grid=(2, 12, 20), tile=(2, 8, 8), stride=(2, 6, 6), d=16, heads=2),
    dict(ndim=2, norm="ln", qk=False, grid=(1, 20, 36), tile=(1, 16, 16), stride=(1, 12, 12), d=16, heads=2),
    dict(ndim=3, norm="ln", qk=False, grid=(3, 5, 6), tile=(2, 3, 4), stride=(1, 2, 3), d=8, heads=2),
]


def _rows_setup(c):
    cfg = tiny_cfg(ndim=c["ndim"], norm=c["norm"], qk=c["qk"], grid=c["grid"], tile=c["tile"],
                   stride=c["stride"], d=c["d"], heads=c["heads"], layers=1, mlp=2 * c["d"])
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rng = np.random.default_rng(9)
    # first, last, every multiply-covered kind, and random rows, unsorted
    counts = np.diff(pl.cover_ptr)
    sel = [pl.n_union - 1, 0]
    for c_ in sorted(set(counts.tolist())):
        sel.append(int(np.nonzero(counts == c_)[0][-1]))
    sel += rng.choice(pl.n_union, size=7, replace=False).tolist()
    return cfg, x, g, layers, pl, np.array(sel)


@pytest.mark.parametrize("c", ROWS_CASES)
def test_shared_layer_rows_equal_full_layer(c):
    cfg, x, g, layers, pl, sel = _rows_setup(c)
    rope = M.Rope(pl, cfg)
    G = np.tile(g[None].astype(np.float64), (pl.n_tiles, 1))
    G[-1] -= 0.25
    full_x, full_g = M.shared_layer(x.astype(np.float64), G, layers[0], cfg, pl, rope)
    rx, rg = M.shared_layer_rows(x.astype(np.float64), G, layers[0], cfg, pl, rope, sel)
    assert np.allclose(rx, full_x[sel], atol=1e-12, rtol=0)
    assert np.allclose(rg, full_g, atol=1e-12, rtol=0)


def test_shared_layer_rows_against_brute_force():
    c = BRUTE[2]
    cfg = tiny_cfg(ndim=c["ndim"], norm=c["norm"], qk=c["qk"], grid=c["grid"], tile=c["tile"],
                   stride=c["stride"], layers=1)
    x, g, layers = make_inputs(cfg, qk_scale=3.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    G = np.tile(g[None].astype(np.float64), (pl.n_tiles, 1))
    sel = np.array([5, 17, 0, pl.n_union - 1])
    rx, rg = M.shared_layer_rows(x.astype(np.float64), G, layers[0], cfg, pl, M.Rope(pl, cfg), sel)
    bx, bg = brute_shared_layer(x.astype(np.float64).tolist(), G.tolist(), layers[0], cfg,
                                cfg["grid"], cfg["tile"], cfg["stride"])
    assert np.allclose(rx, np.array(bx)[sel], atol=1e-10, rtol=0)
    assert np.allclose(rg, np.array(bg), atol=1e-10, rtol=0)


@pytest.mark.parametrize("c", ROWS_CASES)
def test_tiled_layer_rows_equal_one_layer_stack(c):
    cfg, x, g, layers, pl, sel = _rows_setup(c)
    full_x, full_g = M.stack_forward(cfg, pl, x, g, layers, 1)
    rx, rg = M.tiled_layer_rows(cfg, pl, x, g, layers[0], sel)
    assert np.allclose(rx, full_x[sel], atol=1e-12, rtol=0)
    assert np.allclose(rg, full_g, atol=1e-12, rtol=0)


def test_rows_functions_refuse_fp8():
    cfg = dict(tiny_cfg(layers=1), gemm_shared="fp8")
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    G = np.tile(g[None].astype(np.float64), (pl.n_tiles, 1))
    with pytest.raises(ValueError):
        M.shared_layer_rows(x, G, layers[0], cfg, pl, M.Rope(pl, cfg), [0])


# --- merging once at layer l, then per tile (Figure 3b) ----------------------

@pytest.mark.parametrize("ndim", [2, 3])
def test_merge_once_at_the_ends_is_the_tiled_decoder(ndim):
    """Merging at l = L merges the already-final states (a second merge of
    identical per-tile copies, which w-bar summing to 1 leaves unchanged);
    merging at l = 0 merges copies of the input.  Both equal the released
    tiled decoder up to the fp32 rounding of w-bar."""
    if ndim == 2:
        cfg = tiny_cfg(layers=3)
    else:
        cfg = tiny_cfg(ndim=3, norm="rms", qk=True, grid=(3, 5, 6), tile=(2, 3, 4), stride=(1, 2, 3), layers=3)
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, gbase = M.tiled_forward(cfg, pl, x, g, layers)
    for l in (0, 3):
        got, gg = M.merge_once_forward(cfg, pl, x, g, layers, l)
        assert M.rel_err(got, base) < 1e-6 and M.rel_err(gg, gbase) < 1e-6


def test_merge_once_without_overlap_is_the_tiled_decoder():
    cfg = tiny_cfg(grid=(1, 4, 8), tile=(1, 4, 4), stride=(1, 4, 4), layers=3)
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    for l in range(4):
        got, _ = M.merge_once_forward(cfg, pl, x, g, layers, l)
        assert np.array_equal(got, base)


def test_merge_once_in_the_middle_differs_and_keeps_global_rows_per_tile():
    cfg = tiny_cfg(layers=3)
    x, g, layers = make_inputs(cfg, qk_scale=3.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    got, gg = M.merge_once_forward(cfg, pl, x, g, layers, 1)
    assert 0 < M.rel_err(got, base) < 1.0
    assert gg.shape == (pl.n_tiles, cfg["d"]) and not np.allclose(gg[0], gg[1])
    # by hand: the merged state re-enters every tile
    rope = M.Rope(pl, cfg)
    X = M.gather_tiles(pl, x, g)
    X = [M.per_tile_layer(Xt, layers[0], cfg, rope) for Xt in X]
    xs, G = M.merge(pl, X)
    X2 = [np.vstack([xs[pl.tile_rows[t]], G[t][None]]) for t in range(pl.n_tiles)]
    for li in (1, 2):
        X2 = [M.per_tile_layer(Xt, layers[li], cfg, rope) for Xt in X2]
    ref, gref = M.merge(pl, X2)
    assert np.array_equal(got, ref) and np.array_equal(gg, gref)


# --- fp8 scope ------------------------------------------------------------------

def test_fp8_scope_selects_gemms_and_layers():
    cfg = dict(tiny_cfg(), gemm_shared="fp8")
    assert M.fp8_scope(cfg, True) == M.ALL_GEMMS and M.fp8_scope(cfg, False) == ()
    cfg2 = dict(cfg, fp8_gemms=("fc1", "fc2"), fp8_per_tile=True)
    assert M.fp8_scope(cfg2, True) == ("fc1", "fc2") == M.fp8_scope(cfg2, False)
    assert M.fp8_scope(dict(tiny_cfg(), fp8_per_tile=True), False) == ()
    assert M.f8(True, "qkv") and not M.f8(False, "qkv")
    assert M.f8(("fc1",), "fc1") and not M.f8(("fc1",), "out")


def test_batched_per_tile_layers_equal_per_tile_layers_in_bf16_and_fp8():
    """Without fp8 the batched form is the per-tile block row for row; with fp8
    it quantises each GEMM operand once over all tiles: a per-tile call with the
    scales of the batch gives the same rows."""
    cfg = tiny_cfg(ndim=3, norm="rms", qk=True, grid=(3, 5, 6), tile=(2, 3, 4), stride=(1, 2, 3), layers=1)
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rope = M.Rope(pl, cfg)
    X = M.gather_tiles(pl, x, g)
    a = M.per_tile_layers(X, layers[0], cfg, rope)
    for t in range(pl.n_tiles):
        assert np.allclose(a[t], M.per_tile_layer(X[t], layers[0], cfg, rope), atol=1e-12, rtol=0)
    # MLP-only fp8 on a batch of two identical tiles equals fp8 on one tile
    # (absmax and hence scales are unchanged by duplicating rows)
    Y = [X[0], X[0].copy()]
    b = M.per_tile_layers(Y, layers[0], cfg, rope, ("fc1", "fc2"))
    c = M.per_tile_layers([X[0]], layers[0], cfg, rope, ("fc1", "fc2"))
    assert np.allclose(b[0], c[0], atol=1e-12, rtol=0) and np.allclose(b[1], c[0], atol=1e-12, rtol=0)
    # and the MLP-only fp8 result differs from bf16 by a quantisation-sized amount
    e = M.rel_err(c[0], a[0])
    assert 1e-4 < e < 0.2


# --- partial sharing with per-tile residual streams (Table 1, Table S7) --------

def _ps_setup(layers=3, qk=3.0):
    cfg = tiny_cfg(ndim=3, norm="rms", qk=True, grid=(3, 5, 6), tile=(2, 3, 4), stride=(1, 2, 3), layers=layers)
    x, g, lay = make_inputs(cfg, qk_scale=qk)
    return cfg, x, g, lay, Plan(cfg["grid"], cfg["tile"], cfg["stride"])


@pytest.mark.parametrize("k", [0, 1, 3])
def test_partial_sharing_extremes(k):
    """Nothing shared is the tiled decoder; everything shared keeps the blended
    state on TileShare-k's path, so the final merge equals TileShare-k."""
    cfg, x, g, layers, pl = _ps_setup()
    base, gbase = M.tiled_forward(cfg, pl, x, g, layers)
    none, gnone = M.partial_share_forward(cfg, pl, x, g, layers, k, set())
    assert M.rel_err(none, base) < 1e-12 and M.rel_err(gnone, gbase) < 1e-12
    ts, gts = M.stack_forward(cfg, pl, x, g, layers, k)
    allx, gall = M.partial_share_forward(cfg, pl, x, g, layers, k, {"q", "o", "m"})
    # equal up to the fp32 rounding of w-bar: the broadcast deltas re-enter the
    # blend with weight sum 1 + O(2^-24)
    assert M.rel_err(allx, ts) < 1e-6 and M.rel_err(gall, gts) < 1e-6


@pytest.mark.parametrize("k", [0, 2])
def test_partial_sharing_q_plus_m_equals_all(k):
    """Table S7: sharing q and m is equivalent to sharing everything (the
    out-projection is linear and w-bar sums to 1, so only blends of it are
    ever read)."""
    cfg, x, g, layers, pl = _ps_setup()
    a, ga = M.partial_share_forward(cfg, pl, x, g, layers, k, {"q", "m"})
    b, gb = M.partial_share_forward(cfg, pl, x, g, layers, k, {"q", "o", "m"})
    assert M.rel_err(a, b) < 1e-6 and M.rel_err(ga, gb) < 1e-6


def test_partial_sharing_o_only_at_k0_is_tileshare0():
    """Table 1 footnote: with only the out-projection shared at k = 0 the
    per-tile states stay identical, so the result equals TileShare-0."""
    cfg, x, g, layers, pl = _ps_setup()
    a, ga = M.partial_share_forward(cfg, pl, x, g, layers, 0, {"o"})
    b, gb = M.stack_forward(cfg, pl, x, g, layers, 0)
    assert M.rel_err(a, b) < 1e-6 and M.rel_err(ga, gb) < 1e-6


def test_partial_sharing_single_ops_differ_and_zero_overlap_is_exact():
    cfg, x, g, layers, pl = _ps_setup()
    for p in layers:   # large enough layer updates that the approximation shows
        p["w_qkv"] = p["w_qkv"] * 20
        p["w_o"] = p["w_o"] * 20
        p["w_1"] = p["w_1"] * 10
    base, _ = M.tiled_forward(cfg, pl, x, g, layers)
    outs = {}
    for share in ({"q"}, {"o"}, {"m"}, {"q", "o"}):
        outs[tuple(sorted(share))], _ = M.partial_share_forward(cfg, pl, x, g, layers, 1, share)
        assert M.rel_err(outs[tuple(sorted(share))], base) > 1e-6
    assert M.rel_err(outs[("q",)], outs[("m",)]) > 1e-6
    cfg0 = tiny_cfg(grid=(1, 4, 8), tile=(1, 4, 4), stride=(1, 4, 4), layers=2)
    x0, g0, l0 = make_inputs(cfg0)
    p0 = Plan(cfg0["grid"], cfg0["tile"], cfg0["stride"])
    b0, _ = M.tiled_forward(cfg0, p0, x0, g0, l0)
    for share in ({"q"}, {"o"}, {"m"}, {"q", "o", "m"}):
        got, _ = M.partial_share_forward(cfg0, p0, x0, g0, l0, 0, share)
        assert M.rel_err(got, b0) < 1e-12
