"""GPU parity of the shared layer, the TileShare-k stack and the tiled baseline
against the oracle, on seeded inputs at sizes the oracle finishes in seconds
(several tiles, ragged query and key blocks), plus the invariants of the
pages checked GPU-against-GPU at the same sizes."""
import numpy as np
import pytest

from oracle import model as M
from oracle.plan import Plan
from synth import configs, make_inputs

from gpu_helpers import TOL, Run, max_rel, say

pytestmark = pytest.mark.gpu

# Reduced-size versions of the workloads: same block type, head size, norm and
# tiling pattern (overlap, clamped last tile), fewer tokens / channels / layers.
REDUCED = {
    "minimax_h3": dict(grid=(2, 12, 20), tile=(2, 8, 8), stride=(2, 6, 6), d=256, n_heads=2, mlp_hidden=1024,
                       n_layers=3),
    "minimax_h3_fp8": dict(grid=(2, 12, 20), tile=(2, 8, 8), stride=(2, 6, 6), d=256, n_heads=2,
                           mlp_hidden=1024, n_layers=3),
    "small_video": dict(grid=(2, 12, 28), tile=(2, 12, 12), stride=(2, 8, 8), d=256, n_heads=4, mlp_hidden=1024,
                        n_layers=2),
    "vitok4k": dict(grid=(1, 20, 36), tile=(1, 16, 16), stride=(1, 12, 12), d=256, n_heads=4, mlp_hidden=1024,
                    n_layers=2),
    "vitok4k_enc": dict(grid=(1, 20, 36), tile=(1, 16, 16), stride=(1, 12, 12), d=256, n_heads=4, mlp_hidden=1024,
                        n_layers=2),
}


def reduced(name):
    return configs.get(name, **REDUCED[name])


def _oracle(cfg, x, g, layers, k):
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"], blend=cfg.get("blend", "ramp"))
    return M.stack_forward(cfg, pl, x, g, layers, k)


CASES = [("tiny2d", None, 0), ("tiny2d", None, 1),
         ("minimax_h3", "r", 0), ("minimax_h3", "r", 1), ("minimax_h3", "r", 3),
         ("minimax_h3_fp8", "r", 0), ("minimax_h3_fp8", "r", 1),
         ("small_video", "r", 0), ("small_video", "r", 2),
         ("vitok4k", "r", 0), ("vitok4k", "r", 2)]


@pytest.mark.parametrize("name,size,k", CASES)
@pytest.mark.parametrize("qk_scale", [1.0, 4.0, 8.0])
def test_stack_against_oracle(name, size, k, qk_scale):
    cfg = configs.get(name) if size is None else reduced(name)
    say(f"stack {name} {'reduced' if size else 'full'} k={k} qk_scale={qk_scale} grid={cfg['grid']}")
    x, g, layers = make_inputs(cfg, qk_scale=qk_scale)
    ref, gref = _oracle(cfg, x, g, layers, k)
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, k)
    finally:
        run.close()
    tol = TOL["fp8" if cfg["gemm_shared"] == "fp8" and k < cfg["n_layers"] else cfg["dtype"]]
    e = max_rel(got, ref)
    eg = max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


@pytest.mark.parametrize("name", ["minimax_h3", "minimax_h3_fp8"])
def test_stack_with_padded_hidden_rows(name):
    # a bf16 MLP hidden row of 4 KB (2048 channels) is stored at a padded
    # pitch, written by fc1 and read by fc2 with it; an fp8 fc2 (the shared
    # layers of the fp8 workload) takes the hidden unpadded
    cfg = configs.get(name, **dict(REDUCED[name], mlp_hidden=2048, n_layers=2))
    say(f"stack {name} reduced, hidden 2048, k=1")
    x, g, layers = make_inputs(cfg)
    ref, gref = _oracle(cfg, x, g, layers, 1)
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, 1)
    finally:
        run.close()
    tol = TOL["fp8" if cfg["gemm_shared"] == "fp8" else cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


@pytest.mark.parametrize("name", ["minimax_h3", "vitok4k", "tiny2d"])
def test_shared_layer_against_oracle(name):
    cfg = configs.get(name) if name == "tiny2d" else reduced(name)
    say(f"shared layer {name}")
    x, g, layers = make_inputs(cfg, n_layers=1)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    rng = np.random.default_rng(5)
    G = (np.tile(g[None], (pl.n_tiles, 1)) + 0.1 * rng.standard_normal((pl.n_tiles, cfg["d"]))).astype(np.float32)
    xa = np.vstack([x, G]).astype(np.float32)
    ref_x, ref_g = M.shared_layer(x.astype(np.float64), G.astype(np.float64), layers[0], cfg, pl, M.Rope(pl, cfg))
    run = Run(dict(cfg, n_layers=1), layers)
    try:
        got = run.shared_layer(xa)
    finally:
        run.close()
    tol = TOL[cfg["dtype"]]
    assert max_rel(got[: pl.n_union], ref_x) < tol
    assert max_rel(got[pl.n_union:], ref_g) < tol


def test_repeat_runs_are_bit_identical():
    cfg = reduced("minimax_h3")
    say("determinism minimax_h3 reduced")
    x, g, layers = make_inputs(cfg)
    run = Run(cfg, layers)
    try:
        a, ga = run.stack(x, g, 1)
        b, gb = run.stack(x, g, 1)
    finally:
        run.close()
    assert np.array_equal(a, b) and np.array_equal(ga, gb)


@pytest.mark.parametrize("name", ["minimax_h3", "small_video"])
def test_zero_overlap_every_k_matches_baseline_on_gpu(name):
    """Figure 2 caption: the blend is the only approximate step, so without
    overlap TileShare-k equals per-tile decoding for every k."""
    base = reduced(name)
    T = base["grid"][0]
    cfg = dict(base, grid=(T, 8, 24), tile=(T, 8, 8), stride=(T, 8, 8))
    say(f"zero overlap {name}")
    x, g, layers = make_inputs(cfg)
    run = Run(cfg, layers)
    try:
        ref, _ = run.stack(x, g, cfg["n_layers"])
        for k in range(cfg["n_layers"]):
            got, _ = run.stack(x, g, k)
            assert max_rel(got, ref) < 1e-5
    finally:
        run.close()


def test_identical_states_blend_to_themselves_on_gpu():
    """Table 1 caption: identical per-tile states stay identical.  With W_v = 0
    and b_v = 0 every tile's state of a token is the same, so TileShare-0
    equals the tiled baseline up to the fp32 rounding of w-bar."""
    cfg = reduced("small_video")
    say("identical states small_video reduced")
    x, g, layers = make_inputs(cfg)
    d = cfg["d"]
    for p in layers:
        p["w_qkv"][2 * d:] = 0
        p["b_qkv"][2 * d:] = 0
    run = Run(cfg, layers)
    try:
        base, _ = run.stack(x, g, cfg["n_layers"])
        ts0, _ = run.stack(x, g, 0)
    finally:
        run.close()
    assert max_rel(ts0, base) < 1e-5


HARD = [("tiny2d", None, 0), ("minimax_h3", "r", 0), ("minimax_h3", "r", 1), ("vitok4k", "r", 0)]


@pytest.mark.parametrize("name,size,k", HARD)
def test_hard_stitching_stack_against_oracle(name, size, k):
    """Hard stitching (Table 2 / Table S2): the same kernels with a one-hot
    w-bar from the plan."""
    cfg = dict(configs.get(name) if size is None else reduced(name), blend="hard")
    say(f"hard stitching stack {name} k={k}")
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    ref, gref = _oracle(cfg, x, g, layers, k)
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, k)
    finally:
        run.close()
    tol = TOL["fp8" if cfg["gemm_shared"] == "fp8" and k < cfg["n_layers"] else cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


MERGE_ONCE = [("tiny2d", None, 0), ("tiny2d", None, 1), ("minimax_h3", "r", 1), ("minimax_h3", "r", 2),
              ("small_video", "r", 1), ("vitok4k", "r", 1)]


@pytest.mark.parametrize("name,size,l", MERGE_ONCE)
def test_merge_once_against_oracle(name, size, l):
    """Figure 3b: merge the per-tile states once at layer l, then continue per tile."""
    cfg = configs.get(name) if size is None else reduced(name)
    say(f"merge once {name} l={l}")
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    ref, gref = M.merge_once_forward(cfg, pl, x, g, layers, l)
    run = Run(cfg, layers)
    try:
        got, ggot = run.merge_once(x, g, l)
    finally:
        run.close()
    tol = TOL[cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


FP8_SCOPE = [
    # (k, fp8 GEMMs, per-tile layers too): the tiled decoder with fp8 MLPs
    # ("FP8 MLP layers only"), TileShare with fp8 MLPs in every layer, and
    # TileShare with all four GEMMs fp8 in shared layers only
    (3, ("fc1", "fc2"), True),
    (1, ("fc1", "fc2"), True),
    (1, ("qkv", "out", "fc1", "fc2"), False),
    (0, ("out", "fc2"), False),
]


@pytest.mark.parametrize("k,gemms,per_tile", FP8_SCOPE)
def test_fp8_scope_against_oracle(k, gemms, per_tile):
    """Table S2 ("FP8 MLP layers only", "TileShare-4 + FP8") and Table S5
    ("V0 + FP8"): which GEMMs run in e4m3, and whether per-tile layers do."""
    cfg = dict(reduced("minimax_h3_fp8"), fp8_gemms=gemms, fp8_per_tile=per_tile)
    say(f"fp8 scope k={k} gemms={gemms} per_tile={per_tile}")
    x, g, layers = make_inputs(cfg)
    ref, gref = _oracle(cfg, x, g, layers, k)
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, k)
    finally:
        run.close()
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {TOL['fp8']}")
    assert e < TOL["fp8"] and eg < TOL["fp8"]


@pytest.mark.parametrize("k,gemms,per_tile", [(1, ("qkv", "out", "fc1", "fc2"), False),
                                              (1, ("fc1", "fc2"), True), (0, ("out", "fc2"), False)])
@pytest.mark.parametrize("rows_kernel", [False, True])
def test_fp8_fused_amax_bit_identical(k, gemms, per_tile, rows_kernel, monkeypatch):
    """The fp8 operand's max |value| taken by its producer (norm, blend, the
    fc1 epilogue, and the ragged-row GEMM kernel when rows_kernel) gives the
    same outputs, bit for bit, as the separate max pass (TS_FP8_SEPARATE_AMAX=1):
    the max of the same stored values does not depend on the order."""
    cfg = dict(reduced("minimax_h3_fp8"), fp8_gemms=gemms, fp8_per_tile=per_tile)
    say(f"fp8 fused amax k={k} gemms={gemms} per_tile={per_tile} rows_kernel={rows_kernel}")
    if rows_kernel:
        monkeypatch.setenv("TS_GEMM_ROWS", "always")
    x, g, layers = make_inputs(cfg)
    outs = []
    for separate in (False, True):
        if separate:
            monkeypatch.setenv("TS_FP8_SEPARATE_AMAX", "1")
        else:
            monkeypatch.delenv("TS_FP8_SEPARATE_AMAX", raising=False)
        run = Run(cfg, layers)
        try:
            outs.append(run.stack(x, g, k))
        finally:
            run.close()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


PARTIAL = [("tiny2d", None, 0, "o"), ("tiny2d", None, 0, "qm"),
           ("minimax_h3", "r", 1, "q"), ("minimax_h3", "r", 1, "o"), ("minimax_h3", "r", 1, "m"),
           ("minimax_h3", "r", 0, "qo"), ("minimax_h3", "r", 1, "qom"), ("minimax_h3", "r", 2, ""),
           ("vitok4k", "r", 0, "om"), ("small_video", "r", 1, "qm")]


@pytest.mark.parametrize("name,size,k,share", PARTIAL)
def test_partial_sharing_against_oracle(name, size, k, share):
    """Table 1 (top) and Table S7: per-tile residual streams from layer k with
    the listed operations (q: Norm1/QKV/QK-norm, o: out-projection, m: MLP)
    run once per token on the blended state."""
    cfg = configs.get(name) if size is None else reduced(name)
    say(f"partial sharing {name} k={k} share={share!r}")
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    ref, gref = M.partial_share_forward(cfg, pl, x, g, layers, k, set(share))
    run = Run(cfg, layers)
    try:
        got, ggot = run.partial_share(x, g, k, set(share))
    finally:
        run.close()
    tol = TOL[cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


DEDUP = [("stack", "tiny2d", None, 1), ("stack", "minimax_h3", "r", 1), ("stack", "minimax_h3", "r", 3),
         ("stack", "small_video", "r", 2), ("stack", "vitok4k", "r", 1), ("stack", "minimax_h3_fp8", "r", 1),
         ("merge_once", "minimax_h3", "r", 0), ("merge_once", "minimax_h3", "r", 2),
         ("partial", "minimax_h3", "r", 1)]


@pytest.mark.parametrize("entry,name,size,k", DEDUP)
def test_layer0_dedup_against_oracle_and_per_tile_rows(entry, name, size, k):
    """Table S1, layer 0: Norm1, QKV and QK-norm once per token (every tile
    holds copies of the same rows) and attention through the tile map give
    the per-tile layer 0's result: against the oracle (which runs layer 0 per
    tile) to the usual bound, and against the same GPU entry point without the
    dedup to rounding."""
    cfg = configs.get(name) if size is None else reduced(name)
    say(f"layer-0 dedup {entry} {name} k={k}")
    x, g, layers = make_inputs(cfg, qk_scale=2.0)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    if entry == "stack":
        ref, gref = _oracle(cfg, x, g, layers, k)
    elif entry == "merge_once":
        ref, gref = M.merge_once_forward(cfg, pl, x, g, layers, k)
    else:
        ref, gref = M.partial_share_forward(cfg, pl, x, g, layers, k, {"q"})
    outs = {}
    for dd in (False, True):
        run = Run(dict(cfg, layer0_dedup=dd), layers)
        try:
            if entry == "stack":
                outs[dd] = run.stack(x, g, k)
            elif entry == "merge_once":
                outs[dd] = run.merge_once(x, g, k)
            else:
                outs[dd] = run.partial_share(x, g, k, {"q"})
        finally:
            run.close()
    (got, ggot), (plain, gplain) = outs[True], outs[False]
    tol = TOL["fp8" if cfg["gemm_shared"] == "fp8" and k < cfg["n_layers"] else cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    ep = max(max_rel(got, plain), max_rel(ggot, gplain))
    print(f"  max|err|/rms = {e:.3e} (globals {eg:.3e}), tolerance {tol}; against per-tile rows {ep:.3e}")
    assert e < tol and eg < tol
    # the same kernels on the same values: equal up to the summation order of
    # rows that fall into the ragged-row GEMM in one layout and not the other
    assert ep < 1e-3


@pytest.mark.parametrize("k_enc,k_dec", [(0, 0), (2, 2), (0, 1)])
def test_encoder_then_decoder(k_enc, k_dec):
    """TileShare also in the encoder (paper page, Tables S11 and S12, "+enc"):
    the encoder stack's output rows are the decoder's input tokens.  Each
    stack is held to the per-stack tolerance: the encoder against the oracle
    on the same inputs, the decoder against the oracle fed the GPU encoder's
    output; the end-to-end difference is reported."""
    enc, dec = reduced("vitok4k_enc"), reduced("vitok4k")
    say(f"pipeline encoder k={k_enc} then decoder k={k_dec} grid={dec['grid']}")
    xe, g, le = make_inputs(enc)
    _, _, ld = make_inputs(dec)
    run_e, run_d = Run(enc, le), Run(dec, ld)
    try:
        lat, _ = run_e.stack(xe, g, k_enc)
        got, ggot = run_d.stack(lat, g, k_dec)
    finally:
        run_e.close()
        run_d.close()
    ref_lat, _ = _oracle(enc, xe, g, le, k_enc)
    ref, gref = _oracle(dec, lat, g, ld, k_dec)
    end, _ = _oracle(dec, ref_lat, g, ld, k_dec)
    tol = TOL[dec["dtype"]]
    e_enc, e_dec, eg = max_rel(lat, ref_lat), max_rel(got, ref), max_rel(ggot, gref)
    print(f"  encoder {e_enc:.3e}, decoder {e_dec:.3e} (globals {eg:.3e}), end to end {max_rel(got, end):.3e}; "
          f"tolerance {tol} per stack")
    assert e_enc < tol and e_dec < tol and eg < tol
