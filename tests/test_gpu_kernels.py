"""GPU parity of the building-block kernels against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import shared_token_tiled_amd as ts
from oracle import fp8 as ofp8
from oracle import model as M
from oracle.plan import Plan
from synth import round_bf16

import attn_cases as AC
import attn_rounding as AR
from gpu_helpers import DEV, max_rel, say

pytestmark = pytest.mark.gpu


def _rng(seed):
    return np.random.default_rng(seed)


GEMM_SHAPES = [(300, 512, 320), (257, 768, 64), (1000, 256, 1024), (64, 16, 128), (513, 2304, 768),
               (300, 272, 4096)]


@pytest.mark.parametrize("M_,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype,ws", [("bf16", False), ("bf16", True), ("f32", False)])
def test_gemm_against_oracle(M_, N, K, epi, dtype, ws):
    """ws: with the workspace, the tiles of a partial last round of a long-K
    GEMM run K-split (here every shape is one partial round; (300, 272, 4096),
    64 K blocks, splits its 4 tiles 8 ways, the others are too short in K)."""
    say(f"gemm {dtype} epi={epi} M={M_} N={N} K={K} ws={ws}")
    r = _rng(M_ + N + K + epi)
    A = r.standard_normal((M_, K)).astype(np.float32)
    B = (0.05 * r.standard_normal((N, K))).astype(np.float32)
    bias = r.standard_normal(N).astype(np.float32)
    c0 = r.standard_normal((M_, N)).astype(np.float32)
    if dtype == "bf16":
        A, B = round_bf16(A), round_bf16(B)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    a = torch.from_numpy(A).to(DEV, tdt)
    b = torch.from_numpy(B).to(DEV, tdt)
    bt = torch.from_numpy(bias).to(DEV)
    out_f32 = epi >= 2 or dtype == "f32"
    c = torch.from_numpy(c0).to(DEV) if out_f32 else torch.zeros(M_, N, dtype=tdt, device=DEV)
    wst = torch.empty(ts.TS_GEMM_SPLIT_WS_BYTES, dtype=torch.uint8, device=DEV) if ws else None
    ts.ts_op_gemm(ts.TS_F32 if dtype == "f32" else ts.TS_BF16, epi, a, b, bt, c, ws=wst)
    torch.cuda.synchronize()
    ref = A.astype(np.float64) @ B.astype(np.float64).T + bias
    if epi == 1:
        ref = M.gelu(ref)
    if epi == 2:
        ref = ref + c0
    got = c.float().cpu().numpy()
    if out_f32:
        # fp32 sums of K terms: the rounding error grows like sqrt(K) (random
        # signs); fp32 operands also round each product
        assert max_rel(got, ref) < 1e-5 * max(1.0, np.sqrt(K / 1024))
    else:
        # fp32 accumulation, then one round-to-nearest to bf16 (half an ulp
        # is at most 2^-8 of the value)
        rms = np.sqrt(np.mean(ref * ref))
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * rms)


@pytest.mark.parametrize("M_,N,K", [(40 * 256 + 100, 2048, 256), (40 * 256, 2048, 192)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("ws", [False, True])
def test_gemm_many_tiles(M_, N, K, epi, ws):
    """More 256x256 tiles than compute units (several rounds), an even and an
    odd K block count, and (first shape) a partial last row tile, whose lanes
    past the last row store into the epilogue's sink instead of C.  With a
    workspace the residual epilogue's partial last round runs first as K
    halves in the same launch as the full tiles."""
    test_gemm_against_oracle(M_, N, K, epi, "bf16", ws)


@pytest.mark.parametrize("M_", [5, 512 + 7, 256 + 32])
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gemm_ragged_rows_kernel(M_, epi, dtype, monkeypatch):
    """Rows past the last full 256-row tile through the ragged-row kernel
    (forced here; the library takes it when it saves a round of tiles): every
    epilogue, both MFMA dtypes, N not a multiple of its 32-column blocks, K
    spanning several k-groups per wavefront."""
    monkeypatch.setenv("TS_GEMM_ROWS", "always")
    N, K = 80, (1280 if dtype == "bf16" else 2304)
    say(f"gemm ragged rows {dtype} epi={epi} M={M_} N={N} K={K}")
    r = _rng(M_ + epi)
    A = round_bf16(r.standard_normal((M_, K)).astype(np.float32))
    B = round_bf16((0.05 * r.standard_normal((N, K))).astype(np.float32))
    bias = r.standard_normal(N).astype(np.float32)
    c0 = r.standard_normal((M_, N)).astype(np.float32)
    a = torch.from_numpy(A).to(DEV, torch.bfloat16)
    b = torch.from_numpy(B).to(DEV, torch.bfloat16)
    out_f32 = epi >= 2
    c = torch.from_numpy(c0).to(DEV) if out_f32 else torch.zeros(M_, N, dtype=torch.bfloat16, device=DEV)
    if dtype == "bf16":
        ts.ts_op_gemm(ts.TS_BF16, epi, a, b, torch.from_numpy(bias).to(DEV), c)
        ref = A.astype(np.float64) @ B.astype(np.float64).T + bias
    else:
        a8 = torch.empty(M_, K, dtype=torch.uint8, device=DEV)
        b8 = torch.empty(N, K, dtype=torch.uint8, device=DEV)
        sc = torch.empty(2, dtype=torch.float32, device=DEV)
        ws = torch.empty(256, dtype=torch.uint8, device=DEV)
        ts.ts_fp8_quantize(a, a8, sc[0:1], ws)
        ts.ts_fp8_quantize(b, b8, sc[1:2], ws)
        ts.ts_op_gemm(ts.TS_FP8E4M3, epi, a8, b8, torch.from_numpy(bias).to(DEV), c, sc[0:1], sc[1:2])
        ref = ofp8.fp8_linear(A, B, bias)
    torch.cuda.synchronize()
    if epi == 1:
        ref = M.gelu(ref)
    if epi == 2:
        ref = ref + c0
    got = c.float().cpu().numpy()
    rms = np.sqrt(np.mean(ref * ref))
    # bf16 products are exact and summed in fp32 (1e-5); fp8: the MFMA's
    # internal sum of one instruction's 64 products (2e-4); bf16 outputs add
    # one round to nearest (2^-8 of the value)
    bound = (1e-5 if dtype == "bf16" else 2e-4) * rms + (0 if out_f32 else 2.0 ** -8 * np.abs(ref))
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("Mq,N,K,split", [(333, 512, 640, False), (333, 512, 8192, True)])
def test_gemm_fp8_against_oracle(Mq, N, K, split):
    """split: with the GEMM workspace; the second case splits its 4 tiles 8
    ways along K (64 K blocks of 128 fp8)."""
    say(f"gemm fp8 M={Mq} N={N} K={K} split={split}")
    r = _rng(7)
    A = round_bf16(r.standard_normal((Mq, K)).astype(np.float32))
    B = round_bf16((0.05 * r.standard_normal((N, K))).astype(np.float32))
    bias = r.standard_normal(N).astype(np.float32)
    a = torch.from_numpy(A).to(DEV, torch.bfloat16)
    b = torch.from_numpy(B).to(DEV, torch.bfloat16)
    a8 = torch.empty(Mq, K, dtype=torch.uint8, device=DEV)
    b8 = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    sc = torch.empty(2, dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    ts.ts_fp8_quantize(a, a8, sc[0:1], ws)
    ts.ts_fp8_quantize(b, b8, sc[1:2], ws)
    for epi in (0, 3):
        c = torch.empty(Mq, N, dtype=torch.float32 if epi == 3 else torch.bfloat16, device=DEV)
        wst = torch.empty(ts.TS_GEMM_SPLIT_WS_BYTES, dtype=torch.uint8, device=DEV) if split else None
        ts.ts_op_gemm(ts.TS_FP8E4M3, epi, a8, b8, torch.from_numpy(bias).to(DEV), c, sc[0:1], sc[1:2], ws=wst)
        torch.cuda.synchronize()
        ref = ofp8.fp8_linear(A, B, bias)
        got = c.float().cpu().numpy()
        rms = np.sqrt(np.mean(ref * ref))
        # same e4m3 codes on both sides; the MFMA's internal sum of the 64
        # products of one instruction is not a round-per-add fp32 sum, which
        # leaves a few 1e-5 of the output RMS
        assert np.all(np.abs(got - ref) <= (2.0 ** -8 * np.abs(ref) if epi == 0 else 0) + 2e-4 * rms)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_fp8_quantize_bit_exact(src):
    say(f"fp8 quantize {src}")
    r = _rng(3)
    x = (r.standard_normal(40003) * 3).astype(np.float32)
    # values that land exactly on e4m3 midpoints after scaling: s = 448/448 = 1
    table = ofp8.e4m3_decode_table()
    fin = np.sort(np.unique(np.abs(table[np.isfinite(table)])))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    x[: len(mids)] = mids
    x[len(mids): 2 * len(mids)] = -mids
    x[-1] = 448.0
    if src == "bf16":
        x = round_bf16(x)
    t = torch.from_numpy(x).to(DEV, torch.float32 if src == "f32" else torch.bfloat16)
    q = torch.empty(x.size, dtype=torch.uint8, device=DEV)
    s = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    ts.ts_fp8_quantize(t, q, s, ws)
    torch.cuda.synchronize()
    s_ref = ofp8.tensor_scale(x)
    assert s.cpu().numpy()[0] == s_ref
    codes_ref = ofp8.encode_e4m3(ofp8.round_e4m3(x / s_ref))
    got = q.cpu().numpy()
    # +0 / -0 may differ in sign only when the value is zero
    zero = ofp8.round_e4m3(x / s_ref) == 0
    assert np.array_equal(got[~zero], codes_ref[~zero])
    assert np.all((got[zero] & 0x7F) == 0)


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def run_attention_op(cfg, pl, qkv, q_g, k_g, shared):
    """ts_op_attention on cuda: returns (output, qkv after the call) as float64."""
    tdt = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    n, d = pl.tile_tokens, cfg["d"]
    h = ts.ts_plan_create(cfg["ndim"], cfg["grid"], cfg["tile"], cfg["stride"])
    try:
        ts.ts_plan_upload(h, cfg["head_dim"])
        model = ts.model_desc(cfg)
        tq = torch.from_numpy(qkv).to(DEV, tdt)
        rows_out = pl.n_union + pl.n_tiles if shared else pl.n_tiles * (n + 1)
        out = torch.full((rows_out, d), float("nan"), dtype=tdt, device=DEV)
        ws = torch.empty(ts.ts_workspace_size(model, h, 1), dtype=torch.uint8, device=DEV)
        g = [None if v is None else torch.from_numpy(v).to(DEV) for v in (q_g, k_g)]
        ts.ts_op_attention(model, h, shared, tq, g[0], g[1], out, ws)
        torch.cuda.synchronize()
        return out.double().cpu().numpy(), tq.double().cpu().numpy()
    finally:
        ts.ts_plan_destroy(h)


def check_attention(cfg, pl, qkv, q_g, k_g, shared, got, qkv_gpu, ref, emu_blocks=None, rows=None):
    """The three checks of the attention step (see test_attention_step_against_oracle).
    rows: the output rows compared (default all)."""
    d = cfg["d"]
    sel = slice(None) if rows is None else rows
    assert np.all(np.isfinite(got[sel]))
    if cfg["dtype"] == "f32":
        e = AC.rel(got[sel], ref[sel])
        print(f"  fp32: max|err|/rms {e:.3e}")
        assert e < 1e-4
        return
    # 1. q and k as the library rotated them: the model's values, at most one
    #    bf16 ulp apart (an fp32 ulp can move a rounding decision) plus the fp32
    #    rounding of the rotation's two products (cancellation near zero);
    #    almost all bit-identical; v untouched
    qk_emu, mag = AR.qk_prep(qkv, cfg, pl, shared, q_g, k_g, terms=True)
    dq = np.abs(qkv_gpu[:, :2 * d] - qk_emu[:, :2 * d])
    qb = bf16_ulp(qk_emu[:, :2 * d]) + 2.0 ** -22 * mag
    bad = np.argwhere(dq > qb)
    assert len(bad) == 0, (len(bad), [(int(r), int(c), qkv_gpu[r, c], qk_emu[r, c], mag[r, c]) for r, c in bad[:5]])
    same = float(np.mean(dq == 0))
    assert same > 0.999, same
    assert np.array_equal(qkv_gpu[:, 2 * d:], np.asarray(qkv, np.float64)[:, 2 * d:])
    # 2. the attention on those q and k against the rounding model, element by
    #    element: one output rounding decision (2^-7 relative) plus fp32
    #    accumulation, plus one bf16 ulp of every softmax weight that lies too
    #    close to a rounding midpoint for the model to tell which way the
    #    GPU's fp32 weight rounds (attn_rounding._ambiguous_ulp)
    emu, amb = AR.attention(qkv_gpu, cfg, pl, shared, blocks=emu_blocks, q_g=q_g, k_g=k_g, ambiguity=True)
    rms = float(np.sqrt(np.nanmean(emu[sel] ** 2)))
    bound = 2.0 ** -7 * np.abs(emu[sel]) + 4e-3 * rms + amb[sel]
    dev = np.abs(got[sel] - emu[sel])
    print(f"  qk bit-identical {same:.5f}; max|gpu-model|/rms {np.max(dev) / rms:.3e}, "
          f"worst fraction of bound {np.max(dev / bound):.3f}; ambiguous-weight term max/rms "
          f"{np.max(amb[sel]) / rms:.2e}")
    bad = np.argwhere(dev > bound)
    assert len(bad) == 0, (len(bad), [(int(r), int(c), got[sel][r, c], emu[sel][r, c]) for r, c in bad[:5]])
    # 3. against the oracle, element by element: within what the rounding
    #    points give (the model's own error on these inputs plus the step-2
    #    bound) and under the cap for the logit scale
    ref_rms = float(np.sqrt(np.mean(ref[sel] ** 2)))
    err = np.abs(got[sel] - ref[sel])
    assert np.all(err <= np.abs(emu[sel] - ref[sel]) + bound)
    return float(np.max(err) / ref_rms)


@pytest.mark.parametrize("case", AC.CASES, ids=lambda c: f"{c[1]}-hd{c[5]}-qkn{int(c[6])}-{c[7]}")
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("qk_scale", AC.QK_SCALES)
def test_attention_step_against_oracle(case, shared, qk_scale):
    """The attention step the layers run (ts_op_attention: qk_prep, the window
    kernel with K and V staged from the qkv rows, the global-row kernels and,
    shared, the w-bar blend inside the window kernel) against the oracle,
    element by element: (1) rotated q and k within one bf16 ulp of the rounding
    model, (2) the output within one bf16 ulp plus 4e-3 x RMS of the model run
    on the GPU's own q and k, (3) max|GPU - oracle| / RMS under the cap
    derived from the rounding points (attn_cases.CAP)."""
    cfg = AC.case_cfg(*case)
    say(f"attention step {cfg['dtype']} grid={cfg['grid']} tile={cfg['tile']} hd={cfg['head_dim']} "
        f"qk_norm={cfg['qk_norm']} shared={shared} qk_scale={qk_scale}")
    pl, qkv, q_g, k_g = AC.case_inputs(cfg, shared, qk_scale)
    got, qkv_gpu = run_attention_op(cfg, pl, qkv, q_g, k_g, shared)
    ref = AC.oracle_attention(qkv, cfg, pl, shared, q_g, k_g)
    e = check_attention(cfg, pl, qkv, q_g, k_g, shared, got, qkv_gpu, ref)
    if cfg["dtype"] == "bf16":
        print(f"  max|gpu-oracle|/rms {e:.3e} (cap {AC.CAP[qk_scale]})")
        assert e < AC.CAP[qk_scale]


@pytest.mark.parametrize("gain", [1.3, 1.8])
@pytest.mark.parametrize("shared", [True, False])
def test_attention_softmax_offset_edges(gain, shared):
    """QK-norm gains scaled to near the fixed softmax offset's limit (1.3:
    an offset of 31, weights down to 2^-62) and past it (1.8: the running
    maximum under QK-norm), checked as the other attention cases; the logits
    grow by gain^2, within the cap of qk_scale 3."""
    cfg = AC.case_cfg(*AC.CASES[0])
    assert cfg["qk_norm"]
    say(f"attention step, QK-norm gains x{gain}, shared={shared}")
    pl, qkv, q_g, k_g = AC.case_inputs(cfg, shared, 1.0)
    q_g, k_g = (q_g * np.float32(gain)).astype(np.float32), (k_g * np.float32(gain)).astype(np.float32)
    off = AR.fixed_offset(cfg, q_g, k_g)
    assert (off is not None) == (gain < 1.5), off
    got, qkv_gpu = run_attention_op(cfg, pl, qkv, q_g, k_g, shared)
    ref = AC.oracle_attention(qkv, cfg, pl, shared, q_g, k_g)
    e = check_attention(cfg, pl, qkv, q_g, k_g, shared, got, qkv_gpu, ref)
    print(f"  offset {off}: max|gpu-oracle|/rms {e:.3e} (cap {AC.CAP[3.0]})")
    assert e < AC.CAP[3.0]


@pytest.mark.parametrize("target", [31.5, 33.0])
@pytest.mark.parametrize("shared", [True, False])
def test_attention_norm_offset_edges(target, shared):
    """Without QK-norm: q and k scaled so that the score bound from the
    largest head norms (1.01 max|q| max|k|) is 31.5, an offset of 32 at the
    limit (weights down to 2^-64), or 33, past it (the running maximum);
    checked as the other attention cases.  The logits grow by the square of
    the scale, about 1.6, within the cap of qk_scale 3."""
    case = [c for c in AC.CASES if not c[6] and c[7] == "bf16"][0]
    cfg = AC.case_cfg(*case)
    d, H, hd = cfg["d"], cfg["n_heads"], cfg["head_dim"]
    pl, qkv, _, _ = AC.case_inputs(cfg, shared, 1.0)
    x = AR.qk_prep(qkv, cfg, pl, shared)
    scale = float(np.sqrt(target / AR.norm_bound(x[:, :d], x[:, d:2 * d], H, hd)))
    say(f"attention step, no QK-norm, score bound {target} (q, k x{scale:.3f}), shared={shared}")
    pl, qkv, _, _ = AC.case_inputs(cfg, shared, scale)
    x = AR.qk_prep(qkv, cfg, pl, shared)
    off = AR.norm_offset(x[:, :d], x[:, d:2 * d], H, hd)
    assert (off is not None) == (target < AR.FIXED_MAX_LIMIT), off
    got, qkv_gpu = run_attention_op(cfg, pl, qkv, None, None, shared)
    ref = AC.oracle_attention(qkv, cfg, pl, shared)
    e = check_attention(cfg, pl, qkv, None, None, shared, got, qkv_gpu, ref)
    print(f"  offset {off}: max|gpu-oracle|/rms {e:.3e} (cap {AC.CAP[3.0]})")
    assert e < AC.CAP[3.0]


def test_attention_hard_stitching_blocks():
    """Hard stitching: every grid row's query block holds one tile (the one of
    weight 1), so a shared layer attends each row once; the output is that
    tile's window output."""
    cfg = AC.case_cfg(*AC.CASES[1])
    say("attention step hard stitching")
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"], blend="hard")
    _, qkv, q_g, k_g = AC.case_inputs(cfg, True, 1.0)
    h = ts.ts_plan_create(cfg["ndim"], cfg["grid"], cfg["tile"], cfg["stride"], blend=1)
    try:
        ts.ts_plan_upload(h, cfg["head_dim"])
        tq = torch.from_numpy(qkv).to(DEV, torch.bfloat16)
        out = torch.full((pl.n_union + pl.n_tiles, cfg["d"]), float("nan"), dtype=torch.bfloat16, device=DEV)
        model = ts.model_desc(cfg)
        ws = torch.empty(ts.ts_workspace_size(model, h, 1), dtype=torch.uint8, device=DEV)
        ts.ts_op_attention(model, h, True, tq, None, None, out, ws)
        torch.cuda.synchronize()
        got, qkv_gpu = out.double().cpu().numpy(), tq.double().cpu().numpy()
    finally:
        ts.ts_plan_destroy(h)
    ref = AC.oracle_attention(qkv, cfg, pl, True)
    e = check_attention(cfg, pl, qkv, q_g, k_g, True, got, qkv_gpu, ref)
    print(f"  max|gpu-oracle|/rms {e:.3e}")
    assert e < AC.CAP[1.0]
