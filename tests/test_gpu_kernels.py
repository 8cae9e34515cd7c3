"""GPU parity of the building-block kernels against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import shared_token_tiled_amd as ts
from oracle import fp8 as ofp8
from oracle import model as M
from oracle.plan import Plan
from synth import round_bf16

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
def test_gemm_many_tiles(M_, N, K, epi):
    """More 256x256 tiles than compute units (several rounds), an even and an
    odd K block count, and (first shape) a partial last row tile, whose lanes
    past the last row store into the epilogue's sink instead of C."""
    test_gemm_against_oracle(M_, N, K, epi, "bf16", False)


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


ATTN_CASES = [
    # ndim, grid, tile, stride, H, hd, dtype
    (3, (2, 12, 20), (2, 8, 8), (2, 6, 6), 2, 128, "bf16"),
    (3, (2, 12, 28), (2, 12, 12), (2, 8, 8), 3, 64, "bf16"),
    (2, (1, 20, 36), (1, 16, 16), (1, 12, 12), 2, 64, "bf16"),
    (2, (1, 16, 24), (1, 16, 16), (1, 8, 8), 2, 32, "f32"),
    (3, (2, 9, 10), (2, 7, 5), (2, 3, 3), 2, 64, "f32"),
]


@pytest.mark.parametrize("ndim,grid,tile,stride,H,hd,dtype", ATTN_CASES)
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("qk_scale", [1.0, 3.0])
def test_window_attention_against_oracle(ndim, grid, tile, stride, H, hd, dtype, shared, qk_scale):
    say(f"attention {dtype} grid={grid} tile={tile} hd={hd} shared={shared} qk_scale={qk_scale}")
    d = H * hd
    cfg = dict(ndim=ndim, grid=grid, tile=tile, stride=stride, d=d, n_heads=H, head_dim=hd, mlp_hidden=4 * d,
               n_layers=1, norm="ln", qk_norm=False, dtype=dtype, gemm_shared=dtype)
    pl = Plan(grid, tile, stride)
    n = pl.tile_tokens
    rows = pl.n_union + pl.n_tiles if shared else pl.n_tiles * (n + 1)
    r = _rng(11)
    qkv = r.standard_normal((rows, 3 * d)).astype(np.float32)
    qkv[:, : 2 * d] *= qk_scale
    if dtype == "bf16":
        qkv = round_bf16(qkv)
    h = ts.ts_plan_create(ndim, grid, tile, stride)
    try:
        ts.ts_plan_upload(h, hd)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        tq = torch.from_numpy(qkv).to(DEV, tdt)
        out = torch.zeros(pl.n_tiles * (n + 1), d, dtype=tdt, device=DEV)
        ts.ts_op_window_attention(ts.model_desc(cfg), h, shared, tq, out)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
    finally:
        ts.ts_plan_destroy(h)
    rope = M.Rope(pl, cfg)
    q64 = qkv.astype(np.float64)
    row_err, frob = [], []
    for t in range(pl.n_tiles):
        if shared:
            idx = np.concatenate([pl.tile_rows[t].astype(np.int64), [pl.n_union + t]])
        else:
            idx = np.arange(t * (n + 1), (t + 1) * (n + 1))
        ref = M.tile_attention(q64[idx, :d], q64[idx, d:2 * d], q64[idx, 2 * d:], rope.cos, rope.sin, cfg)
        out_t = got[t * (n + 1):(t + 1) * (n + 1)]
        row_err.append(np.max(np.linalg.norm(out_t - ref, axis=1) / np.linalg.norm(ref, axis=1)))
        frob.append(np.linalg.norm(out_t - ref) / np.linalg.norm(ref))
    # bf16: the rotated q and k, the softmax weights and the output are each
    # rounded to bf16 once; with qk_scale 3 the logits are ~9x larger, so the
    # rounding of q and k moves them ~9x more.  A wrong row or key would give
    # per-row errors of order 1.
    if dtype == "f32":
        row_tol, frob_tol = 1e-4, 1e-5
    else:
        row_tol, frob_tol = (2e-2 if qk_scale == 1.0 else 6e-2), 1e-2
    print(f"  worst row rel-L2 {max(row_err):.3e}, frobenius {max(frob):.3e}")
    assert max(row_err) < row_tol and max(frob) < frob_tol, (row_err, frob)
