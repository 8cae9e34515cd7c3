"""Inputs and oracle values shared by the attention tests (CPU and GPU).

Cases: window attention over the tilings of the workloads at reduced size
(several tiles, clamped last tile, ragged key and query blocks), with and
without QK-RMSNorm, on qkv rows drawn N(0, 1) and rounded to bf16, the q and k
columns scaled by qk_scale (1: the model's scale; 3 and 8: sharper softmax).

Caps on max|GPU - oracle| / RMS(oracle), from the rounding points of the
bf16 path (tests/attn_rounding.py): bf16 q and k move a score by about 2^-8
of its size and bf16 softmax weights and outputs add about 2^-9 each, so the
error grows with the logits; the caps sit above what the rounding model gives
on these inputs (test_attn_rounding.py checks that with a 1.25x margin).
"""
import numpy as np

from oracle import model as M
from oracle.plan import Plan
from synth import round_bf16

# ndim, grid, tile, stride, heads, head_dim, qk_norm, dtype
CASES = [
    (3, (2, 12, 20), (2, 8, 8), (2, 6, 6), 2, 128, True, "bf16"),
    (3, (2, 12, 28), (2, 12, 12), (2, 8, 8), 3, 64, False, "bf16"),
    (2, (1, 20, 36), (1, 16, 16), (1, 12, 12), 2, 64, False, "bf16"),
    (3, (2, 12, 20), (2, 8, 8), (2, 6, 6), 2, 128, False, "bf16"),
    (2, (1, 20, 36), (1, 16, 16), (1, 12, 12), 2, 64, True, "bf16"),
    (2, (1, 16, 24), (1, 16, 16), (1, 8, 8), 2, 32, False, "f32"),
    (3, (2, 9, 10), (2, 7, 5), (2, 3, 3), 2, 64, False, "f32"),
]
QK_SCALES = (1.0, 3.0, 8.0)
CAP = {1.0: 0.06, 3.0: 0.16, 8.0: 0.95}   # bf16; fp32 is 1e-4 at every scale


def case_cfg(ndim, grid, tile, stride, H, hd, qk_norm, dtype):
    d = H * hd
    return dict(ndim=ndim, grid=grid, tile=tile, stride=stride, d=d, n_heads=H, head_dim=hd, mlp_hidden=4 * d,
                n_layers=1, norm="rms" if qk_norm else "ln", qk_norm=qk_norm, dtype=dtype, gemm_shared=dtype,
                eps=1e-6)


def case_inputs(cfg, shared, qk_scale, seed=11):
    """(plan, qkv [rows, 3d] fp32 holding bf16 values for bf16, q_g, k_g)."""
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    n, d, hd = pl.tile_tokens, cfg["d"], cfg["head_dim"]
    rows = pl.n_union + pl.n_tiles if shared else pl.n_tiles * (n + 1)
    r = np.random.default_rng(seed)
    qkv = r.standard_normal((rows, 3 * d)).astype(np.float32)
    qkv[:, :2 * d] *= np.float32(qk_scale)
    if cfg["dtype"] == "bf16":
        qkv = round_bf16(qkv)
    q_g = k_g = None
    if cfg["qk_norm"]:
        q_g = (1 + 0.02 * r.standard_normal(hd)).astype(np.float32)
        k_g = (1 + 0.02 * r.standard_normal(hd)).astype(np.float32)
    return pl, qkv, q_g, k_g


def oracle_attention(qkv, cfg, plan, shared, q_g=None, k_g=None):
    """The attention step by the oracle's definition: per-head QK-RMSNorm,
    tile-local RoPE, dense softmax attention per window (tile tokens plus the
    tile's global token); shared: the w-bar blend of every grid row's window
    outputs [n_union] followed by the global rows [n_tiles]; else per-tile
    rows."""
    d, n, nt = cfg["d"], plan.tile_tokens, plan.n_tiles
    x = np.asarray(qkv, np.float64)
    q, k, v = x[:, :d], x[:, d:2 * d], x[:, 2 * d:]
    if cfg["qk_norm"]:
        q = M.head_rms_norm(q, q_g, cfg)
        k = M.head_rms_norm(k, k_g, cfg)
    rope = M.Rope(plan, cfg)
    outs = []
    for t in range(nt):
        if shared:
            idx = np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]])
        else:
            idx = np.arange(t * (n + 1), (t + 1) * (n + 1))
        outs.append(M.tile_attention(q[idx], k[idx], v[idx], rope.cos, rope.sin, cfg))
    if shared:
        return np.vstack([M.blend(plan, outs), np.stack([o[n] for o in outs])])
    return np.vstack(outs)


def rel(a, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(a, np.float64) - ref)) / np.sqrt(np.mean(ref * ref)))


def oracle_attention_rows(qkv, cfg, plan, rows, q_g=None, k_g=None):
    """Grid rows ``rows`` of the shared-layout oracle_attention followed by the
    n_tiles global rows, computing queries only for those rows."""
    d, n, nt = cfg["d"], plan.tile_tokens, plan.n_tiles
    rows = np.asarray(rows, np.int64)
    x = np.asarray(qkv, np.float64)
    need = np.concatenate([rows, plan.n_union + np.arange(nt)])
    q, k, v = x[need, :d], x[:, d:2 * d], x[:, 2 * d:]
    if cfg["qk_norm"]:
        q = M.head_rms_norm(q, q_g, cfg)
        k = M.head_rms_norm(k, k_g, cfg)
    rope = M.Rope(plan, cfg)
    out = np.zeros((len(rows) + nt, d))
    pos = {int(r): i for i, r in enumerate(rows)}
    for t in range(nt):
        win = np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]])
        which, local, wts = [], [], []
        for j, r in enumerate(plan.tile_rows[t]):
            if int(r) in pos:
                which.append(pos[int(r)])
                local.append(j)
                wts.append(dict((tt, w) for tt, _, w in plan.cover_of(int(r)))[t])
        qi = np.array(which + [len(rows) + t], np.int64)
        o = M.attention_rows(q[qi], k[win], v[win], local + [n], rope.cos, rope.sin, cfg)
        for m in range(len(which)):
            out[which[m]] += np.float64(np.float32(wts[m])) * o[m]
        out[len(rows) + t] = o[-1]
    return out
