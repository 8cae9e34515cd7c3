"""Oracle forward passes, float64: per-tile block, shared layer, TileShare-k stack.

Pages.  Figure 2 caption: in a shared layer every token has one state;
normalisation, the QKV projection and QK-normalisation run once per token, as
do the out-projection and the MLP; attention still runs per released tile
with the tile's own global token and coordinates; an overlap token's per-tile
attention outputs are blended with the released weights w-bar, the only
approximate step.  Table S1: layer 0's Norm1/QKV/QK-RMSNorm are exact once per
token; RoPE stays per tile on tile coordinates; keys and values of layers >= k
come from the shared states; the blend of attention outputs happens in every
layer >= k.  Abstract and Table 1 caption: TileShare-k keeps the first k
layers per tile (per-tile residual streams).

Readings taken where the pages leave a step open: pre-norm block
x += Attn(Norm1(x)); x += MLP(Norm2(x)); MLP = fc1 -> exact erf GELU -> fc2;
LayerNorm for the ViT-style configurations, RMSNorm plus per-head
QK-RMSNorm for the MiniMax-style ones; eps 1e-6; q|k|v split of the QKV
output with head h at columns h*hd .. (h+1)*hd; linear weights stored
[out, in]; the global token is one vector, copied into every tile; at layer k
the per-tile states are merged with w-bar (global rows stay per tile); the
tiled baseline is k = L followed by the same merge; no final norm.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import erf

from . import fp8 as fp8mod
from .plan import rope_tables

F = np.float64


def layer_norm(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def rms_norm(x, g, eps):
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def gelu(x):
    """Exact GELU, x * Phi(x) with the normal CDF written through erf."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def norm(x, p, which, cfg):
    g = p[which + "_g"].astype(F)
    if cfg["norm"] == "ln":
        return layer_norm(x, g, p[which + "_b"].astype(F), cfg.get("eps", 1e-6))
    return rms_norm(x, g, cfg.get("eps", 1e-6))


def linear(x, w, b, fp8=False):
    """y = x W^T + b; with ``fp8`` both operands are per-tensor e4m3 fake-quantised."""
    if fp8:
        return fp8mod.fp8_linear(x, w, b)
    return x @ w.astype(F).T + b.astype(F)


ALL_GEMMS = ("qkv", "out", "fc1", "fc2")


def f8(fp8, gemm):
    """Whether GEMM `gemm` runs in fp8: ``fp8`` is a bool (all four GEMMs) or
    a collection of GEMM names."""
    if isinstance(fp8, bool):
        return fp8
    return gemm in fp8


def fp8_scope(cfg, shared):
    """The fp8 GEMMs of a shared (or per-tile) layer.  Table S2 names "FP8 MLP
    layers only" and "TileShare-4 + FP8", Table S5 "V0 + FP8"; the pages fix
    neither the GEMMs nor the layers, so the configuration states them:
    "fp8_gemms" (default all four) in shared layers, and in per-tile layers
    too when "fp8_per_tile" is set."""
    if cfg.get("gemm_shared") != "fp8" or not (shared or cfg.get("fp8_per_tile", False)):
        return ()
    return tuple(cfg.get("fp8_gemms") or ALL_GEMMS)


def rope_rotate(x, cos, sin):
    """Rotate consecutive pairs (2k, 2k+1) of x [n, hd] by the per-row angles."""
    a = x[:, 0::2]
    b = x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = a * cos - b * sin
    out[:, 1::2] = a * sin + b * cos
    return out


def softmax_attention(q, k, v, scale):
    s = (q @ k.T) * scale
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e @ v) / e.sum(axis=-1, keepdims=True)


def head_rms_norm(z, gain, cfg):
    """RMSNorm over each head's hd channels of z [rows, d], with gain [hd]."""
    hd = cfg["head_dim"]
    z = z.copy()
    for hh in range(cfg["n_heads"]):
        cs = slice(hh * hd, (hh + 1) * hd)
        z[:, cs] = rms_norm(z[:, cs], gain.astype(F), cfg.get("eps", 1e-6))
    return z


def qkv_heads(h, p, cfg, fp8=False):
    """QKV projection and per-head QK-RMSNorm, once per row of h."""
    d = cfg["d"]
    qkv = linear(h, p["w_qkv"], p["b_qkv"], f8(fp8, "qkv"))
    q, k, v = qkv[:, :d].copy(), qkv[:, d:2 * d].copy(), qkv[:, 2 * d:].copy()
    if cfg["qk_norm"]:
        q = head_rms_norm(q, p["q_g"], cfg)
        k = head_rms_norm(k, p["k_g"], cfg)
    return q, k, v


def per_head(fn, n_heads):
    """fn(h) for every head, heads evaluated concurrently when that pays.

    The heads are independent, so this changes only when each is computed,
    not what: every head runs exactly the numpy expressions of fn.  BLAS is
    held to one thread per head meanwhile, so the threads do not compete for
    cores inside the products."""
    workers = min(n_heads, len(os.sched_getaffinity(0)))
    if workers <= 1:
        for h in range(n_heads):
            fn(h)
        return
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fn, range(n_heads)))


def tile_attention(q, k, v, cos_t, sin_t, cfg):
    """Dense attention of one tile window.

    q, k, v: [n+1, d], rows 0..n-1 the tile's tokens in local raster order,
    row n its global token.  cos_t/sin_t: [n+1, hd/2] with the identity
    rotation in the global row.  Returns o [n+1, d].
    """
    hd = cfg["head_dim"]
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(hd)

    def head(hh):
        cs = slice(hh * hd, (hh + 1) * hd)
        qh = rope_rotate(q[:, cs], cos_t, sin_t)
        kh = rope_rotate(k[:, cs], cos_t, sin_t)
        out[:, cs] = softmax_attention(qh, kh, v[:, cs], scale)

    per_head(head, cfg["n_heads"])
    return out


def mlp(x, p, cfg, fp8=False):
    hid = gelu(linear(x, p["w_1"], p["b_1"], f8(fp8, "fc1")))
    return linear(hid, p["w_2"], p["b_2"], f8(fp8, "fc2"))


class Rope:
    """Tile-local rotation table with an identity row appended for the global token."""

    def __init__(self, plan, cfg):
        cos, sin = rope_tables(plan, cfg["ndim"], cfg["head_dim"],
                               cfg.get("rope_base", 10000.0))
        P = cfg["head_dim"] // 2
        self.cos = np.vstack([cos.astype(F), np.ones((1, P))])
        self.sin = np.vstack([sin.astype(F), np.zeros((1, P))])


def per_tile_layer(X, p, cfg, rope):
    """One released block on one tile's state X [n+1, d] (global row last)."""
    h = norm(X, p, "norm1", cfg)
    q, k, v = qkv_heads(h, p, cfg)
    o = tile_attention(q, k, v, rope.cos, rope.sin, cfg)
    X = X + linear(o, p["w_o"], p["b_o"])
    X = X + mlp(norm(X, p, "norm2", cfg), p, cfg)
    return X


def per_tile_layers(X, p, cfg, rope, fp8=()):
    """The released block on every tile, the tiles batched as one operand
    per GEMM (Table S5 "V0, batched"): equal to per_tile_layer on each tile,
    except that fp8 GEMMs (``fp8``) take one per-tensor scale over all
    tiles' rows."""
    if not fp8:
        return [per_tile_layer(Xt, p, cfg, rope) for Xt in X]
    n1 = X[0].shape[0]
    allx = np.vstack(X)
    q, k, v = qkv_heads(norm(allx, p, "norm1", cfg), p, cfg, fp8)
    o = np.vstack([tile_attention(q[t * n1:(t + 1) * n1], k[t * n1:(t + 1) * n1], v[t * n1:(t + 1) * n1],
                                  rope.cos, rope.sin, cfg) for t in range(len(X))])
    allx = allx + linear(o, p["w_o"], p["b_o"], f8(fp8, "out"))
    allx = allx + mlp(norm(allx, p, "norm2", cfg), p, cfg, fp8)
    return [allx[t * n1:(t + 1) * n1] for t in range(len(X))]


def blend(plan, per_tile_rows):
    """a[p] = sum over the tiles covering p (ascending) of w-bar * row(t, j)."""
    d = per_tile_rows[0].shape[1]
    a = np.zeros((plan.n_union, d), dtype=F)
    for p in range(plan.n_union):
        for e in range(plan.cover_ptr[p], plan.cover_ptr[p + 1]):
            t, j = plan.cover_tile[e], plan.cover_local[e]
            a[p] += F(plan.cover_w[e]) * per_tile_rows[t][j]
    return a


def shared_layer(x, G, p, cfg, plan, rope, fp8=False, blend_after_out=False):
    """One shared layer.  x [n_union, d] union states, G [n_tiles, d] global rows.

    Norm1/QKV/QK-norm, the out-projection and the MLP run once per row of the
    union plus the global rows; attention runs per tile over the tile's rows
    of the shared q/k/v; the per-tile outputs are blended with w-bar.
    ``blend_after_out`` blends after the out-projection instead (equal by
    linearity and sum w-bar = 1; used only as a pin).
    """
    n = plan.tile_tokens
    xa = np.vstack([x, G])
    h = norm(xa, p, "norm1", cfg)
    q, k, v = qkv_heads(h, p, cfg, fp8)
    outs = []
    for t in range(plan.n_tiles):
        rows = np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]])
        outs.append(tile_attention(q[rows], k[rows], v[rows], rope.cos, rope.sin, cfg))
    if blend_after_out:
        proj = [linear(o, p["w_o"], p["b_o"], f8(fp8, "out")) for o in outs]
        delta = np.vstack([blend(plan, proj), np.stack([pr[n] for pr in proj])])
    else:
        a = np.vstack([blend(plan, outs), np.stack([o[n] for o in outs])])
        delta = linear(a, p["w_o"], p["b_o"], f8(fp8, "out"))
    xa = xa + delta
    xa = xa + mlp(norm(xa, p, "norm2", cfg), p, cfg, fp8)
    return xa[: plan.n_union], xa[plan.n_union:]


def gather_tiles(plan, x, g):
    """Per-tile states X_t = [x[tile_rows[t]]; g] as float64."""
    return [np.vstack([x[plan.tile_rows[t]].astype(F), g.astype(F)[None, :]])
            for t in range(plan.n_tiles)]


def merge(plan, X):
    """Merge per-tile states into one shared state; global rows stay per tile."""
    n = plan.tile_tokens
    return blend(plan, X), np.stack([Xt[n] for Xt in X])


def stack_forward(cfg, plan, x, g, layers, k, rope=None):
    """TileShare-k: layers < k per tile, merge at layer k, layers >= k shared.

    Returns (x_out [n_union, d], g_out [n_tiles, d]) in float64.  k = L is the
    released tiled decoder (per-tile layers throughout, merged at the end).
    """
    rope = rope or Rope(plan, cfg)
    L = len(layers)
    if k > 0:
        X = gather_tiles(plan, x, g)
        for li in range(k):
            X = per_tile_layers(X, layers[li], cfg, rope, fp8_scope(cfg, False))
        xs, G = merge(plan, X)
    else:
        xs = x.astype(F)
        G = np.tile(g.astype(F)[None, :], (plan.n_tiles, 1))
    for li in range(k, L):
        xs, G = shared_layer(xs, G, layers[li], cfg, plan, rope, fp8=fp8_scope(cfg, True))
    return xs, G


def tiled_forward(cfg, plan, x, g, layers, rope=None):
    """Released overlapping-tile decoding, tiles outermost: every tile runs the
    whole stack on its own window, then the outputs are blended with w-bar."""
    rope = rope or Rope(plan, cfg)
    if fp8_scope(cfg, False):   # fp8 scales span the batch of tiles
        X = gather_tiles(plan, x, g)
        for p in layers:
            X = per_tile_layers(X, p, cfg, rope, fp8_scope(cfg, False))
        return merge(plan, X)
    outs = []
    for t in range(plan.n_tiles):
        Xt = np.vstack([x[plan.tile_rows[t]].astype(F), g.astype(F)[None, :]])
        for p in layers:
            Xt = per_tile_layer(Xt, p, cfg, rope)
        outs.append(Xt)
    return merge(plan, outs)


# --- the same layers evaluated only for some output rows ------------------
#
# Every step of a block except attention is per row, and a row's attention
# output depends only on its own query and on its window's keys and values.
# So one output row of a layer needs the keys and values of every row of the
# windows it lies in, and nothing else of the other rows.  The functions
# below evaluate exactly that, with the same operations as the full functions
# above, so that outputs at the full workload sizes can be checked on a
# sample of rows.  Per-tensor fp8 scales depend on every row of each GEMM
# operand, so these functions take the bf16 / fp32 path only.

def attention_rows(q_sel, k, v, local, cos_t, sin_t, cfg):
    """Rows ``local`` of tile_attention(q, k, v, ...), given only their queries.

    q_sel [len(local), d] are the queries of window rows ``local``; k, v
    [n+1, d] the whole window (global row last).
    """
    hd = cfg["head_dim"]
    local = np.asarray(local, dtype=np.int64)
    out = np.empty_like(q_sel)
    scale = 1.0 / math.sqrt(hd)

    def head(hh):
        cs = slice(hh * hd, (hh + 1) * hd)
        qh = rope_rotate(q_sel[:, cs], cos_t[local], sin_t[local])
        kh = rope_rotate(k[:, cs], cos_t, sin_t)
        out[:, cs] = softmax_attention(qh, kh, v[:, cs], scale)

    per_head(head, cfg["n_heads"])
    return out


def _kv_and_q(h, q_rows, p, cfg):
    """Keys and values of every row of h, queries of rows ``q_rows`` only."""
    d = cfg["d"]
    w, b = p["w_qkv"], p["b_qkv"]
    kv = linear(h, w[d:], b[d:])
    k, v = kv[:, :d].copy(), kv[:, d:].copy()
    q = linear(h[q_rows], w[:d], b[:d])
    if cfg["qk_norm"]:
        q = head_rms_norm(q, p["q_g"], cfg)
        k = head_rms_norm(k, p["k_g"], cfg)
    return q, k, v


def _finish_rows(x_rows, attn_rows, p, cfg):
    """Out-projection, residual and MLP of the rows whose attention is known."""
    xs = x_rows + linear(attn_rows, p["w_o"], p["b_o"])
    return xs + mlp(norm(xs, p, "norm2", cfg), p, cfg)


def _no_fp8(cfg):
    if cfg.get("gemm_shared") == "fp8":
        raise ValueError("per-tensor fp8 scales depend on every row; use the full functions")


def shared_layer_rows(x, G, p, cfg, plan, rope, sel):
    """Union rows ``sel`` and every global row of shared_layer(x, G, ...).

    Returns (x_out [len(sel), d], G_out [n_tiles, d]).
    """
    _no_fp8(cfg)
    sel = np.asarray(sel, dtype=np.int64)
    n, d = plan.tile_tokens, cfg["d"]
    xa = np.vstack([x, G]).astype(F)
    h = norm(xa, p, "norm1", cfg)
    q_rows = np.concatenate([sel, plan.n_union + np.arange(plan.n_tiles)])
    q, k, v = _kv_and_q(h, q_rows, p, cfg)
    a = np.zeros((len(q_rows), d), dtype=F)
    for t in range(plan.n_tiles):
        win = np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]])
        which, local, wts = [], [], []
        for i, r in enumerate(sel):
            for tt, j, w in plan.cover_of(int(r)):
                if tt == t:
                    which.append(i)
                    local.append(j)
                    wts.append(w)
        which.append(len(sel) + t)
        local.append(n)
        o = attention_rows(q[which], k[win], v[win], local, rope.cos, rope.sin, cfg)
        for m in range(len(which) - 1):
            a[which[m]] += F(np.float32(wts[m])) * o[m]
        a[len(sel) + t] = o[-1]
    out = _finish_rows(xa[q_rows], a, p, cfg)
    return out[: len(sel)], out[len(sel):]


def per_tile_layer_rows(X, p, cfg, rope, local):
    """Rows ``local`` of per_tile_layer(X, ...) for one tile state X [n+1, d]."""
    local = np.asarray(local, dtype=np.int64)
    X = np.asarray(X, dtype=F)
    h = norm(X, p, "norm1", cfg)
    q, k, v = _kv_and_q(h, local, p, cfg)
    o = attention_rows(q, k, v, local, rope.cos, rope.sin, cfg)
    return _finish_rows(X[local], o, p, cfg)


def tiled_layer_rows(cfg, plan, x, g, p, sel, rope=None):
    """Rows ``sel`` and the global rows of one per-tile layer followed by the
    merge: stack_forward with one layer and k = 1 (the one-layer tiled
    baseline).  Returns (x_out [len(sel), d], G_out [n_tiles, d])."""
    rope = rope or Rope(plan, cfg)
    sel = np.asarray(sel, dtype=np.int64)
    n, d = plan.tile_tokens, cfg["d"]
    xs = np.zeros((len(sel), d), dtype=F)
    G = np.empty((plan.n_tiles, d), dtype=F)
    for t in range(plan.n_tiles):
        Xt = np.vstack([x[plan.tile_rows[t]].astype(F), g.astype(F)[None, :]])
        which, local, wts = [], [], []
        for i, r in enumerate(sel):
            for tt, j, w in plan.cover_of(int(r)):
                if tt == t:
                    which.append(i)
                    local.append(j)
                    wts.append(w)
        rows = per_tile_layer_rows(Xt, p, cfg, rope, local + [n])
        for m in range(len(which)):
            xs[which[m]] += F(np.float32(wts[m])) * rows[m]
        G[t] = rows[-1]
    return xs, G


def merge_once_forward(cfg, plan, x, g, layers, l, rope=None):
    """Figure 3b: per-tile layers 0 .. l-1, the per-tile states merged once
    into one state (global rows kept per tile), every tile re-gathered from
    it with its own global row, per-tile layers l .. L-1, then the merge of
    the released decoder.  Returns (x_out, g_out) in float64."""
    rope = rope or Rope(plan, cfg)
    scope = fp8_scope(cfg, False)
    X = gather_tiles(plan, x, g)
    for li in range(l):
        X = per_tile_layers(X, layers[li], cfg, rope, scope)
    xs, G = merge(plan, X)
    X = [np.vstack([xs[plan.tile_rows[t]], G[t][None, :]]) for t in range(plan.n_tiles)]
    for li in range(l, len(layers)):
        X = per_tile_layers(X, layers[li], cfg, rope, scope)
    return merge(plan, X)


def partial_share_forward(cfg, plan, x, g, layers, k, share, rope=None):
    """Table 1 (top) and Table S7: from layer k on every tile keeps its own
    residual stream and only the operations in ``share`` run once per token;
    attention always runs per tile.  ``share`` holds any of "q" (Norm1, QKV,
    QK-norm), "o" (out-projection) and "m" (Norm2 and MLP).

    Reading: a shared operation takes the token's w-bar blend of the tiles'
    states as its input (for "o": the blend of the tiles' attention outputs)
    and adds its one result to every tile's stream; global rows stay per tile.
    With every operation shared the blended state follows TileShare-k, with
    none the tiled decoder; the pages state "q + m" = all and, at k = 0,
    "o" alone = TileShare-0.  Returns the final merge (x_out, g_out)."""
    rope = rope or Rope(plan, cfg)
    n = plan.tile_tokens
    X = gather_tiles(plan, x, g)
    for li in range(k):
        X = per_tile_layers(X, layers[li], cfg, rope)

    def blended(rows):
        u, G = merge(plan, rows)
        return np.vstack([u, G])                      # [n_union + n_tiles, d]

    def add_to_tiles(delta):
        return [X[t] + np.vstack([delta[plan.tile_rows[t]], delta[plan.n_union + t][None, :]])
                for t in range(plan.n_tiles)]

    for li in range(k, len(layers)):
        p = layers[li]
        if "q" in share:
            q, kk, v = qkv_heads(norm(blended(X), p, "norm1", cfg), p, cfg)
            outs = []
            for t in range(plan.n_tiles):
                rows = np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]])
                outs.append(tile_attention(q[rows], kk[rows], v[rows], rope.cos, rope.sin, cfg))
        else:
            outs = []
            for Xt in X:
                q, kk, v = qkv_heads(norm(Xt, p, "norm1", cfg), p, cfg)
                outs.append(tile_attention(q, kk, v, rope.cos, rope.sin, cfg))
        if "o" in share:
            X = add_to_tiles(linear(blended(outs), p["w_o"], p["b_o"]))
        else:
            X = [X[t] + linear(outs[t], p["w_o"], p["b_o"]) for t in range(plan.n_tiles)]
        if "m" in share:
            X = add_to_tiles(mlp(norm(blended(X), p, "norm2", cfg), p, cfg))
        else:
            X = [Xt + mlp(norm(Xt, p, "norm2", cfg), p, cfg) for Xt in X]
    return merge(plan, X)


def rel_err(got, ref):
    """max |got - ref| / RMS(ref): the parity metric on the union output."""
    ref = np.asarray(ref, dtype=F)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(np.asarray(got, dtype=F) - ref))) / rms
