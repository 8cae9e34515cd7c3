"""Pure-Python per-token loops for tiny grids: a second formulation of the oracle.

Written independently of ``plan`` and ``model`` (no shared helpers): tiles are
found by testing every candidate start, coverage by testing containment of
every token in every tile, w-bar in exact rational arithmetic, and the block
as per-token loops with ``math``.  Used only to pin the vectorised oracle on
grids of at most a few dozen tokens with d around 8.
"""
import math
from fractions import Fraction


def brute_tiles(grid, tile, stride):
    """Tile starts per axis: every min(i*S, N-L) for i >= 0 that is new, in order."""
    per_axis = []
    for n, L, S in zip(grid, tile, stride):
        if n <= L:
            per_axis.append(([0], n))
            continue
        starts = []
        i = 0
        while True:
            s = min(i * S, n - L)
            if s not in starts:
                starts.append(s)
            if s == n - L:
                break
            i += 1
        per_axis.append((starts, L))
    tiles = []
    for st in per_axis[0][0]:
        for sh in per_axis[1][0]:
            for sw in per_axis[2][0]:
                tiles.append((st, sh, sw))
    ext = tuple(e for _, e in per_axis)
    return tiles, ext, [s for s, _ in per_axis]


def brute_cover(grid, tile, stride, hard=False):
    """{grid row p: [(tile t, local j, Fraction w)]}, exact rational weights;
    with ``hard`` the weight is 1 on the tile of largest ramp (lowest index
    among equal ones) and 0 elsewhere."""
    T, H, W = grid
    tiles, ext, axis_starts = brute_tiles(grid, tile, stride)

    def ramp(ax, start, u):
        starts = axis_starts[ax]
        L = ext[ax]
        i = starts.index(start)
        r = Fraction(1)
        if i > 0:
            o = starts[i - 1] + L - start
            if u < o:
                r *= Fraction(u + 1, o + 1)
        if i + 1 < len(starts):
            o = start + L - starts[i + 1]
            if u >= L - o:
                r *= Fraction(L - u, o + 1)
        return r

    cover = {}
    for tau in range(T):
        for y in range(H):
            for x in range(W):
                p = (tau * H + y) * W + x
                ents = []
                for t, (st, sh, sw) in enumerate(tiles):
                    if st <= tau < st + ext[0] and sh <= y < sh + ext[1] and sw <= x < sw + ext[2]:
                        u = (tau - st, y - sh, x - sw)
                        j = (u[0] * ext[1] + u[1]) * ext[2] + u[2]
                        r = ramp(0, st, u[0]) * ramp(1, sh, u[1]) * ramp(2, sw, u[2])
                        ents.append((t, j, r))
                if hard:
                    top = max(r for _, _, r in ents)
                    first = min(t for t, _, r in ents if r == top)
                    cover[p] = [(t, j, Fraction(1 if t == first else 0)) for t, j, _ in ents]
                else:
                    tot = sum(r for _, _, r in ents)
                    cover[p] = [(t, j, r / tot) for t, j, r in ents]
    return cover, tiles, ext


def _norm(v, g, b, kind, eps):
    n = len(v)
    if kind == "ln":
        mu = sum(v) / n
        var = sum((a - mu) ** 2 for a in v) / n
        return [(a - mu) / math.sqrt(var + eps) * g[i] + b[i] for i, a in enumerate(v)]
    ms = sum(a * a for a in v) / n
    return [a / math.sqrt(ms + eps) * g[i] for i, a in enumerate(v)]


def _matvec(w, b, v):
    return [sum(float(w[o][i]) * v[i] for i in range(len(v))) + float(b[o]) for o in range(len(w))]


def _angles(local, ndim, hd, base):
    """Angle of every pair for a token at tile-local (tau, y, x)."""
    P = hd // 2
    if ndim == 2:
        chunks = [(1, P // 2), (2, P - P // 2)]
    else:
        chunks = [(0, P - 2 * (P // 3)), (1, P // 3), (2, P // 3)]
    out = []
    for ax, m in chunks:
        for i in range(m):
            c = float(math.cos(local[ax] * base ** (-i / m)))
            s = float(math.sin(local[ax] * base ** (-i / m)))
            out.append((c, s))
    return out


def _rot(v, cs):
    out = list(v)
    for k, (c, s) in enumerate(cs):
        c = float(_f32(c))
        s = float(_f32(s))
        a, b = v[2 * k], v[2 * k + 1]
        out[2 * k] = a * c - b * s
        out[2 * k + 1] = a * s + b * c
    return out


def _f32(v):
    import numpy as np
    return np.float32(v)


def _gelu(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def _tolist(p):
    return {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in p.items()}


def _qkv_token(hrow, p, cfg):
    d, hd, H = cfg["d"], cfg["head_dim"], cfg["n_heads"]
    qkv = _matvec(p["w_qkv"], p["b_qkv"], hrow)
    q, k, v = qkv[:d], qkv[d:2 * d], qkv[2 * d:]
    if cfg["qk_norm"]:
        for hh in range(H):
            sl = slice(hh * hd, (hh + 1) * hd)
            q[sl] = _norm(q[sl], p["q_g"], None, "rms", cfg.get("eps", 1e-6))
            k[sl] = _norm(k[sl], p["k_g"], None, "rms", cfg.get("eps", 1e-6))
    return q, k, v


def _attend(qs, ks, vs, angs, cfg):
    """Per-token attention loop; qs/ks/vs lists of rows of one window, angs per row."""
    d, hd, H = cfg["d"], cfg["head_dim"], cfg["n_heads"]
    n = len(qs)
    out = [[0.0] * d for _ in range(n)]
    for hh in range(H):
        sl = slice(hh * hd, (hh + 1) * hd)
        qr = [_rot(qs[i][sl], angs[i]) for i in range(n)]
        kr = [_rot(ks[i][sl], angs[i]) for i in range(n)]
        for i in range(n):
            sc = [sum(qr[i][c] * kr[j][c] for c in range(hd)) / math.sqrt(hd) for j in range(n)]
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            z = sum(ex)
            for c in range(hd):
                out[i][hh * hd + c] = sum(ex[j] * vs[j][sl][c] for j in range(n)) / z
    return out


def _window_angles(ext, ndim, hd, base):
    angs = []
    for a in range(ext[0]):
        for b in range(ext[1]):
            for c in range(ext[2]):
                angs.append(_angles((a, b, c), ndim, hd, base))
    angs.append([(1.0, 0.0)] * (hd // 2))     # global token: no rotation
    return angs


def _finish(rows, p, cfg):
    """Residual out-projection already added; add MLP of Norm2 per token."""
    out = []
    for r in rows:
        h2 = _norm(r, p["norm2_g"], p.get("norm2_b"), cfg["norm"], cfg.get("eps", 1e-6))
        u = [_gelu(a) for a in _matvec(p["w_1"], p["b_1"], h2)]
        m = _matvec(p["w_2"], p["b_2"], u)
        out.append([r[i] + m[i] for i in range(len(r))])
    return out


def brute_per_tile_layer(X, p, cfg, ext):
    p = _tolist(p)
    eps = cfg.get("eps", 1e-6)
    hs = [_norm(r, p["norm1_g"], p.get("norm1_b"), cfg["norm"], eps) for r in X]
    qkv = [_qkv_token(h, p, cfg) for h in hs]
    angs = _window_angles(ext, cfg["ndim"], cfg["head_dim"], cfg.get("rope_base", 10000.0))
    o = _attend([a[0] for a in qkv], [a[1] for a in qkv], [a[2] for a in qkv], angs, cfg)
    rows = []
    for i, r in enumerate(X):
        pr = _matvec(p["w_o"], p["b_o"], o[i])
        rows.append([r[c] + pr[c] for c in range(len(r))])
    return _finish(rows, p, cfg)


def brute_shared_layer(x, G, p, cfg, grid, tile, stride):
    """x: list of union rows, G: list of per-tile global rows."""
    p = _tolist(p)
    eps = cfg.get("eps", 1e-6)
    cover, tiles, ext = brute_cover(grid, tile, stride)
    n_union = len(x)
    allrows = list(x) + list(G)
    hs = [_norm(r, p["norm1_g"], p.get("norm1_b"), cfg["norm"], eps) for r in allrows]
    qkv = [_qkv_token(h, p, cfg) for h in hs]
    angs = _window_angles(ext, cfg["ndim"], cfg["head_dim"], cfg.get("rope_base", 10000.0))
    T, H, W = grid
    tile_out = []
    for t, (st, sh, sw) in enumerate(tiles):
        idx = []
        for a in range(ext[0]):
            for b in range(ext[1]):
                for c in range(ext[2]):
                    idx.append(((st + a) * H + (sh + b)) * W + (sw + c))
        idx.append(n_union + t)
        tile_out.append(_attend([qkv[i][0] for i in idx], [qkv[i][1] for i in idx],
                                [qkv[i][2] for i in idx], angs, cfg))
    d = cfg["d"]
    a = []
    for pidx in range(n_union):
        acc = [0.0] * d
        for t, j, w in cover[pidx]:
            wf = float(_f32(float(w)))
            acc = [acc[c] + wf * tile_out[t][j][c] for c in range(d)]
        a.append(acc)
    n = ext[0] * ext[1] * ext[2]
    for t in range(len(tiles)):
        a.append(tile_out[t][n])
    rows = []
    for i, r in enumerate(allrows):
        pr = _matvec(p["w_o"], p["b_o"], a[i])
        rows.append([r[c] + pr[c] for c in range(d)])
    rows = _finish(rows, p, cfg)
    return rows[:n_union], rows[n_union:]
