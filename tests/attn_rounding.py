"""CPU model of the rounding points of the library's attention step.

Test infrastructure (neither the oracle nor the library): it states where the
bf16 path rounds, so that the attention tests can bound the GPU's deviation
from the oracle by what those roundings produce, element by element.

The step (``ts_op_attention``, and the attention of every layer) rounds at:
  1. q and k after QK-RMSNorm and RoPE: computed in fp32, stored as bf16, q
     multiplied first by the softmax scale log2(e)/sqrt(hd) (fp32), so q.k is
     a score s*log2(e)/sqrt(hd) in the log2 domain.  RoPE turns every row by
     its grid coordinate (a tile's global row by the tile's start); a score
     depends only on the coordinate difference, so this equals the pages'
     tile-local rotation before rounding (Table S1: RoPE per tile on tile
     coordinates);
  2. the softmax weights of the window's tile tokens: 2^(s*log2(e)/sqrt(hd) - m)
     rounded to bf16 as the P operand of the PV product (against the fixed
     offset the MFMA chains start from -m); the weight sum uses
     the unrounded weights; the global key's weight is never rounded.  With
     QK-RMSNorm every score obeys |s| <= hd max|q_g| max|k_g| (normalised rows
     have norm sqrt(hd), RoPE rotates them), and m is that bound, rounded up
     to an integer (with a 1 % margin), when it is at most 32.  Otherwise m
     is a running maximum that is raised only when some query of the 32
     handled together sees a block of 64 keys exceed it by 2^8 (then each of
     those queries takes the larger of its running and block maximum);
  3. the output: the window output o = O / l (shared layers: the w-bar sum of
     the windows' outputs, in ascending tile order) rounded once to bf16.
The global token's own query row keeps fp32 weights (rounding 3 only).

Everything else is evaluated in float64 here, so the model differs from the
GPU only by fp32 accumulation order and by the rare rounding decision that an
fp32 ulp moves across a bf16 rounding boundary.
"""
import math

import numpy as np

from oracle.plan import rope_pairs
from synth import round_bf16

QB, WAVE, KB = 256, 32, 64
RESCALE_LOG2 = 8.0
FIXED_MAX_LIMIT = 32.0
AMBIG_TOL = 2.0 ** -15   # relative distance of a weight from a bf16 rounding midpoint


def q_scale(hd):
    """log2(e)/sqrt(hd) as the library forms it in fp32: the bf16 path's
    q_prep multiplies q by it, so q.k is a score in the log2 domain."""
    return np.float32(1.4426950408889634) / np.sqrt(np.float32(hd))


def fixed_offset(cfg, q_g, k_g):
    """The fixed softmax offset of the bf16 kernel under QK-RMSNorm (log2
    domain): ceil(1.01 hd C max|q_g| max|k_g| + 1e-3) with C = log2(e)/sqrt(hd)
    as the library forms it in fp32, when at most FIXED_MAX_LIMIT; else None
    (running maximum)."""
    if not cfg.get("qk_norm") or q_g is None or k_g is None:
        return None
    hd = cfg["head_dim"]
    C = float(q_scale(hd))
    b = math.ceil(1.01 * hd * C * float(np.max(np.abs(q_g))) * float(np.max(np.abs(k_g))) + 1e-3)
    return float(b) if b <= FIXED_MAX_LIMIT else None


def norm_bound(q, k, H, hd):
    """1.01 max|q_h| max|k_h| over all rows and heads of q, k as qk_prep
    stored them (fp32 norms and product, as the library forms them): with q
    carrying log2(e)/sqrt(hd), by Cauchy-Schwarz a bound on every score in the
    log2 domain, with a 1 % margin."""
    def top(a):
        a = np.asarray(a, np.float32).reshape(len(a), H, hd)
        return np.float32(np.sqrt((a * a).sum(axis=-1, dtype=np.float32)).max())
    return float(np.float32(np.float32(1.01) * top(q)) * top(k))


def norm_offset(q, k, H, hd):
    """The fixed softmax offset of the bf16 kernel without QK-norm:
    ceil(norm_bound + 1e-3) when at most FIXED_MAX_LIMIT; else None (running
    maximum)."""
    b = math.ceil(float(np.float32(norm_bound(q, k, H, hd)) + np.float32(1e-3)))
    return float(b) if b <= FIXED_MAX_LIMIT else None


def _bf16(a):
    return round_bf16(np.asarray(a, np.float32)).astype(np.float64)


def row_coords(plan, shared):
    """Grid coordinates (t, h, w) of every row of a shared-layout or
    per-tile-layout qkv array, as the library rotates them."""
    T, H, W = plan.grid
    n = plan.tile_tokens
    starts = np.array(plan.tile_start, dtype=np.int64)
    if shared:
        p = np.arange(plan.n_union)
        grid = np.stack([p // (H * W), (p // W) % H, p % W], axis=1)
        return np.vstack([grid, starts])
    loc = np.vstack([plan.local_pos, np.zeros((1, 3), np.int64)])       # window rows, global last
    return (starts[:, None, :] + loc[None, :, :]).reshape(-1, 3)


def qk_prep(qkv, cfg, plan, shared, q_g=None, k_g=None, bf16=True, terms=False):
    """q and k of qkv [rows, 3d] normalised (if cfg["qk_norm"]) and rotated by
    grid coordinate in fp32, rounded to bf16 (float32 arithmetic in the
    library's operation order).  Returns a float64 copy of the whole array.
    bf16=False: the same steps in float64 without rounding.  terms=True also
    returns |a| + |b| of each rotated value's pair (a, b) before the rotation,
    the size of the two products an fp32 evaluation (with or without a fused
    multiply-add) rounds: a rotated value near zero can differ by that much
    times 2^-23 between two such evaluations."""
    d, hd, H = cfg["d"], cfg["head_dim"], cfg["n_heads"]
    eps = np.float32(cfg.get("eps", 1e-6))
    base = cfg.get("rope_base", 10000.0)
    ft = np.float32 if bf16 else np.float64
    x = np.asarray(qkv, ft).copy()
    co = row_coords(plan, shared)
    counts = rope_pairs(cfg["ndim"], hd)
    P = hd // 2
    ang_c = np.empty((x.shape[0], P), ft)
    ang_s = np.empty((x.shape[0], P), ft)
    k = 0
    for ax in range(3):
        for i in range(counts[ax]):
            inv = math.pow(base, -i / counts[ax])
            ang = co[:, ax].astype(np.float64) * inv
            ang_c[:, k] = np.cos(ang).astype(ft)
            ang_s[:, k] = np.sin(ang).astype(ft)
            k += 1
    mag = np.zeros((x.shape[0], 2 * d)) if terms else None
    for sl in range(2 * H):
        cs = slice(sl * hd, (sl + 1) * hd)
        v = x[:, cs]
        if cfg["qk_norm"]:
            gain = np.asarray(q_g if sl < H else k_g, ft)
            ss = np.sum(v * v, axis=1, dtype=ft)
            inv = ft(1.0) / np.sqrt(ss * ft(1.0 / hd) + ft(eps))
            v = (v * inv[:, None]) * gain[None, :]
        a, b = v[:, 0::2], v[:, 1::2]
        if terms:
            ab = (np.abs(a) + np.abs(b)).astype(np.float64)
            mag[:, sl * hd:(sl + 1) * hd][:, 0::2] = ab
            mag[:, sl * hd:(sl + 1) * hd][:, 1::2] = ab
        out = np.empty_like(v)
        out[:, 0::2] = a * ang_c - b * ang_s
        out[:, 1::2] = a * ang_s + b * ang_c
        if bf16 and sl < H:
            # q takes the softmax scale log2(e)/sqrt(hd) (fp32) before its rounding
            out = out * q_scale(hd)
            if terms:
                mag[:, cs] *= float(q_scale(hd))
        x[:, cs] = round_bf16(out) if bf16 else out
    return (x.astype(np.float64), mag) if terms else x.astype(np.float64)


def _ambiguous_ulp(p):
    """The bf16 spacing at each weight p > 0 where p lies within AMBIG_TOL
    (relative) of a rounding midpoint, else 0: there the GPU's fp32 weight,
    a few 1e-6 away from this float64 one (the fp32 score and its exponent
    argument), may round to the other neighbour, one ulp away."""
    p = np.asarray(p, np.float64)
    pos = p > 0
    e = np.floor(np.log2(np.where(pos, p, 1.0)))
    ulp = np.exp2(e - 7)
    mid = np.floor(p / ulp) * ulp + ulp / 2
    return np.where(pos & (np.abs(p - mid) < AMBIG_TOL * p), ulp, 0.0)


def _window(qs, K, V, kg, vg, hd, groups, round_p=True, fixed=None, C=None):
    """Unnormalised output and weight sum of queries qs [nq, hd] over one
    window (tile keys K, V [n, hd], global key kg, vg), against the fixed
    offset ``fixed`` or with the running maximum shared by the queries of each
    group (list of index arrays).  Returns o = O / l [nq, hd] and the bound
    sum_j ulp_j |V_j| / l over the weights whose rounding is ambiguous
    (_ambiguous_ulp), both float64."""
    if C is None:
        C = (1.0 / math.log(2.0)) / math.sqrt(hd)
    n = K.shape[0]
    aV = np.abs(V)
    sl = (qs @ K.T) * C                         # scores, log2 domain
    if fixed is not None:
        wg = np.exp2((qs @ kg) * C - fixed)     # global key weight
        O = wg[:, None] * vg[None, :]
        A = np.zeros_like(O)
        L = wg.copy()
        for j0 in range(0, n, KB):
            p = np.exp2(sl[:, j0:j0 + KB] - fixed)
            O += (_bf16(p) if round_p else p) @ V[j0:j0 + KB]
            if round_p:
                A += _ambiguous_ulp(p) @ aV[j0:j0 + KB]
            L += p.sum(axis=1)
        return O / L[:, None], A / L[:, None]
    m = (qs @ kg) * C                           # running max starts at the global key's score
    wg = np.ones(len(qs))                       # global key weight relative to m
    O = wg[:, None] * vg[None, :]
    A = np.zeros_like(O)
    L = wg.copy()
    for j0 in range(0, n, KB):
        blk = sl[:, j0:j0 + KB]
        bm = blk.max(axis=1)
        raise_any = np.zeros(len(qs), bool)
        for grp in groups:
            if np.any(bm[grp] > m[grp] + RESCALE_LOG2):
                raise_any[grp] = True
        m_new = np.where(raise_any, np.maximum(m, bm), m)
        alpha = np.exp2(m - m_new)
        O *= alpha[:, None]
        A *= alpha[:, None]
        L *= alpha
        m = m_new
        p = np.exp2(blk - m[:, None])
        O += (_bf16(p) if round_p else p) @ V[j0:j0 + KB]
        if round_p:
            A += _ambiguous_ulp(p) @ aV[j0:j0 + KB]
        L += p.sum(axis=1)
    return O / L[:, None], A / L[:, None]


def _global_row(qg, K, V, kg, vg, hd, log2_q=False):
    """The global token's query over its window, fp32 weights (not rounded).
    log2_q: qg carries log2(e)/sqrt(hd) (the bf16 path)."""
    if log2_q:
        s = np.concatenate([K @ qg, [kg @ qg]])
        e = np.exp2(s - s.max())
    else:
        s = np.concatenate([K @ qg, [kg @ qg]]) / math.sqrt(hd)
        e = np.exp(s - s.max())
    return (e[:-1] @ V + e[-1] * vg) / e.sum()


def _pad_to_wave(rows, fill):
    pad = (-len(rows)) % WAVE
    return np.concatenate([rows, np.full(pad, fill, np.int64)]) if pad else rows


def query_blocks(plan):
    """The blended attention's query blocks: grid rows grouped by the tiles
    holding them with a nonzero w-bar, groups by decreasing size of that set
    then by the tile list, rows ascending, cut into blocks of QB.  Returns a
    list of (tiles, rows array)."""
    groups = {}
    for p in range(plan.n_union):
        key = tuple(t for t, _, w in plan.cover_of(p) if w != 0.0)
        groups.setdefault(key, []).append(p)
    order = sorted(groups, key=lambda k: (-len(k), k))
    out = []
    for key in order:
        rows = groups[key]
        for r0 in range(0, len(rows), QB):
            out.append((key, np.array(rows[r0:r0 + QB], np.int64)))
    return out


def attention(qkv_r, cfg, plan, shared, bf16=True, blocks=None, q_g=None, k_g=None, ambiguity=False):
    """The attention step on qkv_r (float64 array with q, k already as
    ``qk_prep`` returns them).  shared: blended rows [n_union + n_tiles, d];
    else per-tile rows [n_tiles*(n+1), d].  ``blocks`` (shared only): indices
    into query_blocks(plan) to evaluate (default all); rows of other blocks
    are left NaN.  Output values rounded to bf16 when ``bf16``.  q_g, k_g:
    the QK-norm gains qkv_r was prepared with (they set the softmax offset).
    ambiguity: also return, per output element, the bound on what softmax
    weights of ambiguous rounding can move it (zero on the global rows)."""
    d, hd, H = cfg["d"], cfg["head_dim"], cfg["n_heads"]
    q, k, v = qkv_r[:, :d], qkv_r[:, d:2 * d], qkv_r[:, 2 * d:]
    fixed = fixed_offset(cfg, q_g, k_g)
    if bf16 and not cfg.get("qk_norm"):
        fixed = norm_offset(q, k, H, hd)
    # bf16: q as qk_prep leaves it, carrying log2(e)/sqrt(hd); scores in the log2 domain
    C = 1.0 if bf16 else None
    n, nt = plan.tile_tokens, plan.n_tiles
    rnd = _bf16 if bf16 else (lambda a: a)
    if shared:
        out = np.full((plan.n_union + nt, d), np.nan)
        win = [np.concatenate([plan.tile_rows[t].astype(np.int64), [plan.n_union + t]]) for t in range(nt)]
    else:
        out = np.full((nt * (n + 1), d), np.nan)
        win = [np.arange(t * (n + 1), (t + 1) * (n + 1)) for t in range(nt)]
    amb = np.zeros_like(out)
    for h in range(H):
        cs = slice(h * hd, (h + 1) * hd)
        for t in range(nt):                      # global query rows
            K, V = k[win[t][:n], cs], v[win[t][:n], cs]
            g = win[t][n]
            row = plan.n_union + t if shared else g
            out[row, cs] = rnd(_global_row(q[g, cs], K, V, k[g, cs], v[g, cs], hd, bf16))
        if shared:
            qb = query_blocks(plan)
            for bi in (range(len(qb)) if blocks is None else blocks):
                tiles, rows = qb[bi]
                # empty slots of a partly filled wavefront run the block's
                # first row and take part in that wavefront's rescale decision
                ext = _pad_to_wave(rows, rows[0])
                groups = [np.arange(w0, w0 + WAVE) for w0 in range(0, len(ext), WAVE)]
                acc = np.zeros((len(rows), hd))
                acc_a = np.zeros((len(rows), hd))
                for t in tiles:
                    K, V = k[win[t][:n], cs], v[win[t][:n], cs]
                    g = win[t][n]
                    o, a = _window(q[ext, cs], K, V, k[g, cs], v[g, cs], hd, groups, bf16, fixed, C)
                    wts = np.array([dict((tt, w) for tt, _, w in plan.cover_of(int(r)))[t] for r in rows],
                                   np.float32).astype(np.float64)
                    acc += wts[:, None] * o[:len(rows)]
                    acc_a += wts[:, None] * a[:len(rows)]
                out[rows, cs] = rnd(acc)
                amb[rows, cs] = acc_a
        else:
            for t in range(nt):
                K, V = k[win[t][:n], cs], v[win[t][:n], cs]
                g = win[t][n]
                rows = win[t][:n]
                # query slots past the window end run its last token
                ext = _pad_to_wave(rows, rows[-1])
                groups = [np.arange(w0, w0 + WAVE) for w0 in range(0, len(ext), WAVE)]
                o, a = _window(q[ext, cs], K, V, k[g, cs], v[g, cs], hd, groups, bf16, fixed, C)
                out[rows, cs] = rnd(o[:n])
                amb[rows, cs] = a[:n]
    return (out, amb) if ambiguity else out
