"""Oracle tiling plan: tile starts, tile rows, coverage map, blend weights, RoPE.

Pages: the Figure 2 caption (overlap tokens are stored once but attended in
every window that holds them; their per-tile attention outputs are blended
with the released weights w-bar), Figure 5 ("tiles per pixel", tile-start
lines) and Table S10 (tile size and overlap as the tiling's parameters).

The pages give neither a clamp rule for the last tile nor the ramp formula of
w-bar.  Readings taken here:

* per axis of length N with tile extent L and stride S: one tile of extent N
  if N <= L, else starts min(i*S, N-L) for i = 0 .. ceil((N-L)/S), i.e. the
  last tile is clamped to the grid end;
* tiles in raster order over their (t, h, w) indices; a tile's tokens in
  raster order over local (tau, y, x); grid row p = (tau*H + y)*W + x;
* w-bar: per axis a linear ramp across each overlap with a neighbour
  (lead/trail below), the product over axes, normalised to sum 1 per token;
  computed in float64 in the order written here and rounded once to fp32;
* hard stitching (Table 2, Table S2: "Hard stitching"; Table 1 caption: the
  rule for blending an overlap token's tiles): w-bar is 1 on the covering
  tile with the largest float64 ramp and 0 on the others, ties to the lowest
  tile index;
* RoPE: the P = head_dim/2 rotation pairs are split over the axes in
  contiguous chunks (t, then h, then w).  3D: h and w get floor(P/3) pairs
  each and t the rest (head_dim 128: 22, 21, 21; head_dim 64: 12, 10, 10).
  2D: h gets floor(P/2) and w the rest.  Pair i of an axis chunk of m pairs
  turns by pos * base**(-i/m); cos/sin in float64, stored as fp32.  The
  tile's global token is not rotated.
"""
import math

import numpy as np


def axis_starts(n, L, S):
    """Tile starts and extent along one axis (clamped last tile)."""
    if n <= L:
        return [0], n
    count = -(-(n - L) // S) + 1
    return [min(i * S, n - L) for i in range(count)], L


def axis_ramp(starts, L, i, u):
    """Unnormalised ramp r(u) of tile i along one axis, float64.

    O_prev / O_next are the overlaps with the previous / next tile (0 at the
    grid border).  lead rises 1/(O+1) .. O/(O+1) over the leading overlap,
    trail falls O/(O+1) .. 1/(O+1) over the trailing one, so the ramps of two
    neighbours are exact complements across their shared band.
    """
    o_prev = starts[i - 1] + L - starts[i] if i > 0 else 0
    o_next = starts[i] + L - starts[i + 1] if i + 1 < len(starts) else 0
    lead = (u + 1) / (o_prev + 1) if u < o_prev else 1.0
    trail = (L - u) / (o_next + 1) if u >= L - o_next else 1.0
    return lead * trail


class Plan:
    """Plain-Python tiling plan for grid (T, H, W)."""

    def __init__(self, grid, tile, stride, n_global=1, blend="ramp"):
        if n_global != 1:
            raise ValueError("one global token per tile")
        self.grid = tuple(int(v) for v in grid)
        T, H, W = self.grid
        self.n_union = T * H * W
        per_axis = [axis_starts(n, L, S) for n, L, S in zip(self.grid, tile, stride)]
        self.axis_starts = [s for s, _ in per_axis]
        self.extent = tuple(e for _, e in per_axis)
        Lt, Lh, Lw = self.extent
        self.tile_tokens = Lt * Lh * Lw
        # tiles, raster over (it, ih, iw)
        self.tile_index = []   # (it, ih, iw)
        self.tile_start = []   # (st, sh, sw)
        for it, st in enumerate(self.axis_starts[0]):
            for ih, sh in enumerate(self.axis_starts[1]):
                for iw, sw in enumerate(self.axis_starts[2]):
                    self.tile_index.append((it, ih, iw))
                    self.tile_start.append((st, sh, sw))
        self.n_tiles = len(self.tile_start)
        # tile_rows[t][j]: grid row of local token j of tile t
        rows = np.empty((self.n_tiles, self.tile_tokens), dtype=np.int32)
        for t, (st, sh, sw) in enumerate(self.tile_start):
            j = 0
            for a in range(Lt):
                for b in range(Lh):
                    for c in range(Lw):
                        rows[t, j] = ((st + a) * H + (sh + b)) * W + (sw + c)
                        j += 1
        self.tile_rows = rows
        # local coordinates of token j (same for every tile)
        self.local_pos = np.array([(a, b, c) for a in range(Lt) for b in range(Lh)
                                   for c in range(Lw)], dtype=np.int64)
        # unnormalised ramp of (tile, local token)
        ramp = np.empty((self.n_tiles, self.tile_tokens), dtype=np.float64)
        for t, idx in enumerate(self.tile_index):
            for j in range(self.tile_tokens):
                r = 1.0
                for ax in range(3):
                    r = r * axis_ramp(self.axis_starts[ax], self.extent[ax], idx[ax],
                                      int(self.local_pos[j, ax]))
                ramp[t, j] = r
        # coverage map in ascending tile order per token
        cover = [[] for _ in range(self.n_union)]
        for t in range(self.n_tiles):
            for j in range(self.tile_tokens):
                cover[int(rows[t, j])].append((t, j))
        if blend not in ("ramp", "hard"):
            raise ValueError("blend must be 'ramp' or 'hard'")
        self.blend = blend
        ptr = np.zeros(self.n_union + 1, dtype=np.int32)
        ctile, clocal, cw = [], [], []
        for p in range(self.n_union):
            ent = cover[p]
            if blend == "hard":
                # hard stitching: the whole weight on the covering tile with the
                # largest ramp (the token lies deepest inside it), ties to the
                # lowest tile index (ent is in ascending tile order)
                best = 0
                for e in range(1, len(ent)):
                    if ramp[ent[e]] > ramp[ent[best]]:
                        best = e
                for e, (t, j) in enumerate(ent):
                    ctile.append(t)
                    clocal.append(j)
                    cw.append(np.float32(1.0 if e == best else 0.0))
            else:
                total = 0.0
                for t, j in ent:
                    total = total + ramp[t, j]
                for t, j in ent:
                    ctile.append(t)
                    clocal.append(j)
                    cw.append(np.float32(ramp[t, j] / total))
            ptr[p + 1] = ptr[p] + len(ent)
        self.cover_ptr = ptr
        self.cover_tile = np.array(ctile, dtype=np.int32)
        self.cover_local = np.array(clocal, dtype=np.int32)
        self.cover_w = np.array(cw, dtype=np.float32)
        self.n_entries = int(ptr[-1])
        self.max_cover = int(np.max(np.diff(ptr)))

    # -- convenience -------------------------------------------------------
    def cover_of(self, p):
        a, b = self.cover_ptr[p], self.cover_ptr[p + 1]
        return [(int(self.cover_tile[e]), int(self.cover_local[e]), float(self.cover_w[e]))
                for e in range(a, b)]

    def tile_start_array(self):
        return np.array(self.tile_start, dtype=np.int32)


def rope_pairs(ndim, head_dim):
    """Number of rotation pairs per axis (t, h, w): 2D h and w get P/2 each
    (w the odd one if P is odd); 3D h and w get floor(P/3) each, t the rest."""
    P = head_dim // 2
    if ndim == 2:
        return (0, P // 2, P - P // 2)
    third = P // 3
    return (P - 2 * third, third, third)


def rope_tables(plan, ndim, head_dim, base=10000.0):
    """cos/sin per (local token, pair) as fp32 arrays [tile_tokens, head_dim/2].

    Pair k lies in the chunk of axis a(k); within the chunk of m pairs it is
    pair i and turns by pos_a * base**(-i/m).  float64 math module, fp32 out.
    """
    counts = rope_pairs(ndim, head_dim)
    P = head_dim // 2
    cos = np.empty((plan.tile_tokens, P), dtype=np.float32)
    sin = np.empty((plan.tile_tokens, P), dtype=np.float32)
    axis_of, index_of, size_of = [], [], []
    for ax in range(3):
        for i in range(counts[ax]):
            axis_of.append(ax)
            index_of.append(i)
            size_of.append(counts[ax])
    for j in range(plan.tile_tokens):
        for k in range(P):
            pos = int(plan.local_pos[j, axis_of[k]])
            ang = pos * (base ** (-index_of[k] / size_of[k]))
            cos[j, k] = math.cos(ang)
            sin[j, k] = math.sin(ang)
    return cos, sin
