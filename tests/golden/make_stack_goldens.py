"""Write the stored oracle outputs of the full-width MiniMax-H3-scale stack.

The TileShare paper page times TileShare-6 on MiniMax-H3 (abstract; Table S5:
six layers kept per tile).  The float64 oracle needs minutes for that stack at
the full grid (8 x 44 x 80 tokens, six tiles of 8192, d = 2560), too long for a
GPU test, so this script runs it once and stores what the GPU test compares
with: sampled output rows and the RMS of the whole output.

Workload: the minimax_h3 configuration (bf16) and minimax_h3_fp8 (the shared
layers' four GEMMs in e4m3) with seven layers and k = 6 -- six per-tile
layers, the merge, one shared layer -- on ``synth.make_inputs`` seed 0.  It
calls only ``oracle`` and ``synth``.

Stored per variant (``stack_<config>_L7_k6.npz``):
  rows      union rows sampled: the first, middle and last row of every cover
            count, 64- and 256-row block edges, tile-edge columns, seeded
            random rows
  x_rows    oracle x_out at those rows, float32 [len(rows), d]
  g_out     oracle global rows, float32 [n_tiles, d]
  rms       RMS of the whole oracle x_out (float64)
  checksum  float64 sums of the inputs, so a test can tell stale values
            from a parity failure

Run from the repository root:  python tests/golden/make_stack_goldens.py
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import model as M  # noqa: E402
from oracle.plan import Plan  # noqa: E402
from synth import configs, make_inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
L, K = 7, 6


def input_checksum(x, g, layers):
    """Float64 sums of the token input, the global token and every matrix."""
    s = [float(np.sum(x, dtype=np.float64)), float(np.sum(g, dtype=np.float64))]
    for p in layers:
        for key in ("w_qkv", "w_o", "w_1", "w_2"):
            s.append(float(np.sum(p[key], dtype=np.float64)))
    return np.array(s, dtype=np.float64)


def sample_rows(pl, seed=0):
    """Deterministic sample of union rows (see the module docstring)."""
    counts = np.diff(np.asarray(pl.cover_ptr))
    rows = set()
    for c in sorted(set(counts.tolist())):
        idx = np.nonzero(counts == c)[0]
        rows.update(int(v) for v in (idx[0], idx[len(idx) // 2], idx[-1]))
    m = pl.n_union
    rows.update(r for r in (0, 1, 63, 64, 255, 256, 8191, 8192, m - 257, m - 256, m - 64, m - 1) if 0 <= r < m)
    T, H, W = pl.grid
    # tile-edge columns on one row of the middle frame: first / last column of
    # every tile start and the overlap-band edges
    y, tau = H // 2, T // 2
    for sw in pl.axis_starts[2]:
        for x in (sw, sw + pl.extent[2] - 1):
            rows.add((tau * H + y) * W + x)
    rng = np.random.default_rng(seed)
    rows.update(int(v) for v in rng.choice(m, size=10, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def main():
    for name in ("minimax_h3", "minimax_h3_fp8"):
        cfg = configs.get(name, n_layers=L)
        pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
        x, g, layers = make_inputs(cfg)
        t0 = time.time()
        print(f"{name}: oracle stack L={L} k={K} on grid {cfg['grid']} ...", flush=True)
        xo, go = M.stack_forward(cfg, pl, x, g, layers, K)
        rows = sample_rows(pl)
        out = os.path.join(HERE, f"stack_{name}_L{L}_k{K}.npz")
        np.savez_compressed(out, rows=rows, x_rows=xo[rows].astype(np.float32), g_out=go.astype(np.float32),
                            rms=np.float64(np.sqrt(np.mean(xo * xo))), checksum=input_checksum(x, g, layers),
                            L=L, k=K)
        print(f"{name}: {len(rows)} rows, rms {np.sqrt(np.mean(xo * xo)):.6f}, {time.time() - t0:.0f} s -> {out}",
              flush=True)


if __name__ == "__main__":
    main()
