"""End-to-end parity of whole stacks at the full workload sizes.

The tolerances are stated per layer stack: max|GPU - oracle| / RMS(oracle)
over the union output, 2e-2 for bf16 and 6e-2 when the shared layers' GEMMs
are fp8 (TileShare paper page: abstract, TileShare-6; Table S5).

* small video (4 x 44 x 80 grid, two 4 x 44 x 44 tiles, 8 layers, d = 768):
  TileShare-2 and TileShare-8 (= the tiled decoder), every output element
  against the float64 oracle run in the test;
* ViTok-like 4K image (135 x 240 grid, fifteen 64 x 64 tiles, d = 1024): two
  layers of TileShare-0 at full width, every element;
* MiniMax-H3 scale (8 x 44 x 80 grid, six 8 x 32 x 32 tiles, d = 2560): seven
  layers with k = 6 -- six per-tile layers, the merge and one shared layer,
  the launch sequence the benchmark times -- in bf16 and with fp8 shared
  GEMMs, on rows sampled at every cover count, block and tile edges, plus
  the global rows, against oracle values stored by
  tests/golden/make_stack_goldens.py (minutes of float64 work at this size).
"""
import os

import numpy as np
import pytest

from oracle import model as M
from oracle.plan import Plan
from synth import configs, make_inputs

from gpu_helpers import TOL, Run, max_rel, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _stack_case(cfg, k):
    x, g, layers = make_inputs(cfg)
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, k)
    finally:
        run.close()
    say("  GPU done; oracle ...")
    ref, gref = M.stack_forward(cfg, pl, x, g, layers, k)
    return got, ggot, ref, gref


@pytest.mark.parametrize("name,k,n_layers", [("small_video", 2, 8), ("small_video", 8, 8), ("vitok4k", 0, 2)])
def test_full_size_stack_every_element(name, k, n_layers):
    cfg = configs.get(name, n_layers=n_layers)
    say(f"full-size stack {name} grid={cfg['grid']} L={n_layers} k={k}")
    got, ggot, ref, gref = _stack_case(cfg, k)
    tol = TOL[cfg["dtype"]]
    e, eg = max_rel(got, ref), max_rel(ggot, gref)
    print(f"  max|err|/rms = {e:.3e} over {got.size} elements (globals {eg:.3e}), tolerance {tol}")
    assert e < tol and eg < tol


def _input_checksum(x, g, layers):
    s = [float(np.sum(x, dtype=np.float64)), float(np.sum(g, dtype=np.float64))]
    for p in layers:
        for key in ("w_qkv", "w_o", "w_1", "w_2"):
            s.append(float(np.sum(p[key], dtype=np.float64)))
    return np.array(s, dtype=np.float64)


@pytest.mark.parametrize("name", ["minimax_h3", "minimax_h3_fp8"])
def test_full_size_stack_ts6_against_stored_oracle(name):
    path = os.path.join(GOLDEN, f"stack_{name}_L7_k6.npz")
    gold = np.load(path)
    L, k = int(gold["L"]), int(gold["k"])
    cfg = configs.get(name, n_layers=L)
    say(f"full-size stack {name} grid={cfg['grid']} L={L} k={k} against stored oracle rows")
    x, g, layers = make_inputs(cfg)
    # stored values belong to exactly these inputs
    assert np.array_equal(_input_checksum(x, g, layers), gold["checksum"]), "stored oracle values are stale"
    run = Run(cfg, layers)
    try:
        got, ggot = run.stack(x, g, k)
    finally:
        run.close()
    rows = gold["rows"]
    rms = float(gold["rms"])
    ref = gold["x_rows"].astype(np.float64)
    gref = gold["g_out"].astype(np.float64)
    e = float(np.max(np.abs(got[rows] - ref))) / rms
    # global rows, relative to the output's RMS: the stated metric covers the
    # grid output only; bf16 stacks are held to the same bound on them too,
    # fp8 ones are reported (their e4m3 roundings of the shared layer's
    # operands flip wherever the bf16 per-tile layers moved a value across
    # an e4m3 rounding boundary, one in about ten values)
    eg = float(np.max(np.abs(ggot - gref))) / rms
    rms_got = float(np.sqrt(np.mean(got * got)))
    tol = TOL["fp8" if cfg["gemm_shared"] == "fp8" else "bf16"]
    print(f"  {len(rows)} rows x {cfg['d']}: max|err|/rms = {e:.3e} (globals {eg:.3e}), output rms "
          f"{rms_got:.5f} vs oracle {rms:.5f}, tolerance {tol}")
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(ggot))
    assert e < tol
    if cfg["gemm_shared"] != "fp8":
        assert eg < tol
    assert abs(rms_got - rms) < tol * rms
