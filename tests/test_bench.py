"""bench.py: its FLOP accounting against closed forms and its one-GPU guard
(CPU), and one short run whose JSON line carries the fields it promises (GPU)."""
import json
import os
import subprocess
import sys

import pytest

from oracle.plan import Plan
from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _plan(name):
    cfg = configs.get(name)
    return cfg, Plan(cfg["grid"], cfg["tile"], cfg["stride"])


@pytest.mark.parametrize("name", ["minimax_h3", "small_video", "vitok4k"])
def test_decode_flops_closed_forms(name):
    cfg, pl = _plan(name)
    d, dm, L = cfg["d"], cfg["mlp_hidden"], cfg["n_layers"]
    n, T = pl.tile_tokens, pl.n_tiles
    mt, ms = T * (n + 1), pl.n_union + T
    attn = 4.0 * (n + 1) ** 2 * d * T
    lin = 2.0 * (4 * d * d + 2 * d * dm)
    # the tiled decoder: every layer on every tile's rows
    assert bench.decode_flops(cfg, pl, L) == pytest.approx(L * (lin * mt + attn), rel=1e-12)
    # TileShare-0: every layer on the union rows
    assert bench.decode_flops(cfg, pl, 0) == pytest.approx(L * (lin * ms + attn), rel=1e-12)
    # per-tile streams sharing nothing are the tiled decoder
    assert bench.decode_flops(cfg, pl, 2, share="") == pytest.approx(bench.decode_flops(cfg, pl, L), rel=1e-12)
    # layer-0 dedup saves layer 0's QKV on the duplicated rows, only when layer 0 runs per tile
    k = 2
    saved = bench.decode_flops(cfg, pl, k) - bench.decode_flops(cfg, pl, k, dedup0=True)
    assert saved == pytest.approx(2.0 * 3 * d * d * (mt - ms), rel=1e-12)
    assert bench.decode_flops(cfg, pl, 0, dedup0=True) == bench.decode_flops(cfg, pl, 0)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_line_on_the_small_video_workload():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "small_video", "--k", "2",
                        "--steps", "2", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"].startswith("small_video")
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1 and roof["peak"] == 2500.0
    assert d["tiled_baseline"]["ms_per_step"] > 0 and d["speedup_vs_tiled"] > 0
