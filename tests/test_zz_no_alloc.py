"""ts_op_attention_noalloc (the attention step with its scratch in the
library's own device array) against ts_op_attention (the same step with a
caller workspace), through the C ABI.

The two run the same kernels on the same inputs with the same split of the
global rows, so their outputs and the rotated q / k they leave in qkv must
agree bit for bit: on two calls in a row, the second on a smaller plan, in the
blended (shared) and per-tile layouts.  A request whose partial blends exceed
the array is refused with TS_EWORKSPACE before any GPU work."""
import numpy as np
import pytest
import torch

import shared_token_tiled_amd as ts
from attn_cases import case_cfg, case_inputs

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

# (grid, tile, stride, heads, head_dim, qk_norm): the larger plan first
PLANS = [((2, 12, 28), (2, 12, 12), (2, 8, 8), 2, 128, True),
         ((1, 16, 24), (1, 16, 16), (1, 8, 8), 3, 64, False)]


def _run(entry, cfg, plan, shared, qkv, q_g, k_g):
    tq = torch.from_numpy(qkv).to(DEV, torch.bfloat16)
    info = ts.ts_plan_get_info(plan)
    rows = info.n_union + info.n_tiles if shared else info.n_tiles * (info.tile_tokens + 1)
    out = torch.full((rows, cfg["d"]), float("nan"), dtype=torch.bfloat16, device=DEV)
    g = [None if v is None else torch.from_numpy(v).to(DEV) for v in (q_g, k_g)]
    model = ts.model_desc(cfg)
    if entry == "ws":
        ws = torch.empty(ts.ts_workspace_size(model, plan, 1), dtype=torch.uint8, device=DEV)
        ts.ts_op_attention(model, plan, shared, tq, g[0], g[1], out, ws)
    else:
        ts.ts_op_attention_noalloc(model, plan, shared, tq, g[0], g[1], out)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), tq.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("shared", [True, False])
def test_noalloc_attention_matches_workspace_entry_point(shared):
    for i, (grid, tile, stride, H, hd, qkn) in enumerate(PLANS):
        cfg = case_cfg(3 if grid[0] > 1 else 2, grid, tile, stride, H, hd, qkn, "bf16")
        say(f"no-alloc attention call {i + 1}: grid={grid} tile={tile} hd={hd} shared={shared}")
        _, qkv, q_g, k_g = case_inputs(cfg, shared, 2.0, seed=30 + i)
        plan = ts.ts_plan_create(cfg["ndim"], grid, tile, stride)
        try:
            ts.ts_plan_upload(plan, hd)
            ref, ref_qkv = _run("ws", cfg, plan, shared, qkv, q_g, k_g)
            got, got_qkv = _run("noalloc", cfg, plan, shared, qkv, q_g, k_g)
        finally:
            ts.ts_plan_destroy(plan)
        assert np.array_equal(got, ref)
        assert np.array_equal(got_qkv, ref_qkv)


def test_noalloc_attention_refuses_partial_blends_beyond_its_scratch():
    """8 x 44 x 80 tokens of width 2560: the fp32 partial blends take 288 MB
    against the 64 MiB array (the per-tile layout needs none and runs)."""
    say("no-alloc attention size limit")
    cfg = case_cfg(3, (8, 44, 80), (8, 32, 32), (8, 24, 24), 20, 128, True, "bf16")
    plan = ts.ts_plan_create(3, (8, 44, 80), (8, 32, 32), (8, 24, 24))
    try:
        ts.ts_plan_upload(plan, 128)
        info = ts.ts_plan_get_info(plan)
        assert info.n_union * cfg["d"] * 4 > ts.TS_NOALLOC_SCRATCH_BYTES
        qkv = torch.zeros(info.n_union + info.n_tiles, 3 * cfg["d"], dtype=torch.bfloat16, device=DEV)
        out = torch.empty(info.n_union + info.n_tiles, cfg["d"], dtype=torch.bfloat16, device=DEV)
        g = torch.ones(128, device=DEV)
        with pytest.raises(ts.TileShareError, match="TS_EWORKSPACE"):
            ts.ts_op_attention_noalloc(ts.model_desc(cfg), plan, True, qkv, g, g, out)
        torch.cuda.synchronize()
    finally:
        ts.ts_plan_destroy(plan)
