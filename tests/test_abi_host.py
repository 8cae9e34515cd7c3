"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, builds plans bit-exact to the oracle's, and
rejects bad arguments with the documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import shared_token_tiled_amd as ts
from oracle.plan import Plan, rope_tables
from synth import configs

import attn_rounding as AR

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tileshare.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ts_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = ts.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert ts.ts_abi_version() == 6


PLAN_CASES = [(configs.get(n)["ndim"], configs.get(n)["grid"], configs.get(n)["tile"], configs.get(n)["stride"])
              for n in ("tiny2d", "small_video", "minimax_h3", "vitok4k")] + [
    (2, (1, 7, 9), (1, 4, 4), (1, 3, 3)),
    (3, (3, 5, 6), (2, 3, 4), (1, 2, 3)),
    (3, (2, 6, 6), (2, 6, 3), (2, 6, 3)),
    (2, (1, 5, 11), (1, 5, 5), (1, 5, 2)),
    (3, (2, 3, 3), (2, 4, 4), (2, 4, 4)),
    (2, (1, 13, 29), (1, 6, 7), (1, 4, 5)),
]


@pytest.mark.parametrize("blend", [0, 1])
@pytest.mark.parametrize("ndim,grid,tile,stride", PLAN_CASES)
def test_plan_bit_exact_against_oracle(ndim, grid, tile, stride, blend):
    h = ts.ts_plan_create(ndim, grid, tile, stride, blend=blend)
    try:
        info = ts.ts_plan_get_info(h)
        ref = Plan(grid, tile, stride, blend=("ramp", "hard")[blend])
        assert (info.n_tiles, info.tile_tokens, info.n_union, info.n_entries, info.max_cover) == \
            (ref.n_tiles, ref.tile_tokens, ref.n_union, ref.n_entries, ref.max_cover)
        assert tuple(info.extent) == ref.extent
        st, tr, cp, ct, cl, cw = ts.ts_plan_export(h)
        assert np.array_equal(st, ref.tile_start_array())
        assert np.array_equal(tr, ref.tile_rows)
        assert np.array_equal(cp, ref.cover_ptr)
        assert np.array_equal(ct, ref.cover_tile)
        assert np.array_equal(cl, ref.cover_local)
        assert np.array_equal(cw.view(np.uint32), ref.cover_w.view(np.uint32))   # bit-exact w-bar
        for hd in (32, 64, 128):
            c, s = ts.ts_plan_export_rope(h, hd, 10000.0)
            rc, rs = rope_tables(ref, ndim, hd, 10000.0)
            assert np.array_equal(c.view(np.uint32), rc.view(np.uint32))
            assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    finally:
        ts.ts_plan_destroy(h)


@pytest.mark.parametrize("args,msg", [
    ((4, (1, 2, 3), (1, 2, 3), (1, 1, 1)), "ndim"),
    ((2, (2, 4, 4), (2, 4, 4), (1, 1, 1)), "2D"),
    ((3, (2, 4, 4), (2, 0, 4), (1, 1, 1)), ">= 1"),
    ((3, (2, 4, 4), (2, 4, 4), (1, 1, 0)), ">= 1"),
])
def test_plan_rejects_bad_descriptions(args, msg):
    with pytest.raises(ts.TileShareError, match="TS_EINVAL.*" + msg):
        ts.ts_plan_create(*args)
    with pytest.raises(ts.TileShareError, match="n_global"):
        ts.ts_plan_create(2, (1, 4, 4), (1, 4, 4), (1, 4, 4), n_global=2)
    with pytest.raises(ts.TileShareError, match="blend"):
        ts.ts_plan_create(2, (1, 4, 4), (1, 4, 4), (1, 4, 4), blend=2)


def _model(**kw):
    cfg = dict(configs.get("small_video"))
    cfg.update(kw)
    return ts.model_desc(cfg)


def test_model_and_workspace_validation_on_host():
    h = ts.ts_plan_create(3, (4, 12, 20), (4, 12, 12), (4, 8, 8))
    try:
        m = _model()
        n = ts.ts_workspace_size(m, h, 2)
        assert n > 0 and n % 256 == 0
        with pytest.raises(ts.TileShareError, match="TS_EINVAL"):
            ts.ts_workspace_size(m, h, 9)              # k > n_layers
        with pytest.raises(ts.TileShareError, match="TS_ESHAPE"):
            ts.ts_workspace_size(_model(d=700, n_heads=7, head_dim=100), h, 0)
        with pytest.raises(ts.TileShareError, match="TS_ESHAPE"):
            ts.ts_workspace_size(_model(n_heads=6, head_dim=100), h, 0)   # d != heads*hd
        with pytest.raises(ts.TileShareError, match="TS_EDTYPE"):
            ts.ts_workspace_size(_model(dtype="f32", gemm_shared="bf16", head_dim=64), h, 0)
        # forward calls refuse a plan that was never uploaded, before touching a GPU
        L = ts.lib()
        st = L.ts_stack_forward(ctypes.byref(m), None, h, 0, None, None, None, None, None, 0, None)
        assert st == -1 and b"uploaded" in L.ts_last_error()
        st = L.ts_shared_layer_forward(ctypes.byref(m), None, h, None, None, 0, None)
        assert st == -1
        st = L.ts_fp8_quantize(None, 1, 16, None, None, None, 0, None)
        assert st == -1
    finally:
        ts.ts_plan_destroy(h)


def test_gemm_workspace_alignment_is_checked_before_any_gpu_work():
    L = ts.lib()
    p = ctypes.c_void_p(4096)
    st = L.ts_op_gemm_ws(ts.TS_BF16, ts.TS_EPI_BIAS, p, p, 256, 256, 256, None, p, None, None,
                         ctypes.c_void_p(4096 + 3), 1 << 20, None)
    assert st == -7   # TS_EWORKSPACE


def test_fp8_quantize_alignment_is_checked_before_any_gpu_work():
    """The quantiser reads 16 bytes and writes 8 bytes per lane."""
    L = ts.lib()
    ws = ctypes.c_void_p(4096)
    for src, dst in ((4096 + 8, 4096), (4096, 4096 + 4)):
        st = L.ts_fp8_quantize(ctypes.c_void_p(src), ts.TS_BF16, 1024, ctypes.c_void_p(dst), ctypes.c_void_p(8192),
                               ws, 256, None)
        assert st == -1   # TS_EINVAL
        assert b"aligned" in L.ts_last_error()


def test_layer0_dedup_field_is_validated_and_sized():
    """layer0_dedup must be 0 or 1; with it, the tiled decoder (k = n_layers)
    also holds the shared-layout rows of layer 0 in its workspace."""
    h = ts.ts_plan_create(3, (4, 12, 20), (4, 12, 12), (4, 8, 8))
    try:
        m = _model()
        m.layer0_dedup = 2
        with pytest.raises(ts.TileShareError, match="TS_EINVAL.*layer0_dedup"):
            ts.ts_workspace_size(m, h, 0)
        L = m.n_layers
        plain = ts.ts_workspace_size(_model(), h, L)
        dedup = ts.ts_workspace_size(_model(layer0_dedup=True), h, L)
        info = ts.ts_plan_get_info(h)
        assert dedup - plain >= (info.n_union + info.n_tiles) * m.d * 4
        # stacks with shared layers hold those rows already
        assert ts.ts_workspace_size(_model(layer0_dedup=True), h, 1) == ts.ts_workspace_size(_model(), h, 1)
    finally:
        ts.ts_plan_destroy(h)


def test_graft_entry_build_accepts_the_built_library(monkeypatch):
    """__graft_entry__.build() checks the library it built against the
    binding's ABI version (the compile step itself is stubbed here, so the
    library the other tests loaded is not rewritten under them)."""
    import __graft_entry__ as entry
    from shared_token_tiled_amd import build as b
    monkeypatch.setattr(b, "build", lambda *a, **k: None)
    entry.build()


@pytest.mark.parametrize("blend", [0, 1])
@pytest.mark.parametrize("ndim,grid,tile,stride", PLAN_CASES)
def test_query_blocks_bit_exact_against_the_rule(ndim, grid, tile, stride, blend):
    """The attention's query blocks (grid rows grouped by the tiles holding
    them with a nonzero w-bar) equal the ones the rule builds from the
    oracle's plan: same order, rows, tiles and w-bar bits."""
    h = ts.ts_plan_create(ndim, grid, tile, stride, blend=blend)
    try:
        nt, tl, rw, w = ts.ts_plan_export_blocks(h)
    finally:
        ts.ts_plan_destroy(h)
    ref = Plan(grid, tile, stride, blend=("ramp", "hard")[blend])
    blocks = AR.query_blocks(ref)
    assert len(nt) == len(blocks)
    for b, (tiles, rows) in enumerate(blocks):
        assert nt[b] == len(tiles)
        assert list(tl[b, :len(tiles)]) == list(tiles) and np.all(tl[b, len(tiles):] == -1)
        assert np.array_equal(rw[b, :len(rows)], rows) and np.all(rw[b, len(rows):] == -1)
        for i, t in enumerate(tiles):
            want = np.array([dict((tt, ww) for tt, _, ww in ref.cover_of(int(r)))[t] for r in rows], np.float32)
            assert np.array_equal(w[b, i, :len(rows)].view(np.uint32), want.view(np.uint32))
            assert np.all(w[b, i, len(rows):] == 0)


def test_large_tiles_plan_and_rope_export():
    """64 x 64 tiles with head size 128 (8192 tile-local RoPE values per pair
    set): the plan builds and exports its tile-local table; nothing in the
    layer path limits the table size (the layers rotate by grid coordinate)."""
    h = ts.ts_plan_create(2, (1, 160, 208), (1, 64, 64), (1, 48, 48))
    try:
        c, s = ts.ts_plan_export_rope(h, 128, 10000.0)
        ref = Plan((1, 160, 208), (1, 64, 64), (1, 48, 48))
        rc, rs = rope_tables(ref, 2, 128, 10000.0)
        assert c.shape == (4096, 64)
        assert np.array_equal(c.view(np.uint32), rc.view(np.uint32))
        assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    finally:
        ts.ts_plan_destroy(h)


def _xcd_jobs(order, cls, H, x):
    """The (block, head) jobs XCD x takes, in order: its contiguous run of
    the 2H half-heads (u = 2 head + half), class by class, half by half."""
    U = 2 * H
    q8, r8 = divmod(U, 8)
    u0 = x * (q8 + 1) if x < r8 else r8 * (q8 + 1) + (x - r8) * q8
    nu = q8 + (1 if x < r8 else 0)
    jobs = []
    for ca, oa, cb, ob in cls:
        for u in range(u0, u0 + nu):
            cnt, off = (cb, ob) if u & 1 else (ca, oa)
            jobs += [(int(order[off + i]), u >> 1) for i in range(cnt)]
    return jobs


@pytest.mark.parametrize("ndim,grid,tile,stride", PLAN_CASES + [
    (3, (8, 44, 80), (8, 32, 32), (8, 24, 24)), (2, (1, 135, 240), (1, 64, 64), (1, 48, 48)),
    (3, (4, 44, 80), (4, 44, 44), (4, 36, 36))])
def test_blended_job_order_covers_every_job_once(ndim, grid, tile, stride):
    """The job order of the bf16 blended attention: the two halves of a head
    are a partition of its blocks with work (windows) equal up to one block,
    classes run from the most windows down, and the workgroups the launcher
    starts (8 x the most jobs of an XCD, dealt round-robin to the XCDs) take
    every (block, head) exactly once."""
    h = ts.ts_plan_create(ndim, grid, tile, stride)
    try:
        nt = ts.ts_plan_export_blocks(h)[0]
        order, cls = ts.ts_plan_export_job_order(h)
    finally:
        ts.ts_plan_destroy(h)
    nblk = len(nt)
    assert sorted(order.tolist()) == list(range(nblk))
    na = int(cls[:, 0].sum())
    assert np.all(cls[:, 1] == np.concatenate([[0], np.cumsum(cls[:-1, 0])]))
    assert np.all(cls[:, 3] == na + np.concatenate([[0], np.cumsum(cls[:-1, 2])]))
    works = []
    for half, (ci, oi) in enumerate(((0, 1), (2, 3))):
        prev_w, work = None, 0
        for c in cls:
            blocks = order[c[oi]:c[oi] + c[ci]]
            if len(blocks):
                w = set(nt[blocks].tolist())
                assert len(w) == 1 and (prev_w is None or w.pop() < prev_w)
                prev_w = int(nt[blocks[0]])
                assert np.all(np.diff(blocks) > 0)
                work += prev_w * len(blocks)
        works.append(work)
    assert abs(works[0] - works[1]) <= int(nt.max())
    for H in (1, 2, 3, 12, 16, 20):
        per_xcd = [_xcd_jobs(order, cls, H, x) for x in range(8)]
        nwg = 8 * max(len(j) for j in per_xcd)
        taken = [per_xcd[b % 8][b // 8] for b in range(nwg) if b // 8 < len(per_xcd[b % 8])]
        assert sorted(taken) == sorted((b, hh) for b in range(nblk) for hh in range(H))
