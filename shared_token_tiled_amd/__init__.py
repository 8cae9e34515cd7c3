"""Python binding of libtileshare (ctypes): the C ABI of include/tileshare.h,
one Python function per entry point with the same name, plus small helpers
that build the C structs from torch tensors.

Argument marshalling only: every step of the path runs in the HIP library.
torch supplies device memory and the current stream.  Loading fails loudly
when the library has not been built.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtileshare.so")

TS_OK = 0
TS_F32, TS_BF16, TS_FP8E4M3 = 0, 1, 2
STATUS_NAMES = {0: "TS_OK", -1: "TS_EINVAL", -2: "TS_ESHAPE", -3: "TS_EDTYPE", -4: "TS_EHIP",
                -5: "TS_ENOMEM", -6: "TS_EUNSUPPORTED", -7: "TS_EWORKSPACE"}


class TilingDesc(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int32), ("grid", ctypes.c_int32 * 3), ("tile", ctypes.c_int32 * 3),
                ("stride", ctypes.c_int32 * 3), ("n_global", ctypes.c_int32), ("blend", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tiles", ctypes.c_int32), ("tile_tokens", ctypes.c_int32), ("n_union", ctypes.c_int32),
                ("n_entries", ctypes.c_int32), ("max_cover", ctypes.c_int32), ("extent", ctypes.c_int32 * 3)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("mlp_hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("qk_norm", ctypes.c_int32), ("eps", ctypes.c_float), ("rope_base", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("gemm_dtype_shared", ctypes.c_int32),
                ("fp8_gemms", ctypes.c_int32), ("fp8_per_tile", ctypes.c_int32),
                ("layer0_dedup", ctypes.c_int32)]


_VP = ctypes.c_void_p


class LayerWeights(ctypes.Structure):
    _fields_ = [(k, _VP) for k in ("norm1_g", "norm1_b", "w_qkv", "b_qkv", "q_g", "k_g", "w_o", "b_o",
                                   "norm2_g", "norm2_b", "w_1", "b_1", "w_2", "b_2",
                                   "w_qkv_f8", "w_o_f8", "w_1_f8", "w_2_f8", "w_scale_f8")]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class TileShareError(RuntimeError):
    pass


_lib = None
ABI_VERSION = 6   # the layout of the structs below; a library of another version is refused


def lib():
    """Load libtileshare.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TileShareError(f"libtileshare.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "ts_abi_version": (ctypes.c_int32, []),
            "ts_last_error": (ctypes.c_char_p, []),
            "ts_plan_create": (ctypes.c_int32, [P(TilingDesc), P(_VP)]),
            "ts_plan_get_info": (ctypes.c_int32, [_VP, P(PlanInfo)]),
            "ts_plan_export": (ctypes.c_int32, [_VP] + [_VP] * 6),
            "ts_plan_export_rope": (ctypes.c_int32, [_VP, ctypes.c_int32, ctypes.c_float, _VP, _VP]),
            "ts_plan_export_blocks": (ctypes.c_int32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "ts_plan_export_job_order": (ctypes.c_int32, [_VP, _VP, _VP, _VP]),
            "ts_plan_upload": (ctypes.c_int32, [_VP, ctypes.c_int32, ctypes.c_float, _VP]),
            "ts_plan_destroy": (None, [_VP]),
            "ts_workspace_size": (ctypes.c_int32, [P(ModelDesc), _VP, ctypes.c_int32, P(ctypes.c_size_t)]),
            "ts_shared_layer_forward": (ctypes.c_int32, [P(ModelDesc), P(LayerWeights), _VP, _VP, _VP,
                                                         ctypes.c_size_t, _VP]),
            "ts_stack_forward": (ctypes.c_int32, [P(ModelDesc), P(LayerWeights), _VP, ctypes.c_int32, _VP, _VP,
                                                  _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "ts_tiled_forward": (ctypes.c_int32, [P(ModelDesc), P(LayerWeights), _VP, _VP, _VP, _VP, _VP, _VP,
                                                  ctypes.c_size_t, _VP]),
            "ts_merge_once_forward": (ctypes.c_int32, [P(ModelDesc), P(LayerWeights), _VP, ctypes.c_int32, _VP,
                                                       _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "ts_partial_share_forward": (ctypes.c_int32, [P(ModelDesc), P(LayerWeights), _VP, ctypes.c_int32,
                                                          ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                                          _VP]),
            "ts_fp8_quantize": (ctypes.c_int32, [_VP, ctypes.c_int32, ctypes.c_int64, _VP, _VP, _VP,
                                                 ctypes.c_size_t, _VP]),
            "ts_op_gemm": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _VP, _VP, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP]),
            "ts_op_gemm_ws": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _VP, _VP, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                               ctypes.c_size_t, _VP]),
            "ts_op_attention": (ctypes.c_int32, [P(ModelDesc), _VP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                                 ctypes.c_size_t, _VP]),
            "ts_op_attention_noalloc": (ctypes.c_int32, [P(ModelDesc), _VP, ctypes.c_int32, _VP, _VP, _VP, _VP,
                                                         _VP]),
            "ts_profile_begin": (ctypes.c_int32, []),
            "ts_profile_end": (ctypes.c_int32, [P(KernelStat), ctypes.c_int32, P(ctypes.c_int32)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if ABI_VERSION is not None and L.ts_abi_version() != ABI_VERSION:
            raise TileShareError(f"{LIB_PATH} has ABI version {L.ts_abi_version()}, this binding {ABI_VERSION}; "
                                 "rebuild with __graft_entry__.build()")
        _lib = L
    return _lib


def _check(st, what):
    if st != TS_OK:
        msg = lib().ts_last_error().decode(errors="replace")
        raise TileShareError(f"{what} failed: {STATUS_NAMES.get(st, st)}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---- entry points (same names as the C ABI) ----------------------------------

def ts_abi_version():
    return lib().ts_abi_version()


def ts_plan_create(ndim, grid, tile, stride, n_global=1, blend=0):
    d = TilingDesc(ndim, (ctypes.c_int32 * 3)(*grid), (ctypes.c_int32 * 3)(*tile),
                   (ctypes.c_int32 * 3)(*stride), n_global, blend)
    h = ctypes.c_void_p()
    _check(lib().ts_plan_create(ctypes.byref(d), ctypes.byref(h)), "ts_plan_create")
    return h


def ts_plan_get_info(plan):
    info = PlanInfo()
    _check(lib().ts_plan_get_info(plan, ctypes.byref(info)), "ts_plan_get_info")
    return info


def ts_plan_export(plan):
    """Return numpy arrays (tile_start, tile_rows, cover_ptr, cover_tile, cover_local, cover_w)."""
    import numpy as np
    info = ts_plan_get_info(plan)
    ts = np.empty((info.n_tiles, 3), np.int32)
    tr = np.empty((info.n_tiles, info.tile_tokens), np.int32)
    cp = np.empty(info.n_union + 1, np.int32)
    ct = np.empty(info.n_entries, np.int32)
    cl = np.empty(info.n_entries, np.int32)
    cw = np.empty(info.n_entries, np.float32)
    _check(lib().ts_plan_export(plan, *(a.ctypes.data_as(_VP) for a in (ts, tr, cp, ct, cl, cw))),
           "ts_plan_export")
    return ts, tr, cp, ct, cl, cw


def ts_plan_export_rope(plan, head_dim, rope_base=10000.0):
    import numpy as np
    info = ts_plan_get_info(plan)
    c = np.empty((info.tile_tokens, head_dim // 2), np.float32)
    s = np.empty((info.tile_tokens, head_dim // 2), np.float32)
    _check(lib().ts_plan_export_rope(plan, head_dim, rope_base, c.ctypes.data_as(_VP), s.ctypes.data_as(_VP)),
           "ts_plan_export_rope")
    return c, s


def ts_plan_export_blocks(plan):
    """Return numpy arrays (blk_nt [nblk], blk_tiles [nblk, maxc], blk_rows [nblk, 256], blk_w [nblk, maxc, 256])."""
    import numpy as np
    nb, mc = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ts_plan_export_blocks(plan, ctypes.byref(nb), ctypes.byref(mc), None, None, None, None),
           "ts_plan_export_blocks")
    nt = np.empty(nb.value, np.int32)
    tl = np.empty((nb.value, mc.value), np.int32)
    rw = np.empty((nb.value, 256), np.int32)
    w = np.empty((nb.value, mc.value, 256), np.float32)
    _check(lib().ts_plan_export_blocks(plan, None, None, *(a.ctypes.data_as(_VP) for a in (nt, tl, rw, w))),
           "ts_plan_export_blocks")
    return nt, tl, rw, w


def ts_plan_export_job_order(plan):
    """Return numpy arrays (order [nblk], cls [ncls, 4]) of the blended attention's job order."""
    import numpy as np
    nc = ctypes.c_int32()
    _check(lib().ts_plan_export_job_order(plan, ctypes.byref(nc), None, None), "ts_plan_export_job_order")
    nb = ctypes.c_int32()
    _check(lib().ts_plan_export_blocks(plan, ctypes.byref(nb), None, None, None, None, None), "ts_plan_export_blocks")
    order = np.empty(nb.value, np.int32)
    cls = np.empty((nc.value, 4), np.int32)
    _check(lib().ts_plan_export_job_order(plan, None, order.ctypes.data_as(_VP), cls.ctypes.data_as(_VP)),
           "ts_plan_export_job_order")
    return order, cls


def ts_plan_upload(plan, head_dim, rope_base=10000.0, stream=None):
    _check(lib().ts_plan_upload(plan, head_dim, rope_base, _stream(stream)), "ts_plan_upload")


def ts_plan_destroy(plan):
    lib().ts_plan_destroy(plan)


def ts_workspace_size(model, plan, k):
    n = ctypes.c_size_t()
    _check(lib().ts_workspace_size(ctypes.byref(model), plan, k, ctypes.byref(n)), "ts_workspace_size")
    return n.value


def ts_shared_layer_forward(model, weights, plan, x, ws, stream=None):
    _check(lib().ts_shared_layer_forward(ctypes.byref(model), ctypes.byref(weights), plan, _ptr(x), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)),
           "ts_shared_layer_forward")


def ts_stack_forward(model, layers, plan, k, x_in, g, x_out, g_out, ws, stream=None):
    arr = (LayerWeights * len(layers))(*layers)
    _check(lib().ts_stack_forward(ctypes.byref(model), arr, plan, k, _ptr(x_in), _ptr(g), _ptr(x_out),
                                  _ptr(g_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "ts_stack_forward")


def ts_tiled_forward(model, layers, plan, x_in, g, x_out, g_out, ws, stream=None):
    arr = (LayerWeights * len(layers))(*layers)
    _check(lib().ts_tiled_forward(ctypes.byref(model), arr, plan, _ptr(x_in), _ptr(g), _ptr(x_out),
                                  _ptr(g_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "ts_tiled_forward")


def ts_merge_once_forward(model, layers, plan, l, x_in, g, x_out, g_out, ws, stream=None):
    arr = (LayerWeights * len(layers))(*layers)
    _check(lib().ts_merge_once_forward(ctypes.byref(model), arr, plan, l, _ptr(x_in), _ptr(g), _ptr(x_out),
                                       _ptr(g_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "ts_merge_once_forward")


TS_SHARE_Q, TS_SHARE_O, TS_SHARE_M = 1, 2, 4


def ts_partial_share_forward(model, layers, plan, k, share, x_in, g, x_out, g_out, ws, stream=None):
    arr = (LayerWeights * len(layers))(*layers)
    _check(lib().ts_partial_share_forward(ctypes.byref(model), arr, plan, k, share, _ptr(x_in), _ptr(g),
                                          _ptr(x_out), _ptr(g_out), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)),
           "ts_partial_share_forward")


def ts_fp8_quantize(src, dst, scale, ws, stream=None):
    import torch
    dt = TS_F32 if src.dtype == torch.float32 else TS_BF16
    _check(lib().ts_fp8_quantize(_ptr(src), dt, src.numel(), _ptr(dst), _ptr(scale), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "ts_fp8_quantize")


TS_EPI_BIAS, TS_EPI_BIAS_GELU, TS_EPI_RESIDUAL, TS_EPI_F32 = 0, 1, 2, 3
TS_GEMM_SPLIT_WS_BYTES = 64 << 20   # workspace that allows every K-split (8 x 256 KB per CU)


def ts_op_gemm(dtype, epilogue, a, b, bias, c, scale_a=None, scale_b=None, stream=None, ws=None):
    """c = epilogue(a b^T + bias); a [m, k], b [n, k] device tensors.  ws: an
    optional device workspace (uint8 tensor) for the K-split last round."""
    m, k = a.shape[0], a.shape[1]
    n = b.shape[0]
    if ws is None:
        _check(lib().ts_op_gemm(dtype, epilogue, _ptr(a), _ptr(b), m, n, k, _ptr(bias), _ptr(c), _ptr(scale_a),
                                _ptr(scale_b), _stream(stream)), "ts_op_gemm")
    else:
        _check(lib().ts_op_gemm_ws(dtype, epilogue, _ptr(a), _ptr(b), m, n, k, _ptr(bias), _ptr(c),
                                   _ptr(scale_a), _ptr(scale_b), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "ts_op_gemm_ws")


def ts_op_attention(model, plan, shared, qkv, q_g, k_g, out, ws, stream=None):
    """The layer's attention step: qkv (device, modified in place: q and k
    normalised and rotated), q_g / k_g (device fp32 [head_dim] or None), out
    (device, blended rows when shared), ws (device uint8 workspace)."""
    _check(lib().ts_op_attention(ctypes.byref(model), plan, 1 if shared else 0, _ptr(qkv), _ptr(q_g), _ptr(k_g),
                                 _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "ts_op_attention")


TS_NOALLOC_SCRATCH_BYTES = 64 << 20


def ts_op_attention_noalloc(model, plan, shared, qkv, q_g, k_g, out, stream=None):
    """ts_op_attention without a workspace: its scratch is the library's own
    device array (TS_NOALLOC_SCRATCH_BYTES per GPU); calls that overlap on one
    GPU race."""
    _check(lib().ts_op_attention_noalloc(ctypes.byref(model), plan, 1 if shared else 0, _ptr(qkv), _ptr(q_g),
                                         _ptr(k_g), _ptr(out), _stream(stream)), "ts_op_attention_noalloc")


def ts_profile_begin():
    _check(lib().ts_profile_begin(), "ts_profile_begin")


def ts_profile_end(max_records=64):
    arr = (KernelStat * max_records)()
    n = ctypes.c_int32()
    _check(lib().ts_profile_end(arr, max_records, ctypes.byref(n)), "ts_profile_end")
    return [dict(name=arr[i].name.decode(), launches=arr[i].launches, total_ms=arr[i].total_ms,
                 flops=arr[i].flops, bytes=arr[i].bytes) for i in range(n.value)]


# ---- helpers ------------------------------------------------------------------

TS_FP8_QKV, TS_FP8_OUT, TS_FP8_FC1, TS_FP8_FC2 = 1, 2, 4, 8
FP8_BITS = {"qkv": TS_FP8_QKV, "out": TS_FP8_OUT, "fc1": TS_FP8_FC1, "fc2": TS_FP8_FC2}


def model_desc(cfg):
    """ts_model_desc from a configuration dict (synth.configs keys; optional
    "fp8_gemms": names of the fp8 GEMMs, default all four; "fp8_per_tile";
    "layer0_dedup")."""
    act = TS_F32 if cfg["dtype"] == "f32" else TS_BF16
    gs = {"f32": TS_F32, "bf16": TS_BF16, "fp8": TS_FP8E4M3}[cfg.get("gemm_shared", cfg["dtype"])]
    mask = sum(FP8_BITS[n] for n in cfg.get("fp8_gemms", ()))
    return ModelDesc(cfg["d"], cfg["n_heads"], cfg["head_dim"], cfg["mlp_hidden"], cfg["n_layers"],
                     1 if cfg["norm"] == "rms" else 0, 1 if cfg["qk_norm"] else 0,
                     cfg.get("eps", 1e-6), cfg.get("rope_base", 10000.0), act, gs, mask,
                     1 if cfg.get("fp8_per_tile", False) else 0, 1 if cfg.get("layer0_dedup", False) else 0)


def layer_weights(p):
    """ctypes LayerWeights from a dict of device tensors (missing keys -> NULL).
    The caller keeps the tensors alive."""
    return LayerWeights(*[(p[k].data_ptr() if p.get(k) is not None else None)
                          for k, _ in LayerWeights._fields_])


MATRIX_KEYS = ("w_qkv", "w_o", "w_1", "w_2")


def device_layers(layers, cfg, device="cuda"):
    """Upload layer parameter dicts (numpy or torch) to the device: weight
    matrices in the model's act dtype, vectors fp32, and e4m3 copies of the
    matrices with their scales (through ts_fp8_quantize) when the shared GEMMs
    are fp8.  Returns (tensor dicts, LayerWeights structs); keep both alive."""
    import torch
    act = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    fp8 = cfg.get("gemm_shared") == "fp8"
    ws = torch.empty(256, dtype=torch.uint8, device=device) if fp8 else None
    tens, structs = [], []
    for p in layers:
        t = {}
        for k, v in p.items():
            v = torch.as_tensor(v)
            t[k] = v.to(device=device, dtype=act if k in MATRIX_KEYS else torch.float32).contiguous()
        if fp8:
            t["w_scale_f8"] = torch.empty(4, dtype=torch.float32, device=device)
            for i, k in enumerate(MATRIX_KEYS):
                t[k + "_f8"] = torch.empty(t[k].shape, dtype=torch.uint8, device=device)
                ts_fp8_quantize(t[k], t[k + "_f8"], t["w_scale_f8"][i:i + 1], ws)
        tens.append(t)
        structs.append(layer_weights(t))
    return tens, structs


__all__ = [n for n in dir() if n.startswith("ts_")] + ["model_desc", "layer_weights", "lib",
                                                        "TileShareError", "TS_F32", "TS_BF16", "device_layers",
                                                        "TS_FP8E4M3"]
