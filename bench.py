"""Decoded tokens/s of TileShare-k against the per-tile (tiled) baseline on one MI355X.

Workload (default): the MiniMax-H3-scale decoder -- 28 pre-norm blocks,
d = 2560, 20 heads of 128, MLP 4x GELU, RMSNorm + QK-norm, bf16 -- over an
8 x 44 x 80 latent grid tiled 8 x 32 x 32 with stride 24 (6 tiles of 8192
tokens plus one global token each).  One step = one TileShare-6 stack
forward over the whole grid (gather, 6 per-tile layers, merge, 22 shared
layers); tokens per step = 28160 grid tokens.  The tiled baseline (every
layer per tile, then the blend) is timed the same way for the speed-up.
Inputs are synthetic and seeded: weights N(0, 0.02) (norm gains 1 + N(0, 0.02))
rounded to bf16, tokens N(0, 1), drawn on the GPU; they are resident in HBM
before the timed region starts.

Prints one JSON line.  --gpus N with N > 1 exits: the library runs on one GPU.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decoded tokens/s TileShare-k vs per-tile baseline; % bf16/fp8 MFMA peak"
PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "f32": 157.3e12}
HBM_PEAK = 8.0e12


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(cfg, seed, device):
    """Seeded synthetic weights and tokens drawn on the GPU (same distributions
    as synth.make_inputs; a different generator, for speed at full size)."""
    import torch
    import shared_token_tiled_amd as ts
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    d, hd, dm, L = cfg["d"], cfg["head_dim"], cfg["mlp_hidden"], cfg["n_layers"]
    act = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

    def rn(shape, std, mean=0.0, dtype=torch.float32):
        return (torch.randn(shape, generator=gen, device=device) * std + mean).to(dtype)

    x = rn((math.prod(cfg["grid"]), d), 1.0, dtype=act).float()
    g = rn((d,), 1.0, dtype=act).float()
    layers = []
    for _ in range(L):
        p = {"norm1_g": rn((d,), 0.02, 1.0), "w_qkv": rn((3 * d, d), 0.02, dtype=act), "b_qkv": rn((3 * d,), 0.02),
             "w_o": rn((d, d), 0.02, dtype=act), "b_o": rn((d,), 0.02), "norm2_g": rn((d,), 0.02, 1.0),
             "w_1": rn((dm, d), 0.02, dtype=act), "b_1": rn((dm,), 0.02),
             "w_2": rn((d, dm), 0.02, dtype=act), "b_2": rn((d,), 0.02)}
        if cfg["norm"] == "ln":
            p["norm1_b"] = rn((d,), 0.02)
            p["norm2_b"] = rn((d,), 0.02)
        if cfg["qk_norm"]:
            p["q_g"] = rn((hd,), 0.02, 1.0)
            p["k_g"] = rn((hd,), 0.02, 1.0)
        layers.append(p)
    tens, structs = ts.device_layers(layers, cfg, device)
    return x, g, tens, structs


def cpu_baseline(cfg, k):
    """Time the CPU oracle (float64 numpy, as it stands) on a bounded sample of
    the workload: one per-tile block on one tile window (tile_tokens + 1 rows),
    then scale to decoded tokens/s of the whole TileShare-k decode by the
    ratio of algorithmic FLOPs."""
    from threadpoolctl import threadpool_limits

    from oracle import model as M
    from oracle.plan import Plan
    from synth import make_inputs
    threads = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=threads):
        return _cpu_baseline(cfg, k, threads, M, Plan, make_inputs)


def _cpu_baseline(cfg, k, threads, M, Plan, make_inputs):
    pl = Plan(cfg["grid"], cfg["tile"], cfg["stride"])
    x, g, layers = make_inputs(cfg, n_layers=1)
    rope = M.Rope(pl, cfg)
    X = M.gather_tiles(pl, x, g)
    # one per-tile block on successive tile windows until about 10 s of CPU work
    dt, windows = 0.0, 0
    while windows < pl.n_tiles and dt < 10.0:
        t0 = time.perf_counter()
        M.per_tile_layer(X[windows], layers[0], cfg, rope)
        dt += time.perf_counter() - t0
        windows += 1
    d, n1 = cfg["d"], pl.tile_tokens + 1
    lin = 2.0 * (3 * d * d + d * d + 2 * d * cfg["mlp_hidden"])
    sample_flops = windows * (lin * n1 + 4.0 * n1 * n1 * d)
    total = decode_flops(cfg, pl, k)
    est = dt * total / sample_flops
    return {"value": pl.n_union / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one per-tile block of {cfg['name']} on {windows} tile window(s) ({n1} rows each, d={d}), "
                      f"float64 numpy, {dt:.2f} s for {sample_flops / 1e12:.3f} TFLOP; scaled by FLOPs to the whole "
                      f"TileShare-{k} decode ({total / 1e12:.1f} TFLOP)"}


def measured_traffic(name, workload, k):
    """HBM bytes per launch of kernel `name` from the committed FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when there is none or the
    kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_ts{k}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    ent = doc.get("kernels", {}).get(name)
    if ent is None:
        return None
    for src, digest in ent["sources"].items():
        with open(os.path.join(ROOT, src), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return ent["hbm_bytes_per_launch"]


def decode_flops(cfg, pl, k, share="qom", dedup0=False):
    """Algorithmic FLOPs of a TileShare-k decode: 2*(3d^2 + d^2 + 2 d dm) per row
    per layer for the projections, 4 (n+1)^2 d per tile per layer for attention.
    ``pl``: anything with n_tiles, tile_tokens and n_union (the library's
    ts_plan_info).
    ``share``: the operations that run once per token from layer k on (q: QKV,
    o: out-projection, m: MLP); the others run on every tile's rows.
    ``dedup0``: a per-tile layer 0 runs its QKV once per token."""
    d, dm, L = cfg["d"], cfg["mlp_hidden"], cfg["n_layers"]
    mt = pl.n_tiles * (pl.tile_tokens + 1)
    ms = pl.n_union + pl.n_tiles
    attn = 4.0 * (pl.tile_tokens + 1) ** 2 * d * pl.n_tiles
    per_tile = 2.0 * (3 * d * d + d * d + 2 * d * dm) * mt + attn
    later = attn
    for op, fl in (("q", 2.0 * 3 * d * d), ("o", 2.0 * d * d), ("m", 2.0 * 2 * d * dm)):
        later += fl * (ms if op in share else mt)
    saved = 2.0 * 3 * d * d * (mt - ms) if dedup0 and k > 0 else 0.0
    return k * per_tile + (L - k) * later - saved


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="minimax_h3")
    ap.add_argument("--k", type=int, default=None, help="per-tile depth (default: the config's TileShare-k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baseline", action="store_true", help="skip timing the tiled baseline")
    ap.add_argument("--blend", choices=("ramp", "hard"), default="ramp",
                    help="w-bar rule: linear ramps (default) or hard stitching")
    ap.add_argument("--merge-once", type=int, default=None, metavar="L",
                    help="time merge-once-at-layer-L-then-per-tile instead of TileShare-k")
    ap.add_argument("--fp8-gemms", default=None,
                    help="comma list of the fp8 GEMMs (qkv,out,fc1,fc2) for fp8 configurations")
    ap.add_argument("--fp8-per-tile", action="store_true", help="fp8 GEMMs in per-tile layers too")
    ap.add_argument("--layer0-dedup", action="store_true",
                    help="TileShare-k with k >= 1: layer 0's Norm1, QKV and QK-norm once per token "
                         "(the tiled baseline stays as released)")
    ap.add_argument("--partial-share", default=None, metavar="OPS",
                    help="time partial sharing from layer k with per-tile streams; OPS from q, o, m (e.g. qo)")
    ap.add_argument("--enc", action="store_true",
                    help="time the pipeline: the config's encoder stack, then the decoder, TileShare in both "
                         "(the encoder at its own k) against tiled in both")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import shared_token_tiled_amd as ts
    from synth import configs

    cfg = configs.get(args.config)
    enc_cfg = None
    if args.enc:
        if args.config not in configs.ENCODERS:
            print(f"bench.py: no encoder is defined for {args.config}", file=sys.stderr)
            sys.exit(2)
        if args.merge_once is not None or args.partial_share is not None:
            print("bench.py: --enc times TileShare-k stacks only", file=sys.stderr)
            sys.exit(2)
        enc_cfg = configs.get(configs.ENCODERS[args.config])
    if args.fp8_gemms:
        cfg["fp8_gemms"] = tuple(args.fp8_gemms.split(","))
    cfg["fp8_per_tile"] = args.fp8_per_tile
    cfg["layer0_dedup"] = args.layer0_dedup
    k = cfg["k_values"][0] if args.k is None else args.k
    L = cfg["n_layers"]
    dev = "cuda"
    torch.cuda.set_device(0)
    log(f"bench: {args.config} {'merge-once' if args.merge_once is not None else f'TileShare-{k}'} vs tiled, "
        f"steps={args.steps} warmup={args.warmup}")
    plan = ts.ts_plan_create(cfg["ndim"], cfg["grid"], cfg["tile"], cfg["stride"],
                             blend=1 if args.blend == "hard" else 0)
    ts.ts_plan_upload(plan, cfg["head_dim"], cfg.get("rope_base", 10000.0))
    info = ts.ts_plan_get_info(plan)
    model = ts.model_desc(cfg)
    model_base = ts.model_desc(dict(cfg, layer0_dedup=False))
    x, g, tens, structs = device_inputs(cfg, cfg.get("seed", 0), dev)
    ws_bytes = max(ts.ts_workspace_size(model, plan, kk) for kk in (k, L, -1))
    if enc_cfg is not None:
        # the encoder: same grid, tiling and width, its own weights; its output
        # rows are the decoder's input tokens, the global tokens stay learned
        k_enc = enc_cfg["k_values"][0]
        enc_model = ts.model_desc(enc_cfg)
        ex, _, enc_tens, enc_structs = device_inputs(enc_cfg, enc_cfg.get("seed", 1), dev)
        ws_bytes = max(ws_bytes, *(ts.ts_workspace_size(enc_model, plan, kk)
                                   for kk in (k_enc, enc_cfg["n_layers"])))
        x_lat = torch.empty_like(ex)
        g_lat = torch.empty(info.n_tiles, cfg["d"], device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    xo = torch.empty_like(x)
    go = torch.empty(info.n_tiles, cfg["d"], device=dev)
    torch.cuda.synchronize()

    share_mask = sum(b for c, b in (("q", ts.TS_SHARE_Q), ("o", ts.TS_SHARE_O), ("m", ts.TS_SHARE_M))
                     if args.partial_share and c in args.partial_share)

    def step_ts():
        if args.merge_once is not None:
            ts.ts_merge_once_forward(model, structs, plan, args.merge_once, x, g, xo, go, ws)
        elif args.partial_share is not None:
            ts.ts_partial_share_forward(model, structs, plan, k, share_mask, x, g, xo, go, ws)
        elif enc_cfg is not None:
            ts.ts_stack_forward(enc_model, enc_structs, plan, k_enc, ex, g, x_lat, g_lat, ws)
            ts.ts_stack_forward(model, structs, plan, k, x_lat, g, xo, go, ws)
        else:
            ts.ts_stack_forward(model, structs, plan, k, x, g, xo, go, ws)

    def step_base():
        if enc_cfg is not None:
            ts.ts_tiled_forward(enc_model, enc_structs, plan, ex, g, x_lat, g_lat, ws)
            ts.ts_tiled_forward(model_base, structs, plan, x_lat, g, xo, go, ws)
        else:
            ts.ts_tiled_forward(model_base, structs, plan, x, g, xo, go, ws)

    def timed(fn, steps, warmup, profile):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if profile:
            ts.ts_profile_begin()
        e0.record(s)
        for _ in range(steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        stats = ts.ts_profile_end() if profile else None
        return e0.elapsed_time(e1) / steps, stats

    # the step time is taken without per-kernel events; the same number of
    # steps then runs again with the library's HIP events around every
    # kernel for the per-kernel figures and the roofline
    ms_ts, _ = timed(step_ts, args.steps, args.warmup, False)
    ms_prof, stats = timed(step_ts, args.steps, 0, True)
    log(f"bench: TileShare-{k}: {ms_ts:.2f} ms/step ({ms_prof:.2f} with per-kernel events)")
    ms_base = None
    if not args.no_baseline:
        ms_base, _ = timed(step_base, args.steps, 1, False)
        log(f"bench: tiled baseline: {ms_base:.2f} ms/step")
    tok = info.n_union
    value = tok / (ms_ts / 1e3)

    # roofline of the dominant kernel, from the library's event timings of the timed steps
    stats = sorted(stats, key=lambda r: -r["total_ms"])
    dom = stats[0]
    dt = "fp8" if "fp8" in dom["name"] else ("f32" if "f32" in dom["name"] else "bf16")
    traffic = measured_traffic(dom["name"], args.config, k)
    if dom["flops"] > 0:
        ach = dom["flops"] / (dom["total_ms"] / 1e3)
        roof = {"kernel": dom["name"], "bound": "mfma", "achieved": ach / 1e12, "peak": PEAK[dt] / 1e12,
                "unit": "TFLOP/s", "frac": ach / PEAK[dt], "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": dom["bytes"] / dom["launches"],
                "launches_per_step": dom["launches"] / args.steps,
                "avg_launch_ms": dom["total_ms"] / dom["launches"],
                "flops_per_launch": dom["flops"] / dom["launches"]}
    else:
        ach = dom["bytes"] / (dom["total_ms"] / 1e3)
        roof = {"kernel": dom["name"], "bound": "hbm", "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": ach / HBM_PEAK, "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "launches_per_step": dom["launches"] / args.steps,
                "avg_launch_ms": dom["total_ms"] / dom["launches"], "bytes_per_launch": dom["bytes"] / dom["launches"]}
    kernels = {}
    for r in stats[:10]:
        sec = r["total_ms"] / 1e3
        kernels[r["name"]] = {"ms_per_step": round(r["total_ms"] / args.steps, 3),
                              "tflops": round(r["flops"] / sec / 1e12, 1) if r["flops"] else None,
                              "gbps": round(r["bytes"] / sec / 1e9, 1)}
    pl = info   # FLOP count needs only the tile counts, from the library's plan
    pl_flops = (decode_flops(cfg, pl, L, dedup0=args.layer0_dedup)
                if args.merge_once is not None else
                decode_flops(cfg, pl, k, args.partial_share if args.partial_share is not None else "qom",
                             dedup0=args.layer0_dedup))
    if enc_cfg is not None:
        pl_flops += decode_flops(enc_cfg, pl, k_enc)
    mode = (f"merge once at layer {args.merge_once}, then per tile" if args.merge_once is not None
            else (f"per-tile streams from layer {k} sharing {args.partial_share or 'nothing'}"
                  if args.partial_share is not None else f"TileShare-{k}"))
    extras = []
    if args.blend == "hard":
        extras.append("hard stitching")
    if args.layer0_dedup:
        extras.append("layer 0 Norm1/QKV/QK-norm once per token")
    if enc_cfg is not None:
        extras.append(f"pipeline: {enc_cfg['name']} encoder ({enc_cfg['n_layers']} blocks, TileShare-{k_enc}) "
                      f"before the decoder; tiled baseline tiled in both")
    if cfg["gemm_shared"] == "fp8":
        extras.append(f"fp8 GEMMs {','.join(cfg.get('fp8_gemms') or ('qkv', 'out', 'fc1', 'fc2'))} in shared"
                      + (" and per-tile" if args.fp8_per_tile else "") + " layers")
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_ts, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if cfg["gemm_shared"] == "fp8" else cfg["dtype"], "data": "synthetic",
        "config": {"workload": f"{args.config} {mode}: grid {'x'.join(map(str, cfg['grid']))}, tiles "
                               f"{'x'.join(map(str, cfg['tile']))} stride {cfg['stride'][-1]}, {L} blocks d={cfg['d']} "
                               f"{cfg['n_heads']}x{cfg['head_dim']} heads, MLP {cfg['mlp_hidden']} GELU"
                               + "".join(f"; {e}" for e in extras),
                   "k": k, "tokens_per_step": tok, "n_tiles": info.n_tiles, "tile_tokens": info.tile_tokens,
                   "parallelism": "single GPU"},
        "tiled_baseline": None if ms_base is None else {"ms_per_step": round(ms_base, 3),
                                                         "tokens_per_s": round(tok / (ms_base / 1e3), 1)},
        "speedup_vs_tiled": None if ms_base is None else round(ms_base / ms_ts, 4),
        "decode_tflops": round(pl_flops / (ms_ts / 1e3) / 1e12, 1),
        "frac_of_bf16_peak": round(pl_flops / (ms_ts / 1e3) / PEAK["bf16"], 4),
        "frac_of_fp8_peak": (round(pl_flops / (ms_ts / 1e3) / PEAK["fp8"], 4)
                             if cfg["gemm_shared"] == "fp8" else None),
        "roofline": roof,
        "kernels": kernels,
        "profiled_ms_per_step": round(ms_prof, 3),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, k)
    ts.ts_plan_destroy(plan)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
