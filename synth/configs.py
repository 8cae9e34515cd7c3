"""Workload definitions: the synthetic decoder configurations and one encoder.

Pure data, no arithmetic of the method.  Each entry gives the token grid, the
tiling (tile extent and stride per axis, T/H/W order), the transformer block
shape and the variants that are compared.  Shapes follow the decoders the
TileShare paper page times (MiniMax-H3, ViTok-v2; Tables S5, S6, S12), with
random-initialised weights and seeded synthetic inputs of those shapes.
"""

CONFIGS = {
    # Tiny 2D check: one pre-norm ViT block, fp32 end to end.
    "tiny2d": dict(
        ndim=2, grid=(1, 16, 24), tile=(1, 16, 16), stride=(1, 8, 8),
        n_layers=1, d=64, n_heads=2, head_dim=32, mlp_hidden=256,
        norm="ln", qk_norm=False, dtype="f32", gemm_shared="f32",
        k_values=(0, 1), seed=0),
    # Small video decoder: 704p latent at 16 px patches, 4 latent frames.
    "small_video": dict(
        ndim=3, grid=(4, 44, 80), tile=(4, 44, 44), stride=(4, 36, 36),
        n_layers=8, d=768, n_heads=12, head_dim=64, mlp_hidden=3072,
        norm="ln", qk_norm=False, dtype="bf16", gemm_shared="bf16",
        k_values=(2, 8), seed=0),
    # MiniMax-H3-scale decoder: 28 blocks, d=2560, RMSNorm + QK-norm.
    "minimax_h3": dict(
        ndim=3, grid=(8, 44, 80), tile=(8, 32, 32), stride=(8, 24, 24),
        n_layers=28, d=2560, n_heads=20, head_dim=128, mlp_hidden=10240,
        norm="rms", qk_norm=True, dtype="bf16", gemm_shared="bf16",
        k_values=(6, 28), seed=0),
    # Same stack with the shared layers' GEMMs in fp8 e4m3.
    "minimax_h3_fp8": dict(
        ndim=3, grid=(8, 44, 80), tile=(8, 32, 32), stride=(8, 24, 24),
        n_layers=28, d=2560, n_heads=20, head_dim=128, mlp_hidden=10240,
        norm="rms", qk_norm=True, dtype="bf16", gemm_shared="fp8",
        k_values=(6, 28), seed=0),
    # ViTok-v2-like 4K image decoder: 240x135 tokens, 64x64 tiles, stride 48.
    "vitok4k": dict(
        ndim=2, grid=(1, 135, 240), tile=(1, 64, 64), stride=(1, 48, 48),
        n_layers=24, d=1024, n_heads=16, head_dim=64, mlp_hidden=4096,
        norm="ln", qk_norm=False, dtype="bf16", gemm_shared="bf16",
        k_values=(0, 24), seed=0),
    # The encoder of the ViTok-like 4K pipeline ("+enc": TileShare also in the
    # encoder).  Same token grid, tiling and block shape as the decoder; the
    # pages give no encoder shape, and its depth is read off the tiled
    # timings: pipeline minus decoder is about a fifth of the decoder's time,
    # so five blocks against the decoder's 24.
    "vitok4k_enc": dict(
        ndim=2, grid=(1, 135, 240), tile=(1, 64, 64), stride=(1, 48, 48),
        n_layers=5, d=1024, n_heads=16, head_dim=64, mlp_hidden=4096,
        norm="ln", qk_norm=False, dtype="bf16", gemm_shared="bf16",
        k_values=(0, 5), seed=1),
}

# decoder workload -> the encoder that runs before it in the pipeline
ENCODERS = {"vitok4k": "vitok4k_enc"}

ORDER = ("tiny2d", "small_video", "minimax_h3", "minimax_h3_fp8", "vitok4k", "vitok4k_enc")

ROPE_BASE = 10000.0
EPS = 1e-6
N_GLOBAL = 1


def get(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg
