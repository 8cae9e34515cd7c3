"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds no arithmetic of the method: it only draws random numbers in
a fixed order and rounds them to the storage format of a configuration.

Draw order (numpy PCG64, ``default_rng(seed)``): x, g, then per layer
norm1 (gain, bias), qkv (weight, bias), q-gain, k-gain, out (weight, bias),
norm2 (gain, bias), fc1 (weight, bias), fc2 (weight, bias).  Norm biases are
drawn only for LayerNorm blocks, q/k gains only when QK-norm is on.

Distributions: tokens and the global token N(0, 1); linear weights and biases
N(0, 0.02); norm gains 1 + N(0, 0.02); LayerNorm biases N(0, 0.02).  Linear
weights are stored [out_features, in_features].  For bf16 configurations the
weight matrices, x and g are rounded to bf16 (round to nearest even) before
either side sees them, so both sides start from the same values; 1-D
parameters stay fp32.
"""
import numpy as np

from . import configs  # noqa: F401

LAYER_KEYS = ("norm1_g", "norm1_b", "w_qkv", "b_qkv", "q_g", "k_g", "w_o", "b_o",
              "norm2_g", "norm2_b", "w_1", "b_1", "w_2", "b_2")
MATRIX_KEYS = ("w_qkv", "w_o", "w_1", "w_2")


def round_bf16(a):
    """Round an fp32 array to the nearest bf16 value (ties to even), kept as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def to_bf16_bits(a):
    """fp32 array holding bf16-representable values -> uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _draw(rng, shape, std, mean=0.0):
    return (mean + std * rng.standard_normal(shape)).astype(np.float32)


def make_inputs(cfg, seed=None, qk_scale=1.0, n_layers=None):
    """Return (x [n_union, d] fp32, g [d] fp32, layers: list of dict of fp32 arrays).

    ``qk_scale`` multiplies the q and k rows of every QKV weight after drawing
    (a sharper-softmax stress case); ``n_layers`` overrides the depth.
    """
    seed = cfg.get("seed", 0) if seed is None else seed
    rng = np.random.default_rng(seed)
    T, H, W = cfg["grid"]
    d, hd, dm = cfg["d"], cfg["head_dim"], cfg["mlp_hidden"]
    L = cfg["n_layers"] if n_layers is None else n_layers
    ln = cfg["norm"] == "ln"
    x = _draw(rng, (T * H * W, d), 1.0)
    g = _draw(rng, (d,), 1.0)
    layers = []
    for _ in range(L):
        p = {}
        p["norm1_g"] = _draw(rng, (d,), 0.02, 1.0)
        if ln:
            p["norm1_b"] = _draw(rng, (d,), 0.02)
        p["w_qkv"] = _draw(rng, (3 * d, d), 0.02)
        p["b_qkv"] = _draw(rng, (3 * d,), 0.02)
        if cfg["qk_norm"]:
            p["q_g"] = _draw(rng, (hd,), 0.02, 1.0)
            p["k_g"] = _draw(rng, (hd,), 0.02, 1.0)
        p["w_o"] = _draw(rng, (d, d), 0.02)
        p["b_o"] = _draw(rng, (d,), 0.02)
        p["norm2_g"] = _draw(rng, (d,), 0.02, 1.0)
        if ln:
            p["norm2_b"] = _draw(rng, (d,), 0.02)
        p["w_1"] = _draw(rng, (dm, d), 0.02)
        p["b_1"] = _draw(rng, (dm,), 0.02)
        p["w_2"] = _draw(rng, (d, dm), 0.02)
        p["b_2"] = _draw(rng, (d,), 0.02)
        if qk_scale != 1.0:
            p["w_qkv"][: 2 * d] *= np.float32(qk_scale)
        layers.append(p)
    if cfg["dtype"] == "bf16":
        x = round_bf16(x)
        g = round_bf16(g)
        for p in layers:
            for k in MATRIX_KEYS:
                p[k] = round_bf16(p[k])
    return x, g, layers
