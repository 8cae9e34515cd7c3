"""FP8 (OCP e4m3) fake quantisation and the per-tensor scaled GEMM.

Pages: FP8 appears as "V0 + FP8" (Table S5), "FP8 MLP layers only" and
"TileShare-4 + FP8" (Table S2) and "up to 1.96x with FP8" (abstract); the
format and the scaling are not given.  Reading taken here: OCP e4m3 (1 sign,
4 exponent bits with bias 7, 3 mantissa bits, largest finite 448, no
infinities, S.1111.111 is NaN); one scale per operand tensor of each GEMM
call, s = absmax/448 (s = 1 when the tensor is all zero); codes by round to
nearest even with saturation at +-448; C = (A_q W_q^T) s_A s_W + b with the
product accumulated exactly (float64 here).

The quantisation decision is taken in fp32, as the kernel takes it: the
operand is rounded to fp32, divided by the fp32 scale with one IEEE fp32
division, clamped to +-448 and rounded to the e4m3 grid.
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table():
    """Value of each of the 256 codes from the bit layout (NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def round_e4m3(v):
    """Round fp32 values to the e4m3 grid: nearest, ties to even, saturate +-448."""
    v = np.clip(np.asarray(v, dtype=np.float32).astype(np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(v)
    _, ex = np.frexp(a)               # a = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)        # binade exponent, subnormals share 2**-6
    quantum = np.ldexp(1.0, e - 3)    # 3 mantissa bits
    q = np.rint(a / quantum) * quantum
    return np.where(v < 0, -q, q)


def encode_e4m3(v):
    """Codes (uint8) of values already on the e4m3 grid."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** -6
    efield = np.where(normal, e + 7, 0)
    mant = np.where(normal, np.rint(a / np.ldexp(1.0, e) * 8.0) - 8.0, np.rint(a / 2.0 ** -9))
    return (sign | (efield.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def tensor_scale(a):
    """fp32 per-tensor scale absmax/448 (1 for an all-zero tensor)."""
    amax = np.float32(np.max(np.abs(np.asarray(a, dtype=np.float32)))) if np.size(a) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def fake_quant(a):
    """Return (values on the e4m3 grid as float64, fp32 scale) for tensor a."""
    a32 = np.asarray(a, dtype=np.float32)
    s = tensor_scale(a32)
    return round_e4m3(a32 / s), s


def fp8_linear(x, w, b):
    qx, sx = fake_quant(x)
    qw, sw = fake_quant(w)
    return (qx @ qw.T) * (np.float64(sx) * np.float64(sw)) + np.asarray(b, dtype=np.float64)
