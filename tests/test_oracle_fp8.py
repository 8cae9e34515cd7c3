"""Pins for the oracle's e4m3 quantiser (CPU): bit layout, brute-force nearest
value with ties to even, and torch's own float8_e4m3fn conversion."""
import numpy as np
import torch

from oracle import fp8


def _finite_sorted():
    t = fp8.e4m3_decode_table()
    codes = [c for c in range(256) if np.isfinite(t[c])]
    return t, codes


def test_decode_table_layout():
    t, codes = _finite_sorted()
    assert len(codes) == 254                       # 2 NaN codes, no infinities
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0   # largest finite
    assert t[0x08] == 2.0 ** -6                     # smallest normal
    assert t[0x01] == 2.0 ** -9                     # smallest subnormal
    assert t[0x38] == 1.0
    # torch's dtype agrees on every finite code
    tt = torch.tensor(list(range(256)), dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    fin = np.isfinite(t)
    assert np.array_equal(tt[fin], t[fin].astype(np.float32))


def _brute_round(v):
    """Nearest finite e4m3 value by exhaustive search; ties go to the even code."""
    t, codes = _finite_sorted()
    v = float(np.clip(np.float32(v), -448.0, 448.0))
    best = None
    for c in codes:
        dist = abs(t[c] - v)
        key = (dist, c & 1)         # even mantissa LSB wins a tie
        if best is None or key < best[0]:
            best = (key, t[c])
    return best[1]


def test_round_matches_brute_force_on_midpoints_and_randoms():
    t, codes = _finite_sorted()
    pos = sorted(set(abs(t[c]) for c in codes))
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        m = (a + b) / 2
        vals += [a, m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))]
    rng = np.random.default_rng(0)
    vals += list(rng.standard_normal(3000) * 40) + list(rng.standard_normal(500) * 0.01)
    vals += [500.0, 448.0, 464.0, 463.99, 1e9]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    got = fp8.round_e4m3(vals)
    exp = np.array([_brute_round(v) for v in vals])
    assert np.array_equal(got, exp)


def test_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    v = np.clip(rng.standard_normal(20000).astype(np.float32) * 60, -448, 448)
    tor = torch.from_numpy(v).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(fp8.round_e4m3(v).astype(np.float32), tor)


def test_encode_roundtrip():
    t, codes = _finite_sorted()
    vals = np.array([t[c] for c in codes])
    enc = fp8.encode_e4m3(vals)
    # +0 and -0 both decode to 0; every other code must round-trip
    for c, e in zip(codes, enc):
        if t[c] == 0:
            assert e in (0x00, 0x80)
        else:
            assert e == c


def test_tensor_scale_and_fake_quant():
    a = np.array([[0.5, -3.0], [1.25, 2.0]], dtype=np.float32)
    s = fp8.tensor_scale(a)
    assert s == np.float32(3.0) / np.float32(448.0)
    q, s2 = fp8.fake_quant(a)
    assert s2 == s and np.max(np.abs(q)) == 448.0
    assert fp8.tensor_scale(np.zeros((3, 3), np.float32)) == 1.0
    # dequantised values are within half a quantum of the input
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    q, s = fp8.fake_quant(x)
    rel = np.abs(q * s - x) / np.maximum(np.abs(x), 2.0 ** -6 * s)
    assert np.max(rel) <= 2.0 ** -4 + 1e-6


def test_fp8_linear_on_exactly_representable_operands():
    """Operands already on the e4m3 grid times a power-of-two scale quantise
    without error, so the scaled GEMM must equal the plain product plus bias;
    a wrong scale product, a transposed operand or a dropped bias fails."""
    table = fp8.e4m3_decode_table()
    fin = table[np.isfinite(table)]
    rng = np.random.default_rng(4)
    for sx, sw in ((1.0, 1.0), (2.0, 0.25), (0.5, 8.0)):
        xq = rng.choice(fin, size=(5, 16))
        wq = rng.choice(fin, size=(7, 16))
        xq[0, 0], wq[0, 0] = 448.0, -448.0           # absmax 448 -> scale = sx, sw exactly
        x, w = (xq * sx).astype(np.float32), (wq * sw).astype(np.float32)
        b = rng.standard_normal(7)
        assert fp8.tensor_scale(x) == np.float32(sx) and fp8.tensor_scale(w) == np.float32(sw)
        got = fp8.fp8_linear(x, w, b)
        ref = x.astype(np.float64) @ w.astype(np.float64).T + b
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-9)
    # a non-square, non-symmetric case where a transposed operand cannot pass
    x = (np.arange(12, dtype=np.float32).reshape(3, 4) - 5) * 0.5
    w = (np.arange(8, dtype=np.float32).reshape(2, 4) + 1)
    assert np.allclose(fp8.fp8_linear(x, w, np.zeros(2)), fp8.round_e4m3(x / fp8.tensor_scale(x)) *
                       fp8.tensor_scale(x) @ (fp8.round_e4m3(w / fp8.tensor_scale(w)) * fp8.tensor_scale(w)).T)
