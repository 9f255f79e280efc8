"""The three-piece bf16 split behind f32_math = BF16X3, emulated in numpy.

The single-write transposed-conv kernel (with f32_math = BF16X3) splits every
fp32 operand v into bf16 pieces, rounding to nearest even at each stage:
v1 = bf16(v), v2 = bf16(v - v1), v3 = bf16(v - v1 - v2), the subtractions in
fp32, and sums the six leading piece products w_i x_j (i + j <= 4) in fp32.
These CPU tests pin the two facts that make the result fp32-accurate: the
pieces reconstruct v exactly (each subtraction is exact and v3 needs no
rounding), and the three dropped products stay within about 2^-23 |w x|
(two units in the last place of one fp32 product).  They check
the arithmetic claim, not the kernel (the GPU parity tests do that).
"""
import numpy as np


def bf16_rne(a):
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding that value."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def split3(v):
    v = np.asarray(v, dtype=np.float32)
    p1 = bf16_rne(v)
    r1 = (v - p1).astype(np.float32)
    p2 = bf16_rne(r1)
    r2 = (r1 - p2).astype(np.float32)
    p3 = bf16_rne(r2)
    return p1, p2, p3, r1, r2


def _samples(n=200000, seed=7):
    rng = np.random.default_rng(seed)
    normal = rng.standard_normal(n).astype(np.float32)
    spread = (rng.standard_normal(n) * 10.0 ** rng.uniform(-30, 30, n)).astype(np.float32)
    bits = rng.integers(0x00800000, 0x7F000000, n, dtype=np.uint32).view(np.float32)  # normal fp32
    edge = np.array([1.0, -1.0, 1.0 + 2 ** -23, 1.0 - 2 ** -24, 2 ** -100, 3.0e38, -3.0e38,
                     np.float32(np.pi), 1.0 / 3.0, 65504.0, 0.5 + 2 ** -9, 0.5 + 2 ** -10 + 2 ** -20],
                    dtype=np.float32)
    return np.concatenate([normal, spread, bits, -bits, edge])


def test_bf16_rounding_matches_torch():
    import torch
    v = _samples(20000)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_rne(v), ref)


def test_three_pieces_reconstruct_every_fp32_exactly():
    # every fp32 of magnitude 2^-100 or more (below that, the third piece can
    # fall among bf16 subnormals, the documented exception)
    v = _samples()
    v = v[np.abs(v) >= 2.0 ** -100]
    p1, p2, p3, r1, r2 = split3(v)
    # each remainder is exact in fp32 (Sterbenz), and the last one needs no rounding
    np.testing.assert_array_equal(r1.astype(np.float64), v.astype(np.float64) - p1.astype(np.float64))
    np.testing.assert_array_equal(r2.astype(np.float64), r1.astype(np.float64) - p2.astype(np.float64))
    np.testing.assert_array_equal(p3, r2)
    np.testing.assert_array_equal(p1.astype(np.float64) + p2 + p3, v.astype(np.float64))
    # sizes: |v2| <= 2^-8 |v|, |v3| <= 2^-16 |v| (round to nearest at 8 significant bits)
    a = np.abs(v.astype(np.float64))
    assert (np.abs(p2) <= 2.0 ** -8 * a).all()
    assert (np.abs(p3) <= 2.0 ** -16 * a).all()


def test_six_products_are_within_two_units_in_the_last_place():
    w = _samples(50000, seed=3)
    x = _samples(50000, seed=5)
    n = min(len(w), len(x))
    w, x = w[:n], x[:n]
    # magnitudes whose products and pieces stay normal in fp32
    lo, hi = 2.0 ** -60, 2.0 ** 60
    keep = (np.abs(w) > lo) & (np.abs(x) > lo) & (np.abs(w) < hi) & (np.abs(x) < hi)
    w, x = w[keep].astype(np.float32), x[keep].astype(np.float32)
    w1, w2, w3, _, _ = split3(w)
    x1, x2, x3, _, _ = split3(x)
    f = lambda a: a.astype(np.float64)
    six = (f(w1) * f(x1) + f(w1) * f(x2) + f(w2) * f(x1) + f(w1) * f(x3) + f(w2) * f(x2)
           + f(w3) * f(x1))
    exact = f(w) * f(x)
    rel = np.abs(six - exact) / np.abs(exact)
    assert rel.max() <= 2.0 ** -23, rel.max()
    # each piece product is exact in fp32 (8 x 8 significant bits)
    for a, b in ((w1, x1), (w1, x2), (w2, x1), (w1, x3), (w2, x2), (w3, x1)):
        prod64 = f(a) * f(b)
        ok = np.abs(prod64) > 1e-37   # away from fp32 subnormals
        assert (f((a * b).astype(np.float32))[ok] == prod64[ok]).all()
