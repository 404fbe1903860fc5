"""Pins of the oracle's group quantizer and row packing.

The quantizer follows the affine map X_Q = round(X / S) - Z of the pgsm.cn
KV-cache quantization article (section 2.1), asymmetric over each group's own
range (KIVI, juejin.cn page, background section).  None of these tests re-types
the oracle's formula: they check properties the definition forces.
"""
import numpy as np
import pytest

from oracle import quantize_groups, dequantize, pack_rows, unpack_rows

RNG = np.random.default_rng(1234)


def _groups(n, G, kind, rng):
    if kind == "normal":
        x = rng.standard_normal((n, G)).astype(np.float32)
    elif kind == "outlier":
        x = rng.standard_normal((n, G)).astype(np.float32) * 10.0
    elif kind == "offset":
        x = rng.standard_normal((n, G)).astype(np.float32) * 0.01 + rng.uniform(-900, 900, (n, 1))
    elif kind == "tiny":
        x = rng.standard_normal((n, G)).astype(np.float32) * 1e-5
    elif kind == "near_const":
        base = rng.uniform(-50, 50, (n, 1)).astype(np.float32)
        x = np.repeat(base, G, axis=1)
        x[:, 0] = np.nextafter(base[:, 0].astype(np.float16), np.float16(np.inf))
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


KINDS = ["normal", "outlier", "offset", "tiny", "near_const"]


@pytest.mark.parametrize("bits", [2, 4])
def test_on_grid_values_are_recovered_exactly(bits):
    """x = s*(z + k) with s a power of two, z an integer and both ends of the
    level range present: the quantizer must return S = s, Z = z, codes = k and
    reconstruct x exactly.  This fixes the sign convention of Z (subtracted after
    rounding, so the group minimum maps to code 0)."""
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(7 + bits)
    for _ in range(200):
        e = int(rng.integers(-6, 5))
        s = np.float32(2.0 ** e)
        z = int(rng.integers(-40, 40))
        k = rng.integers(0, qmax + 1, size=32)
        k[rng.integers(0, 32)] = 0
        k[rng.integers(0, 32)] = qmax
        if k.min() != 0 or k.max() != qmax:
            continue
        x = (s * (z + k)).astype(np.float16)
        assert np.array_equal(x.astype(np.float32), (s * (z + k)).astype(np.float32))
        codes, S, Z = quantize_groups(x[None, :], bits)
        assert S[0] == s
        assert int(Z[0]) == z
        assert np.array_equal(codes[0], k.astype(np.uint8))
        assert np.array_equal(dequantize(codes, S, Z)[0], x.astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_min_max_and_monotone(bits, kind):
    qmax = (1 << bits) - 1
    x = _groups(500, 32, kind, RNG)
    codes, S, Z = quantize_groups(x, bits)
    xf = x.astype(np.float32)
    amin = xf.argmin(axis=1)
    amax = xf.argmax(axis=1)
    rows = np.arange(x.shape[0])
    const = xf.max(axis=1) == xf.min(axis=1)
    assert np.all(codes[rows, amin] == 0), "group minimum must map to code 0"
    top = codes[rows, amax][~const]
    assert np.all((top == qmax) | (top == qmax - 1))
    assert np.all(codes <= qmax)
    # monotone: ordering of inputs is preserved by the codes
    order = np.argsort(xf, axis=1, kind="stable")
    sc = np.take_along_axis(codes.astype(np.int32), order, axis=1)
    assert np.all(np.diff(sc, axis=1) >= 0)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("kind", KINDS)
def test_round_trip_error_bound(bits, kind):
    """|x - x_hat| <= S/2 (plus float32 rounding of the map itself)."""
    x = _groups(2000, 64, kind, RNG)
    codes, S, Z = quantize_groups(x, bits)
    xh = dequantize(codes, S, Z)
    xf = x.astype(np.float32)
    err = np.abs(xf.astype(np.float64) - xh.astype(np.float64))
    mag = np.maximum(np.abs(xf), np.abs(xh)).max(axis=1, keepdims=True).astype(np.float32)
    ulp = np.spacing(mag).astype(np.float64)
    bound = S[:, None].astype(np.float64) * 0.5 * (1 + 2.0 ** -20) + 4 * ulp
    assert np.all(err <= bound)


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_nearest_level_brute_force(bits):
    """Each code picks the level k + Z nearest to the float32 quotient x / S
    (ties to the even level), searched over every k in [0, 2^b - 1]."""
    qmax = (1 << bits) - 1
    x = _groups(300, 32, "normal", np.random.default_rng(99))
    codes, S, Z = quantize_groups(x, bits)
    xq = (x.astype(np.float32) / S[:, None]).astype(np.float32).astype(np.float64)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            best, bestd = None, None
            for k in range(qmax + 1):
                lvl = k + int(Z[i])
                dist = abs(xq[i, j] - lvl)
                if best is None or dist < bestd - 1e-12 or (abs(dist - bestd) <= 1e-12 and lvl % 2 == 0):
                    best, bestd = k, dist
            assert codes[i, j] == best, (i, j, xq[i, j], Z[i])


@pytest.mark.parametrize("bits", [2, 4])
def test_constant_groups_reconstruct_exactly(bits):
    vals = np.array([0.0, 1.0, -3.5, 1000.0, -65504.0, 6e-5, -2 ** -24], dtype=np.float16)
    x = np.repeat(vals[:, None], 32, axis=1)
    codes, S, Z = quantize_groups(x, bits)
    assert np.all(codes == 0)
    assert np.array_equal(dequantize(codes, S, Z), x.astype(np.float32))


def test_zero_point_fits_int16_at_worst_case():
    """Narrow ranges far from zero push |Z| toward (2^b - 1) * 2^11."""
    for bits, lim in ((2, 3 * 2048), (4, 15 * 2048)):
        x = np.array([[60000.0, 60032.0]], dtype=np.float16)  # one fp16 ulp apart
        _, S, Z = quantize_groups(x, bits)
        assert abs(int(Z[0])) <= lim


# ------------------------------------------------------------------ packing
def test_pack_literal_words():
    """Layout definition: channel c at bits [(c*b) % 32, +b) of word (c*b)//32."""
    row = np.zeros(128, np.uint8)
    row[0] = 3
    w = pack_rows(row, 2)
    assert w.shape == (8,) and w[0] == 0x3 and np.all(w[1:] == 0)
    row[:] = 0
    row[1] = 1
    assert pack_rows(row, 2)[0] == 0x4
    row[:] = 0
    row[15] = 2
    assert pack_rows(row, 2)[0] == 0x80000000
    row[:] = 0
    row[16] = 1
    w = pack_rows(row, 2)
    assert w[0] == 0 and w[1] == 1
    row[:] = 0
    row[7] = 15
    w = pack_rows(row, 4)
    assert w.shape == (16,) and w[0] == 0xF0000000
    row[:] = 0
    row[127] = 9
    assert pack_rows(row, 4)[15] == 0x90000000


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_brute_force_first_word(bits):
    """Every combination of the first few codes packs to the expected integer."""
    per = 32 // bits
    lim = 1 << bits
    k = 3 if bits == 4 else 5
    import itertools
    for combo in itertools.product(range(lim), repeat=k):
        row = np.zeros(128, np.uint8)
        row[:k] = combo
        expect = sum(c * (lim ** i) for i, c in enumerate(combo))
        w = pack_rows(row, bits)
        assert int(w[0]) == expect
        assert np.array_equal(unpack_rows(w, bits, 128), row)
    assert per * bits == 32


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_round_trip_random(bits):
    codes = RNG.integers(0, 1 << bits, size=(7, 5, 128)).astype(np.uint8)
    w = pack_rows(codes, bits)
    assert w.dtype == np.uint32 and w.shape == (7, 5, 128 * bits // 32)
    assert np.array_equal(unpack_rows(w, bits, 128), codes)
