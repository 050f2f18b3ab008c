"""Pins of the oracle's bf16 rounding and NF4 quantize / dequantize."""
import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import bf16, nf4


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(1)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-30, 30, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.f32_to_bf16_bits(x), ref)


def test_bf16_ties_go_to_even_and_exact_values_stay():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: even is 1.0.
    assert bf16.f32_to_bf16_bits(np.float32(1 + 2 ** -8)) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd mantissa) and 1+2^-6: goes up.
    assert bf16.f32_to_bf16_bits(np.float32(1 + 3 * 2 ** -8)) == 0x3F82
    vals = np.array([0.0, -0.0, 1.0, -2.5, 0.15625, 3.0e38], dtype=np.float32)
    vals = bf16.round_to_bf16(vals)
    assert np.array_equal(bf16.round_to_bf16(vals), vals)


# ------------------------------------------------------------------ codebook
def test_codebook_construction_properties():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert np.all(np.diff(c) > 0)
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    # Normal-quantile spacing, checked through the forward CDF (not the ppf the
    # oracle calls): scaled back by the largest quantile, the positive levels
    # sit at equally spaced probabilities from 1/2 to delta, the negative ones
    # likewise with one level fewer.
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    top = norm.ppf(delta)
    p_pos = norm.cdf(c[8:].astype(np.float64) * top)
    assert np.allclose(np.diff(p_pos), (delta - 0.5) / 8, atol=2e-7)
    neg_top = -norm.ppf(delta)  # the most negative level maps back to 1 - delta
    p_neg = norm.cdf(c[:7].astype(np.float64) * -neg_top)
    assert np.allclose(np.diff(p_neg), (delta - 0.5) / 7, atol=2e-7)
    # Largest gap is between the two most negative levels: half of it bounds
    # the round-trip error (0.1519...).
    gaps = np.diff(c.astype(np.float64))
    assert np.argmax(gaps) == 0 and abs(gaps.max() / 2 - 0.15190) < 1e-4


# ------------------------------------------------------------------ quantize
def _bits(x):
    return bf16.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_known_block_pins_nibble_order_and_codes():
    """A block whose elements are the bf16-rounded levels themselves (absmax 1)
    quantises to codes 0..15 in order; even element -> high nibble."""
    c = nf4.codebook()
    row = np.concatenate([c, c[::-1], c, c[::-1]])           # 64 elements
    packed, absmax = nf4.quantize(_bits(row)[None, :])
    assert absmax[0, 0] == 1.0
    codes = nf4.unpack_codes(packed)[0]
    assert np.array_equal(codes[:16], np.arange(16))
    assert np.array_equal(codes[16:32], np.arange(16)[::-1])
    assert packed[0, 0] == 0x01 and packed[0, 1] == 0x23 and packed[0, 7] == 0xEF


def test_quantize_invariants_random():
    g = np.random.default_rng(3)
    w = _bits(g.standard_normal((37, 256)) * 0.02)
    w[5, 64:128] = 0                                      # an all-zero block
    w[9, :64] = _bits(np.linspace(-1, 1, 64) * 1e-30)     # tiny magnitudes
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack_codes(packed)
    assert codes.max() <= 15
    x = bf16.bf16_bits_to_f32(w).reshape(37, 4, 64)
    assert np.array_equal(absmax, np.max(np.abs(x), axis=-1))
    # zero element -> zero code -> exactly 0.0 after dequantize
    assert np.all(codes[x.reshape(37, 256) == 0] == 7)
    assert np.all(codes[5, 64:128] == 7) and absmax[5, 1] == 0
    deq = nf4.dequantize_f32(packed, absmax).reshape(37, 4, 64)
    assert np.all(deq[x == 0] == 0)
    # the block's max-|x| element maps to +-1 and dequantizes to exactly +-absmax
    idx = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(x, idx[..., None], -1)[..., 0]
    dtop = np.take_along_axis(deq, idx[..., None], -1)[..., 0]
    assert np.array_equal(dtop, top)
    # round trip within absmax * half the largest gap (+1 ulp of the product)
    half_gap = float(np.max(np.diff(nf4.codebook().astype(np.float64)))) / 2
    err = np.abs(deq.astype(np.float64) - x)
    assert np.all(err <= absmax[..., None] * (half_gap + 1e-6))


def test_quantize_is_nearest_code_brute_force():
    """Loop over every element and all 16 levels on a small input."""
    g = np.random.default_rng(4)
    w = _bits(g.standard_normal((3, 128)))
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack_codes(packed)
    c = [float(v) for v in nf4.codebook()]
    x = bf16.bf16_bits_to_f32(w)
    for r in range(3):
        for k in range(128):
            a = absmax[r, k // 64]
            n = float(np.float32(x[r, k]) / np.float32(a))
            best = min(range(16), key=lambda j: (abs(n - c[j]), j))
            assert codes[r, k] == best


def test_quantize_f32_is_nearest_code_brute_force():
    """The float32 entry, on values no bf16 can hold: every element against all
    16 levels in plain Python floats."""
    g = np.random.default_rng(41)
    x = (g.standard_normal((3, 128)) * 0.02).astype(np.float32)
    assert not np.array_equal(bf16.bf16_bits_to_f32(bf16.f32_to_bf16_bits(x)), x)
    packed, absmax = nf4.quantize_f32(x)
    codes = nf4.unpack_codes(packed)
    c = [float(v) for v in nf4.codebook()]
    for r in range(3):
        for k in range(128):
            a = max(abs(float(v)) for v in x[r, (k // 64) * 64:(k // 64 + 1) * 64])
            assert absmax[r, k // 64] == np.float32(a)
            n = float(np.float32(x[r, k]) / np.float32(a))
            best = min(range(16), key=lambda j: (abs(n - c[j]), j))
            assert codes[r, k] == best


def test_quantize_f32_of_bf16_values_equals_the_bf16_entry():
    g = np.random.default_rng(42)
    w = _bits(g.standard_normal((5, 192)) * 0.02)
    p1, a1 = nf4.quantize(w)
    p2, a2 = nf4.quantize_f32(bf16.bf16_bits_to_f32(w))
    assert np.array_equal(p1, p2) and np.array_equal(a1.view(np.uint32), a2.view(np.uint32))


def test_quantize_f32_exact_midpoint_goes_to_lower_code():
    """A float32 input can sit exactly on a level midpoint (x / 1.0 = x): the
    lower level wins, the next float32 up takes the upper one."""
    c = nf4.codebook().astype(np.float64)
    j = next(j for j in range(8, 15) if float(np.float32((c[j] + c[j + 1]) / 2)) == (c[j] + c[j + 1]) / 2)
    m = np.float32((c[j] + c[j + 1]) / 2)
    row = np.zeros(64, dtype=np.float32)
    row[0] = 1.0                       # absmax 1: the quotient is the value itself
    row[1] = m
    row[2] = np.nextafter(m, np.float32(2))
    codes = nf4.unpack_codes(nf4.quantize_f32(row[None, :])[0])[0]
    assert codes[0] == 15 and codes[1] == j and codes[2] == j + 1


def test_quantize_monotone_within_block():
    g = np.random.default_rng(5)
    x = np.sort(g.standard_normal(64)).astype(np.float32)
    codes = nf4.unpack_codes(nf4.quantize(_bits(x)[None, :])[0])[0]
    xs = bf16.bf16_bits_to_f32(_bits(x))
    order = np.argsort(xs, kind="stable")
    assert np.all(np.diff(codes[order].astype(int)) >= 0)


def test_exact_midpoint_tie_goes_to_lower_code():
    """Four level midpoints are float32 numbers; a normalised value exactly on
    one goes to the lower level, the next float32 up goes to the upper one."""
    c = nf4.codebook().astype(np.float64)
    exact = [j for j in range(15) if float(np.float32((c[j] + c[j + 1]) / 2)) == (c[j] + c[j + 1]) / 2]
    assert len(exact) >= 2
    for j in exact:
        m = np.float32((c[j] + c[j + 1]) / 2)
        up = np.nextafter(m, np.float32(2))
        dn = np.nextafter(m, np.float32(-2))
        assert list(nf4.nearest_code(np.array([dn, m, up], dtype=np.float32))) == [j, j, j + 1]


def test_bf16_inputs_never_hit_a_midpoint():
    """Exhaustive over bf16 mantissa pairs: x / absmax never lands exactly on a
    level midpoint, so the tie rule never decides a bf16 weight.  The ratio is
    invariant to a common power of two, so absmax in [1, 2) and |x| <= absmax
    with every exponent down to the smallest midpoint's covers all cases."""
    c = nf4.codebook().astype(np.float64)
    mids = np.array([(c[j] + c[j + 1]) / 2 for j in range(15)])
    mant = (1 + np.arange(128) / 128).astype(np.float32)
    for ex in range(-6, 1):
        x = np.concatenate([mant, -mant]) * np.float32(2.0 ** ex)
        r = (x[:, None].astype(np.float32) / mant[None, :]).astype(np.float64)
        ok = np.abs(x[:, None]) <= mant[None, :]
        assert not np.isin(r[ok], mids).any()


def test_quantize_rejects_nonfinite_and_bad_shape():
    w = _bits(np.ones((2, 64)))
    w[1, 3] = 0x7FC0
    with pytest.raises(ValueError):
        nf4.quantize(w)
    with pytest.raises(ValueError):
        nf4.quantize(_bits(np.ones((2, 96))))


def test_dequant_bf16_is_rounded_float32_product():
    g = np.random.default_rng(6)
    w = _bits(g.standard_normal((8, 128)) * 0.02)
    packed, absmax = nf4.quantize(w)
    f32 = nf4.dequantize_f32(packed, absmax)
    # float32 product computed independently through float64 (exact) then rounded once
    c = nf4.codebook().astype(np.float64)
    exact = c[nf4.unpack_codes(packed)].reshape(8, 2, 64) * absmax[..., None].astype(np.float64)
    assert np.array_equal(f32, exact.reshape(8, 128).astype(np.float32))
    b = nf4.dequantize_bf16_bits(packed, absmax)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
