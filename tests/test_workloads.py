"""The seeded input generators (they hold none of the method's arithmetic)."""
from fractions import Fraction

import numpy as np

import workloads as wl


def test_splitmix64_published_vector():
    # Reference outputs of SplitMix64 started from state 1234567.
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [int(v) for v in wl.splitmix64(1234567, 0, 5)] == want


def test_normal_is_counter_based():
    a = wl.normal(5, 1001)
    assert np.array_equal(wl.normal(5, 600, start=401), a[401:])
    assert np.array_equal(wl.normal(5, 3, start=7), a[7:10])
    assert not np.array_equal(wl.normal(6, 10), a[:10])


def test_normal_moments():
    z = wl.normal(3, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 5e-3
    assert abs(np.mean(np.abs(z) > 1.96) - 0.05) < 2e-3


def test_bf16_rne_against_rationals():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-20, 20, 3000))
    # add exact ties: values halfway between bf16 neighbours
    base = wl.bf16_bits_to_f32(wl.bf16_rne_bits(v[:200])).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.abs(base))) - 7)
    v = np.concatenate([v, base + ulp / 2, base - ulp / 2])
    bits = wl.bf16_rne_bits(v)
    got = wl.bf16_bits_to_f32(bits).astype(np.float64)
    for val, g in zip(v, got):
        e = int(np.floor(np.log2(abs(val))))
        q = Fraction(2) ** (e - 7)
        n = Fraction(val) / q
        fl = n.numerator // n.denominator
        frac = n - fl
        r = fl + 1 if frac > Fraction(1, 2) else fl if frac < Fraction(1, 2) else (fl if fl % 2 == 0 else fl + 1)
        assert Fraction(g) == r * q, (val, g)


def test_weights_shape_and_scale():
    W = wl.weights(64, 256, 1)
    assert W.dtype == np.float32 and W.shape == (64, 256)
    assert abs(W.std() - 0.02) < 1e-3
    assert np.array_equal(W, wl.weights(64, 256, 1))


def test_activation_recipes():
    x = wl.bf16_bits_to_f32(wl.activation(2048, 3, "unit_rms")).astype(np.float64)
    assert abs(np.sqrt(np.mean(x * x)) - 1) < 1e-2
    s = wl.bf16_bits_to_f32(wl.activation(11008, 1, "swiglu")).astype(np.float64)
    assert s.min() < 0 < s.max()
    X = wl.activations(4, 512, 2, "normal")
    assert X.shape == (4, 512) and not np.array_equal(X[0], X[1])
