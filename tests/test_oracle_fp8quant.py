"""Pins for the float64 oracle of the fp8 input step (CPU only).

The rotation is pinned to scipy's Hadamard construction (Sylvester recursion,
a different formulation from the oracle's popcount rule), to orthogonality,
to the closed form at d = 2 and to the spreading of a single spike; the e4m3
rounding to torch's float8_e4m3fn cast, to every code value, to hand-worked
ties and to saturation; the per-tensor quantisation to its defining
properties.  As for the attention oracles, the planted-mistake test at the
end runs every pin against copies of the module's source with one plausible
mistake edited in.
"""

import types

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle.fp8_quant as fq


def _signs(seed, d):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0)


def pin_hadamard_matches_scipy(m):
    for d in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        assert np.array_equal(m.hadamard_ref(d), scipy.linalg.hadamard(d)), d


def pin_hadamard_orthogonal(m):
    for d in (2, 64, 128):
        h = m.hadamard_ref(d)
        assert np.array_equal(h @ h.T, d * np.eye(d)), d


def pin_rotation_preserves_products(m):
    rng = np.random.default_rng(1)
    for d in (64, 128):
        x = rng.standard_normal((5, d))
        z = rng.standard_normal((7, d))
        s = _signs(d, d)
        got = m.rotate_ref(x, s) @ m.rotate_ref(z, s).T
        assert np.max(np.abs(got - x @ z.T)) < 1e-12, d


def pin_closed_form_d2(m):
    # R = diag(1, -1) [[1, 1], [1, -1]] / sqrt 2: (a, b) -> (a - b, a + b) / sqrt 2.
    a, b = 3.0, -1.25
    y = m.rotate_ref(np.array([[a, b]]), np.array([1.0, -1.0]))
    assert np.allclose(y, [[(a - b) / np.sqrt(2), (a + b) / np.sqrt(2)]], rtol=0, atol=1e-15)


def pin_spike_spreads_evenly(m):
    d, k, a = 128, 37, -5.0
    s = _signs(7, d)
    x = np.zeros((1, d))
    x[0, k] = a
    y = m.rotate_ref(x, s)[0]
    j = np.arange(d)
    parity = np.array([bin(k & jj).count("1") % 2 for jj in j])
    expect = a * s[k] * np.where(parity == 0, 1.0, -1.0) / np.sqrt(d)
    assert np.max(np.abs(y - expect)) < 1e-15


def pin_e4m3_every_code_round_trips(m):
    vals = m.e4m3_values()
    assert vals.shape == (0x7F,) and vals[0x7E] == 448.0 and vals[1] == 2.0 ** -9
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(m.e4m3_round_ref(vals), codes)
    neg = m.e4m3_round_ref(-vals[1:])
    assert np.array_equal(neg, codes[1:] | 0x80)
    assert np.array_equal(m.e4m3_decode_ref(codes | 0x80)[1:], -vals[1:])


def pin_e4m3_matches_torch(m):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * sc for sc in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    v = v.astype(np.float32)
    v = v[np.abs(v) <= 448.0].astype(np.float64)
    # Midpoints between neighbouring codes are exact float32 values: ties.
    ref_vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = (ref_vals[:-1] + ref_vals[1:]) / 2
    v = np.concatenate([v, mids, -mids])
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = m.e4m3_round_ref(v)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first at {v[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


def pin_e4m3_hand_worked(m):
    # 1.0 = 0x38, 1.125 = 0x39, 1.25 = 0x3A: ties go to the even mantissa.
    assert m.e4m3_round_ref(np.array([1.0625]))[0] == 0x38
    assert m.e4m3_round_ref(np.array([1.1875]))[0] == 0x3A
    # Subnormals: 2^-9 = 0x01, 2^-10 ties to 0, 3 * 2^-10 ties to 0x02.
    assert m.e4m3_round_ref(np.array([2.0 ** -10]))[0] == 0x00
    assert m.e4m3_round_ref(np.array([3 * 2.0 ** -10]))[0] == 0x02
    # Saturation at ±448 (0x7E / 0xFE); 0x7F is NaN and never produced.
    assert list(m.e4m3_round_ref(np.array([460.0, 1e6, -1e6]))) == [0x7E, 0x7E, 0xFE]


def pin_quantisation_properties(m):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 128)) * 3.0
    x[3, 17] = 40.0   # an outlier channel entry
    for signs in (None, _signs(11, 128)):
        codes, ds = m.rotate_quantize_ref(x, signs)
        y = m.rotate_ref(x, signs) if signs is not None else x
        assert ds == pytest.approx(np.abs(y).max() / 448.0, rel=1e-15)
        deq = m.e4m3_decode_ref(codes) * ds
        i = np.unravel_index(np.argmax(np.abs(y)), y.shape)
        assert abs(deq[i]) == pytest.approx(np.abs(y).max(), rel=1e-15)
        # Relative half-step of a 3-bit mantissa, or half the subnormal step.
        assert np.all(np.abs(deq - y) <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10 * ds) + 1e-12)
    # The rotation spreads the outlier: the quantised scores of a row pair
    # are closer to the true ones than without it (incoherent processing).
    s = _signs(11, 128)
    q = rng.standard_normal((64, 128))
    q[:, 5] *= 30.0
    k = rng.standard_normal((64, 128))
    k[:, 5] *= 30.0
    exact = q @ k.T
    (cq, dq), (ck, dk) = m.rotate_quantize_ref(q), m.rotate_quantize_ref(k)
    plain = (m.e4m3_decode_ref(cq) * dq) @ (m.e4m3_decode_ref(ck) * dk).T
    (cq, dq), (ck, dk) = m.rotate_quantize_ref(q, s), m.rotate_quantize_ref(k, s)
    rot = (m.e4m3_decode_ref(cq) * dq) @ (m.e4m3_decode_ref(ck) * dk).T
    assert np.abs(rot - exact).mean() < 0.8 * np.abs(plain - exact).mean()


PINS = [pin_hadamard_matches_scipy, pin_hadamard_orthogonal, pin_rotation_preserves_products,
        pin_closed_form_d2, pin_spike_spreads_evenly, pin_e4m3_every_code_round_trips,
        pin_e4m3_matches_torch, pin_e4m3_hand_worked, pin_quantisation_properties]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(fq)


MUTATIONS = {
    "or_instead_of_and": ("bits = np.bitwise_and.outer(i, i)", "bits = np.bitwise_or.outer(i, i)"),
    "no_normalisation": ("return (s[:, None] * hadamard_ref(d)) / np.sqrt(d)",
                         "return (s[:, None] * hadamard_ref(d))"),
    "signs_on_columns": ("return (s[:, None] * hadamard_ref(d)) / np.sqrt(d)",
                         "return (hadamard_ref(d) * s[None, :]) / np.sqrt(d)"),
    "signs_ignored": ("return (s[:, None] * hadamard_ref(d)) / np.sqrt(d)",
                      "return hadamard_ref(d) / np.sqrt(d)"),
    "subnormal_step": ("np.where(e == 0, m * 2.0 ** -9,", "np.where(e == 0, m * 2.0 ** -10,"),
    "exponent_bias": ("(8 + m) * 2.0 ** (e.astype(np.float64) - 10)",
                      "(8 + m) * 2.0 ** (e.astype(np.float64) - 9)"),
    "ties_to_odd": ("((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    "ties_away": ("((d_hi == d_lo) & (hi % 2 == 0))", "(d_hi == d_lo)"),
    "sign_dropped": ("np.where(np.signbit(v), code | 0x80, code)",
                     "np.where(np.signbit(v), code, code)"),
    "descale_240": ("descale = amax / E4M3_MAX if amax > 0 else 1.0",
                    "descale = amax / 240.0 if amax > 0 else 1.0"),
    "amax_signed": ("amax = float(np.abs(y).max()) if y.size else 0.0",
                    "amax = float(y.max()) if y.size else 0.0"),
    "rotation_skipped": ("y = rotate_ref(x, signs) if signs is not None else x", "y = x"),
}


def _mutant(old, new):
    with open(fq.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("fp8_quant_mutant")
    exec(compile(src.replace(old, new), "fp8_quant_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
