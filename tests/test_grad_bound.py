"""CPU checks of the element-wise gradient bound used by the backward GPU tests.

tests/parity.py bounds each element of dQ, dK, dV by the roundings the
kernels make (bf16 P and dS operands, fp32 sums, bf16 outputs, Delta from the
bf16 forward output).  Here the kernels' arithmetic is emulated in float32
with bf16 rounding at the same places (numpy, on the CPU), and

  * every element of the emulated gradients lies within the bound of the
    float64 oracle, for causal and non-causal, GQA and ragged shapes;
  * planted mistakes in the emulation (Delta left out of dS, P normalised
    with an LSE off by 0.01, dS rounded to 4 mantissa bits instead of 8, one
    key of dV dropped) break the bound for some elements,

so the bound is neither looser than the arithmetic needs nor so loose that
errors of that size pass.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import grad_error_bounds

LOG2E = 1.4426950408889634


def _bf16(x):
    return datagen.f64_from_bf16_bits(datagen.bf16_bits_from_f32(np.asarray(x, np.float32)))


def _round_bits(x, bits):
    """Round to `bits` significant bits (nearest, ties away), for the planted
    coarse rounding."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def _emulated_bwd(q, k, v, do, o_given, lse_given, scale, causal, fault=None):
    """The backward kernels' arithmetic in float32 with their bf16 roundings."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    f = np.float32
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    c = f(scale * LOG2E)
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            q32, k32, v32, do32 = (x.astype(f) for x in (q[b, h], k[b, g], v[b, g], do[b, h]))
            lse = lse_given[b, h].astype(f)
            if fault == "lse":
                lse = lse + f(0.01)
            s = q32 @ k32.T
            allowed = oracle.allowed_keys(np.arange(Nq), Nq, Nk, causal)
            p = np.exp2(s * c - (lse * f(LOG2E))[:, None]).astype(f)
            p = np.where(allowed, p, f(0))
            delta = (do32 * o_given[b, h].astype(f)).sum(axis=1, dtype=f)
            if fault == "delta":
                delta = delta * f(0)
            dp = do32 @ v32.T
            ds = p * (dp - delta[:, None])
            ds_b = _round_bits(ds, 4) if fault == "coarse" else _bf16(ds)
            p_b = _bf16(p)
            if fault == "dropkey":
                p_b[:, Nk // 2] = 0.0
            dq[b, h] = _bf16((ds_b.astype(f) @ k32) * f(scale))
            dk[b, g] += (ds_b.astype(f).T @ q32)
            dv[b, g] += (p_b.astype(f).T @ do32)
    return dq, _bf16(dk.astype(f) * f(scale)), _bf16(dv.astype(f))


CASES = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 2, 1, 70, 70, 32, True),
    (1, 2, 2, 40, 150, 64, False),
    (1, 4, 2, 33, 90, 32, True),
]


def _setup(shape, seed):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    cfg = datagen.fwd_config("bound", B, Hq, Nq, d, causal, seed=seed, Hkv=Hkv, Nk=Nk)
    qb, kb, vb, dob = datagen.make_bwd_inputs(cfg)
    q, k, v, do = (datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb, dob))
    o, lse = oracle.attention_ref(q, k, v, cfg.scale, causal)
    o_given = _bf16(o)
    lse_given = lse.astype(np.float32).astype(np.float64)
    rq, rk, rv = oracle.attention_bwd_ref(q, k, v, do, cfg.scale, causal)
    refs = dict(Q=rq, K=rk, V=rv)
    bounds = grad_error_bounds(q, k, v, do, o_given, lse_given, cfg.scale, causal, refs)
    return cfg, (q, k, v, do, o_given, lse_given), refs, bounds


@pytest.mark.parametrize("shape", CASES)
def test_emulated_kernel_arithmetic_is_within_the_bound(shape):
    cfg, args, refs, bounds = _setup(shape, 910)
    got = dict(zip("QKV", _emulated_bwd(*args, cfg.scale, cfg.causal)))
    for name in "QKV":
        err = np.abs(got[name] - refs[name])
        assert np.all(err <= bounds[name]), (name, float((err / bounds[name]).max()))
        # the bound is not vacuous: it is below the element's own scale
        assert float(np.median(bounds[name])) < 0.1 * float(np.median(np.abs(refs[name])) + 1e-30)


@pytest.mark.parametrize("fault", ["delta", "lse", "coarse", "dropkey"])
def test_planted_mistakes_break_the_bound(fault):
    cfg, args, refs, bounds = _setup(CASES[0], 911)
    got = dict(zip("QKV", _emulated_bwd(*args, cfg.scale, cfg.causal, fault=fault)))
    broken = [name for name in "QKV" if np.any(np.abs(got[name] - refs[name]) > bounds[name])]
    assert broken, f"planted mistake '{fault}' stayed within the bound"
