"""Pins for the float64 backward oracle (CPU only).

The gradient oracle is pinned to things other than itself: PyTorch autograd
through float64 scaled_dot_product_attention, central finite differences of
the forward oracle, dV from the forward oracle's probabilities, closed forms
and invariants.  As for the forward oracle, every pin takes the oracle module,
and the planted-mistake test at the end runs all pins against copies of the
backward oracle's source with one plausible mistake edited in.
"""

import types

import numpy as np
import pytest
import torch

import oracle
import oracle.attention_bwd as oracle_bwd


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand(seed, B, Hq, Hkv, Nq, Nk, d):
    r = _rng(seed)
    return (r.standard_normal((B, Hq, Nq, d)), r.standard_normal((B, Hkv, Nk, d)),
            r.standard_normal((B, Hkv, Nk, d)), r.standard_normal((B, Hq, Nq, d)))


def _torch_grads(q, k, v, do, scale, causal):
    """Autograd through torch's float64 SDPA; K/V heads repeated for GQA and a
    bottom-right aligned boolean mask when causal."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kr = tk.repeat_interleave(Hq // Hkv, dim=1)
    vr = tv.repeat_interleave(Hq // Hkv, dim=1)
    mask = None
    if causal:
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        mask = j <= i + (Nk - Nq)
    out = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, attn_mask=mask,
                                                           scale=scale)
    out.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_torch_autograd(mod):
    """Autograd of torch's float64 attention, MHA and GQA, with and without
    the causal mask, square and rectangular."""
    cases = [(1, 2, 2, 9, 9, 5, 0.37, False), (2, 4, 2, 9, 9, 5, 0.37, True),
             (1, 6, 3, 5, 11, 4, 0.6, True), (1, 4, 1, 7, 3, 6, 0.25, False)]
    for i, (B, Hq, Hkv, Nq, Nk, d, sc, causal) in enumerate(cases):
        q, k, v, do = _rand(100 + i, B, Hq, Hkv, Nq, Nk, d)
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, sc, causal)
        tq, tk, tv = _torch_grads(q, k, v, do, sc, causal)
        _close(dq, tq, 1e-12, f"dQ case {i}")
        _close(dk, tk, 1e-12, f"dK case {i}")
        _close(dv, tv, 1e-12, f"dV case {i}")


def pin_finite_differences(mod):
    """Central differences of L = sum(dO * O) with O from the forward oracle."""
    for causal in (False, True):
        q, k, v, do = _rand(7 + causal, 1, 2, 1, 4, 5, 3)
        sc = 0.45
        dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, sc, causal)

        def loss(q_, k_, v_):
            o, _ = oracle.attention_ref(q_, k_, v_, sc, causal)
            return float(np.sum(o * do))

        h = 1e-5
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name] = xp
                args_m[name] = xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                            - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            _close(g, num, 1e-8, f"finite differences d{name} causal={causal}")


def pin_dv_from_forward_probabilities(mod):
    """dV = P^T dO with P taken from the forward oracle."""
    q, k, v, do = _rand(21, 1, 1, 1, 13, 17, 6)
    for causal in (False, True):
        _, _, p = oracle.attention_head_ref(q[0, 0], k[0, 0], v[0, 0], 0.3, causal, return_p=True)
        _, _, dv = mod.attention_bwd_ref(q, k, v, do, 0.3, causal)
        _close(dv[0, 0], p.T @ do[0, 0], 1e-12, f"dV = P^T dO causal={causal}")


def pin_single_key(mod):
    """One key: P = 1, so dS = 0 (dQ = dK = 0) and dV = sum of the group's dO rows."""
    q, k, v, do = _rand(31, 1, 4, 2, 6, 1, 5)
    dq, dk, dv = mod.attention_bwd_ref(q, k, v, do, 0.5, False)
    _close(dq, np.zeros_like(dq), 1e-13, "single key dQ")
    _close(dk, np.zeros_like(dk), 1e-13, "single key dK")
    want = do.reshape(1, 2, 2, 6, 5).sum(axis=(2, 3))[:, :, None, :]
    _close(dv, want, 1e-12, "single key dV")


def pin_zero_queries(mod):
    """Q = 0, no mask: P = 1/Nk for every key, so every dV row is the group's
    dO summed over rows and heads, divided by Nk."""
    _, k, v, do = _rand(41, 2, 2, 1, 5, 7, 4)
    q = np.zeros((2, 2, 5, 4))
    _, _, dv = mod.attention_bwd_ref(q, k, v, do, 0.9, False)
    want = np.repeat(do.sum(axis=(1, 2))[:, None, None, :] / 7, 7, axis=2)
    _close(dv, want, 1e-12, "zero queries dV")


def pin_identical_keys(mod):
    """All keys equal: dS rows sum to zero, so dQ = scale dS K = 0."""
    q, k, v, do = _rand(51, 1, 2, 2, 6, 6, 3)
    k[:] = k[:, :, :1, :]
    for causal in (False, True):
        dq, _, _ = mod.attention_bwd_ref(q, k, v, do, 0.7, causal)
        _close(dq, np.zeros_like(dq), 1e-12, f"identical keys dQ causal={causal}")


def pin_dk_sums_to_zero(mod):
    """Every dS row sums to zero, so the key gradients of a head sum to zero."""
    q, k, v, do = _rand(61, 2, 4, 2, 10, 10, 5)
    for causal in (False, True):
        _, dk, _ = mod.attention_bwd_ref(q, k, v, do, 0.4, causal)
        _close(dk.sum(axis=2), np.zeros((2, 2, 5)), 1e-12, f"sum_j dK_j causal={causal}")


def pin_shift_invariance(mod):
    """Adding one vector to every key shifts each score row by a constant:
    P, dS and all three gradients are unchanged."""
    q, k, v, do = _rand(71, 1, 2, 1, 8, 8, 4)
    u = _rng(72).standard_normal(4)
    for causal in (False, True):
        a = mod.attention_bwd_ref(q, k, v, do, 0.6, causal)
        b = mod.attention_bwd_ref(q, k + u, v, do, 0.6, causal)
        for x, y, n in zip(a, b, ("dQ", "dK", "dV")):
            _close(x, y, 1e-11, f"shift invariance {n} causal={causal}")


def pin_linearity_in_do(mod):
    """The gradients are linear in dO."""
    q, k, v, do1 = _rand(81, 1, 2, 2, 7, 9, 3)
    do2 = _rng(82).standard_normal(do1.shape)
    a1 = mod.attention_bwd_ref(q, k, v, do1, 0.5, True)
    a2 = mod.attention_bwd_ref(q, k, v, do2, 0.5, True)
    c = mod.attention_bwd_ref(q, k, v, 2.0 * do1 - 3.0 * do2, 0.5, True)
    for x1, x2, y, n in zip(a1, a2, c, ("dQ", "dK", "dV")):
        _close(y, 2.0 * x1 - 3.0 * x2, 1e-11, f"linearity {n}")


def pin_row_and_key_subsets(mod):
    """dQ of a row subset and dK/dV of a key subset equal the matching slices of
    the full result (the sampled GPU checks rely on this)."""
    q, k, v, do = _rand(91, 1, 1, 1, 40, 40, 4)
    full = mod.attention_bwd_head_ref(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, True)
    rows = np.array([0, 3, 17, 39])
    keys = np.array([1, 2, 30, 39])
    dq, dk, dv = mod.attention_bwd_head_ref(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, True,
                                            rows=rows, keys=keys)
    _close(dq, full[0][rows], 1e-13, "dQ rows")
    _close(dk, full[1][keys], 1e-13, "dK keys")
    _close(dv, full[2][keys], 1e-13, "dV keys")


PINS = [pin_torch_autograd, pin_finite_differences, pin_dv_from_forward_probabilities,
        pin_single_key, pin_zero_queries, pin_identical_keys, pin_dk_sums_to_zero,
        pin_shift_invariance, pin_linearity_in_do, pin_row_and_key_subsets]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_bwd_pin(pin):
    pin(oracle)


# ---------------------------------------------------------------------------
# Planted mistakes in copies of oracle/attention_bwd.py
# ---------------------------------------------------------------------------

MUTATIONS = {
    "dp_uses_keys": ("dp = dob @ vg.T", "dp = dob @ kg.T"),
    "ds_drops_rowsum": ("ds = p * (dp - dsum)", "ds = p * dp"),
    "ds_drops_p": ("ds = p * (dp - dsum)", "ds = (dp - dsum)"),
    "rowsum_wrong_axis": ("dsum = (p * dp).sum(axis=1, keepdims=True)",
                          "dsum = (p * dp).sum(axis=0, keepdims=True)"),
    "softmax_unnormalised": ("p = e / e.sum(axis=1, keepdims=True)", "p = e"),
    "mask_ignored": ("s = np.where(allowed_keys(rb, Nq, Nk, causal), s, -np.inf)", "s = s"),
    "dq_drops_scale": ("dq[r0:r0 + step] = scale * (ds @ kg)", "dq[r0:r0 + step] = (ds @ kg)"),
    "dq_uses_values": ("dq[r0:r0 + step] = scale * (ds @ kg)",
                       "dq[r0:r0 + step] = scale * (ds @ vg)"),
    "dk_uses_do": ("dk += scale * (ds[:, ksel].T @ qh[rb])",
                   "dk += scale * (ds[:, ksel].T @ doh[rb])"),
    "dk_drops_scale": ("dk += scale * (ds[:, ksel].T @ qh[rb])",
                       "dk += (ds[:, ksel].T @ qh[rb])"),
    "dv_uses_ds": ("dv += p[:, ksel].T @ doh[rb]", "dv += ds[:, ksel].T @ doh[rb]"),
    "gqa_modulo": ("g = h // group", "g = h % Hkv"),
    "gqa_no_sum": ("dk[b, g] += dk_h", "dk[b, g] = dk_h"),
}


def _mutant(old, new):
    with open(oracle_bwd.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
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
