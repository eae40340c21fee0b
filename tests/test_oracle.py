"""Pins for the float64 oracle (CPU only).

The oracle is the reference every GPU result is judged against, so it is
itself pinned to things other than itself: hand-derived worked examples
(tests/golden/hand_examples.json), brute force with exactly rounded sums on
tiny inputs, PyTorch's float64 scaled_dot_product_attention on the CPU, closed
forms, invariants and the online / split-KV identities.

Every pin is a function of the oracle *module*, so that the planted-mistake
test at the end can run the same pins against copies of the oracle source with
one plausible mistake edited in, and show that each mistake is caught.
"""

import json
import math
import os
import types

import numpy as np
import pytest

import oracle
import oracle.attention as oracle_attention

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "hand_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rand(seed, B, Hq, Hkv, Nq, Nk, d, scale_in=1.0):
    r = _rng(seed)
    return (r.standard_normal((B, Hq, Nq, d)) * scale_in,
            r.standard_normal((B, Hkv, Nk, d)) * scale_in,
            r.standard_normal((B, Hkv, Nk, d)))


# ---------------------------------------------------------------------------
# Pins.  Each takes the oracle module and raises AssertionError on mismatch.
# ---------------------------------------------------------------------------

def pin_golden(mod):
    """Hand-derived worked examples (exact rationals and logs of integers)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        if "bounds" in c:
            o, lse = mod.merge_ref(np.array(c["q"]), np.array(c["k"]),
                                   np.array(c["v"]), c["scale"],
                                   [tuple(x) for x in c["bounds"]])
            _close(o, c["o"], 1e-13, c["name"] + " O")
            _close(lse, c["lse"], 1e-13, c["name"] + " LSE")
            o2, l2 = mod.merge_partials(np.array(c["o_parts"]),
                                        np.array(c["lse_parts"]))
            _close(o2, c["o"], 1e-13, c["name"] + " merge O")
            _close(l2, c["lse"], 1e-13, c["name"] + " merge LSE")
            continue
        o, lse = mod.attention_ref(np.array(c["q"]), np.array(c["k"]),
                                   np.array(c["v"]), c["scale"], c["causal"])
        _close(o, c["o"], 1e-13, c["name"] + " O")
        _close(lse, c["lse"], 1e-13, c["name"] + " LSE")


def _brute(q, k, v, scale, causal):
    """Scalar loops with exactly rounded sums (math.fsum)."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = np.zeros((B, Hq, Nq, v.shape[-1]))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk)
                        if (not causal) or j <= i + (Nk - Nq)]
                sc = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, g, j, c])
                                        for c in range(d)) for j in keys]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                den = math.fsum(ex)
                for c in range(v.shape[-1]):
                    o[b, h, i, c] = math.fsum(e * float(v[b, g, j, c])
                                              for e, j in zip(ex, keys)) / den
                lse[b, h, i] = mx + math.log(den)
    return o, lse


def pin_bruteforce(mod):
    cases = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
        (1, 1, 1, 5, 5, 3, False), (1, 1, 1, 6, 6, 4, True),
        (2, 4, 2, 3, 7, 2, True), (1, 2, 1, 8, 5, 4, False),
        (1, 3, 3, 1, 8, 4, False), (1, 2, 2, 4, 4, 1, True),
    ]
    for n, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate(cases):
        q, k, v = _rand(100 + n, B, Hq, Hkv, Nq, Nk, d)
        scale = 0.3 + 0.2 * n
        o, lse = mod.attention_ref(q, k, v, scale, causal)
        ob, lb = _brute(q, k, v, scale, causal)
        _close(o, ob, 1e-12, f"brute O case {n}")
        _close(lse, lb, 1e-12, f"brute LSE case {n}")


def pin_torch_sdpa(mod):
    """PyTorch float64 SDPA on the CPU, K/V heads repeated for GQA.

    O: direct comparison.  LSE: append one extra key with score 0 (a zero key
    vector) whose value is a unit vector in an extra column; SDPA's output in
    that column is 1 / (exp(LSE) + 1), so LSE = ln(1/o_x - 1).
    """
    import torch
    F = torch.nn.functional
    for n, (B, Hq, Hkv, N, Nk, d, causal) in enumerate(
            [(2, 4, 2, 16, 16, 8, True), (1, 6, 3, 9, 23, 16, False),
             (2, 2, 2, 33, 33, 5, False), (1, 8, 1, 12, 12, 4, True)]):
        q, k, v = _rand(200 + n, B, Hq, Hkv, N, Nk, d, 0.5)
        scale = 1.0 / math.sqrt(d)
        o, lse = mod.attention_ref(q, k, v, scale, causal)
        G = Hq // Hkv
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(k).repeat_interleave(G, dim=1)
        tv = torch.from_numpy(v).repeat_interleave(G, dim=1)
        ot = F.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                            is_causal=causal)
        _close(o, ot.numpy(), 1e-12, f"sdpa O case {n}")
        if causal:
            continue
        kx = torch.cat([tk, torch.zeros(B, Hq, 1, d, dtype=torch.float64)], 2)
        vx = torch.zeros(B, Hq, Nk + 1, d + 1, dtype=torch.float64)
        vx[:, :, :Nk, :d] = tv
        vx[:, :, Nk, d] = 1.0
        ox = F.scaled_dot_product_attention(tq, kx, vx, scale=scale)
        lse_t = torch.log(1.0 / ox[..., d] - 1.0).numpy()
        _close(lse, lse_t, 1e-10, f"sdpa LSE case {n}")


def pin_identical_keys(mod):
    """All keys equal: O_i = mean of allowed V rows, LSE_i = s_i + ln|A_i|."""
    for causal, (Nq, Nk) in [(False, (7, 11)), (True, (5, 9)), (True, (6, 6))]:
        r = _rng(3)
        d = 6
        q = r.standard_normal((1, 2, Nq, d))
        kv = r.standard_normal(d)
        k = np.broadcast_to(kv, (1, 2, Nk, d)).copy()
        v = r.standard_normal((1, 2, Nk, d))
        scale = 0.7
        o, lse = mod.attention_ref(q, k, v, scale, causal)
        for h in range(2):
            for i in range(Nq):
                n_allowed = (i + (Nk - Nq) + 1) if causal else Nk
                _close(o[0, h, i], v[0, h, :n_allowed].mean(axis=0), 1e-13,
                       "identical keys O")
                _close(lse[0, h, i],
                       scale * float(q[0, h, i] @ kv) + math.log(n_allowed),
                       1e-12, "identical keys LSE")


def pin_single_key(mod):
    q, k, v = _rand(4, 2, 3, 3, 5, 1, 8)
    o, lse = mod.attention_ref(q, k, v, 0.4, causal=False)
    _close(o, np.broadcast_to(v, o.shape), 1e-14, "single key O")
    _close(lse, 0.4 * np.einsum("bhnd,bhd->bhn", q, k[:, :, 0]), 1e-13,
           "single key LSE")


def pin_causal_row0(mod):
    q, k, v = _rand(5, 1, 2, 2, 9, 9, 4)
    o, lse = mod.attention_ref(q, k, v, 0.5, causal=True)
    _close(o[:, :, 0], v[:, :, 0], 1e-14, "causal row 0 O")
    _close(lse[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
           1e-13, "causal row 0 LSE")


def pin_zero_queries(mod):
    for causal in (False, True):
        _, k, v = _rand(6, 1, 2, 2, 6, 6, 4)
        q = np.zeros((1, 2, 6, 4))
        o, lse = mod.attention_ref(q, k, v, 1.3, causal)
        for i in range(6):
            n = i + 1 if causal else 6
            _close(o[0, :, i], v[0, :, :n].mean(axis=1), 1e-14, "Q=0 O")
            _close(lse[0, :, i], np.full(2, math.log(n)), 1e-14, "Q=0 LSE")


def pin_constant_values(mod):
    q, k, _ = _rand(7, 1, 2, 1, 5, 8, 3)
    u = np.array([1.5, -2.0, 0.25])
    v = np.broadcast_to(u, (1, 1, 8, 3)).copy()
    for causal in (False, True):
        o, _ = mod.attention_ref(q, k, v, 0.9, causal)
        _close(o, np.broadcast_to(u, o.shape), 1e-14, "constant V")


def pin_rows_sum_to_one(mod):
    r = _rng(8)
    qh, kg, vg = (r.standard_normal((12, 5)), r.standard_normal((15, 5)),
                  r.standard_normal((15, 5)))
    o, lse, p = mod.attention_head_ref(qh, kg, vg, 0.6, causal=True,
                                       return_p=True)
    assert np.all(p >= 0)
    _close(p.sum(axis=1), np.ones(12), 1e-15, "rows of P sum to 1")
    mask = np.arange(15)[None, :] <= (np.arange(12)[:, None] + 3)
    assert np.all(p[~mask] == 0.0), "masked probabilities must be exactly 0"
    _close(o, p @ vg, 1e-14, "O = P V")


def pin_shift_invariance(mod):
    q, k, v = _rand(9, 1, 2, 2, 6, 10, 4)
    u = _rng(10).standard_normal(4)
    scale = 0.8
    o1, l1 = mod.attention_ref(q, k, v, scale, causal=False)
    o2, l2 = mod.attention_ref(q, k + u, v, scale, causal=False)
    _close(o2, o1, 1e-12, "shift O")
    _close(l2, l1 + scale * np.einsum("bhnd,d->bhn", q, u), 1e-12, "shift LSE")
    # Large logits: finite, and close to selecting the best key.
    o3, l3 = mod.attention_ref(q * 100, k, v, scale, causal=False)
    assert np.all(np.isfinite(o3)) and np.all(np.isfinite(l3))
    s = np.einsum("bhnd,bhkd->bhnk", q, k)
    best = s.argmax(axis=-1)
    sel = np.take_along_axis(v[:, :, None], best[..., None, None], axis=3)[..., 0, :]
    gap = np.sort(s, axis=-1)
    if np.min(gap[..., -1] - gap[..., -2]) * 100 * scale > 40:
        _close(o3, sel, 1e-10, "one-hot limit")


def pin_permutation(mod):
    q, k, v = _rand(11, 1, 2, 2, 7, 9, 4)
    o, l = mod.attention_ref(q, k, v, 0.5, causal=False)
    pk = _rng(12).permutation(9)
    pq = _rng(13).permutation(7)
    o2, l2 = mod.attention_ref(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.5,
                               causal=False)
    _close(o2, o[:, :, pq], 1e-13, "permutation O")
    _close(l2, l[:, :, pq], 1e-13, "permutation LSE")


def pin_linearity(mod):
    q, k, v1 = _rand(14, 1, 2, 1, 6, 6, 4)
    v2 = _rng(15).standard_normal(v1.shape)
    for causal in (False, True):
        o1, _ = mod.attention_ref(q, k, v1, 0.5, causal)
        o2, _ = mod.attention_ref(q, k, v2, 0.5, causal)
        o3, _ = mod.attention_ref(q, k, 2.0 * v1 - 3.0 * v2, 0.5, causal)
        _close(o3, 2.0 * o1 - 3.0 * o2, 1e-12, "linearity in V")


def pin_causal_prefix(mod):
    q, k, v = _rand(16, 1, 2, 2, 12, 12, 4)
    o, l = mod.attention_ref(q, k, v, 0.5, causal=True)
    for n in (1, 5, 12):
        on, ln_ = mod.attention_ref(q[:, :, :n], k[:, :, :n], v[:, :, :n], 0.5,
                                    causal=True)
        _close(on, o[:, :, :n], 1e-13, "causal prefix O")
        _close(ln_, l[:, :, :n], 1e-13, "causal prefix LSE")


def pin_online_matches(mod):
    for causal, (Nq, Nk) in [(False, (9, 40)), (True, (40, 40)),
                             (True, (13, 70))]:
        r = _rng(17)
        qh, kg, vg = (r.standard_normal((Nq, 8)), r.standard_normal((Nk, 8)),
                      r.standard_normal((Nk, 8)))
        o, l = mod.attention_head_ref(qh, kg, vg, 0.4, causal)
        for tile in (1, 7, 64, Nk):
            o2, l2 = mod.online_ref(qh, kg, vg, 0.4, causal, tile)
            _close(o2, o, 1e-12, f"online O tile {tile}")
            _close(l2, l, 1e-12, f"online LSE tile {tile}")


def pin_merge_matches(mod):
    r = _rng(18)
    B, Hq, Hkv, Nk, d = 2, 4, 2, 50, 8
    q = r.standard_normal((B, Hq, d))
    k = r.standard_normal((B, Hkv, Nk, d))
    v = r.standard_normal((B, Hkv, Nk, d))
    o, l = mod.attention_ref(q[:, :, None], k, v, 0.35, causal=False)
    o, l = o[:, :, 0], l[:, :, 0]
    parts = []
    for S in (1, 2, 16, 64):
        c = -(-Nk // S)
        parts.append([(s * c, min((s + 1) * c, Nk)) for s in range(S)])
    cuts = np.sort(r.choice(np.arange(1, Nk), 6, replace=False))
    edges = [0, 0] + list(cuts) + [cuts[-1], Nk, Nk]   # with empty chunks
    parts.append(list(zip(edges[:-1], edges[1:])))
    for bounds in parts:
        o2, l2 = mod.merge_ref(q, k, v, 0.35, bounds)
        _close(o2, o, 1e-12, f"merge O S={len(bounds)}")
        _close(l2, l, 1e-12, f"merge LSE S={len(bounds)}")


PINS = [pin_golden, pin_bruteforce, pin_torch_sdpa, pin_identical_keys,
        pin_single_key, pin_causal_row0, pin_zero_queries, pin_constant_values,
        pin_rows_sum_to_one, pin_shift_invariance, pin_permutation,
        pin_linearity, pin_causal_prefix, pin_online_matches,
        pin_merge_matches]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


# ---------------------------------------------------------------------------
# Planted mistakes: each edits one line of a copy of the oracle source and
# must make at least one pin fail.  Nothing here touches the real oracle.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "dropped_scale": ("s = scale * (qh[rb] @ kg.T)", "s = (qh[rb] @ kg.T)"),
    "scores_use_values": ("s = scale * (qh[rb] @ kg.T)",
                          "s = scale * (qh[rb] @ vg.T)"),
    "mask_top_left": ("return j <= (rows[:, None] + (Nk - Nq))",
                      "return j <= rows[:, None]"),
    "mask_strict": ("return j <= (rows[:, None] + (Nk - Nq))",
                    "return j < (rows[:, None] + (Nk - Nq))"),
    "gqa_modulo": ("return h // (Hq // Hkv)", "return h % Hkv"),
    "exp_sign": ("e = np.exp(s - m)", "e = np.exp(m - s)"),
    "exp_base2": ("e = np.exp(s - m)", "e = np.exp2(s - m)"),
    "max_is_min": ("m = s.max(axis=1, keepdims=True)",
                   "m = s.min(axis=1, keepdims=True)"),
    "unnormalised": ("p = e / l", "p = e"),
    "output_uses_keys": ("o[r0:r0 + step] = p @ vg", "o[r0:r0 + step] = p @ kg"),
    "lse_drops_max": ("lse[r0:r0 + step] = (m + np.log(l))[:, 0]",
                      "lse[r0:r0 + step] = (np.log(l))[:, 0]"),
    "lse_log2": ("lse[r0:r0 + step] = (m + np.log(l))[:, 0]",
                 "lse[r0:r0 + step] = (m + np.log2(l))[:, 0]"),
    "online_no_acc_rescale": ("acc = alpha * acc + e @ vt", "acc = acc + e @ vt"),
    "online_no_sum_rescale": ("l = alpha * l + e.sum(axis=1, keepdims=True)",
                              "l = l + e.sum(axis=1, keepdims=True)"),
    "merge_unnormalised_weights": (
        "w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - M), 0.0)",
        "w = np.where(np.isfinite(lse_parts), np.exp(lse_parts), 0.0)"),
    "merge_no_division": (
        "o = (w[..., None] * np.nan_to_num(o_parts)).sum(axis=0) / wsum[..., None]",
        "o = (w[..., None] * np.nan_to_num(o_parts)).sum(axis=0)"),
}


def _mutant(old, new):
    with open(oracle_attention.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
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
