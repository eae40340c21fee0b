"""Helpers for the GPU parity tests: device marshalling and the parity bar.

The bar (float inputs rounded to bf16, compared against the float64 oracle):
  O   max-abs error <= 1.5e-2 and mean-abs error <= 2e-3
  LSE max-abs error <= 1e-3
Next to the primary error the report prints the error against the oracle
rounded to bf16 (the output format's own rounding) and the count of outputs
with |O| >= 4, where one bf16 half-ulp (2^-6) already exceeds 1.5e-2.
"""

from __future__ import annotations

import sys

import numpy as np

from datagen import bf16_bits_from_f32, f64_from_bf16_bits

O_MAX_ABS = 1.5e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> contiguous torch.bfloat16 tensor on cuda:0."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0").contiguous()


def host_f64(t):
    """Device tensor (bf16 or fp32) -> float64 numpy array (exact widening)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def report(tag, o, lse, o_ref, lse_ref):
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o - o_ref)
    e_max = float(err.max()) if err.size else 0.0
    e_mean = float(err.mean()) if err.size else 0.0
    e_lse = float(np.abs(np.asarray(lse, dtype=np.float64) - lse_ref).max()) if np.size(lse) else 0.0
    o_ref_bf = f64_from_bf16_bits(bf16_bits_from_f32(o_ref.astype(np.float32)))
    e_bf = float(np.abs(o - o_ref_bf).max()) if err.size else 0.0
    big = int((np.abs(o_ref) >= 4).sum())
    finite = bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse)))
    print(f"[parity] {tag}: O max {e_max:.3e} mean {e_mean:.3e} | vs bf16(oracle) "
          f"max {e_bf:.3e} | LSE max {e_lse:.3e} | |O_ref|>=4: {big} | finite {finite}",
          flush=True)
    return dict(o_max=e_max, o_mean=e_mean, lse_max=e_lse, o_max_bf16=e_bf, big=big,
                finite=finite)


def assert_parity(tag, o, lse, o_ref, lse_ref):
    r = report(tag, o, lse, o_ref, lse_ref)
    assert r["finite"], f"{tag}: non-finite output"
    assert r["o_max"] <= O_MAX_ABS, f"{tag}: O max-abs {r['o_max']:.3e}"
    assert r["o_mean"] <= O_MEAN_ABS, f"{tag}: O mean-abs {r['o_mean']:.3e}"
    assert r["lse_max"] <= LSE_MAX_ABS, f"{tag}: LSE max-abs {r['lse_max']:.3e}"
    return r


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


# Gradients.  Each element of dQ, dK, dV is a sum over keys or query rows of
# products whose bf16 operands (P, dS) carry independent rounding of relative
# size <= 2^-8 (mean square (2^-8)^2 / 3 for uniformly spread roundings), plus
# the bf16 rounding of the result and of the forward output O that Delta =
# rowsum(dO * O) is computed from.  Those roundings give a relative Frobenius
# error of about 2^-8 / sqrt(3) ~ 2e-3; the norm bars below allow about 5x
# that, and the element bound (grad_error_bounds) checks every element:
GRAD_REL_FRO = 1e-2      # ||G - G_ref||_F / ||G_ref||_F
GRAD_MAX_REL = 3e-2      # max |G - G_ref| / max |G_ref|


def report_grad(tag, name, g, g_ref):
    g = np.asarray(g, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    diff = g - g_ref
    ref_fro = float(np.sqrt((g_ref ** 2).sum()))
    ref_max = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    rel_fro = float(np.sqrt((diff ** 2).sum())) / ref_fro if ref_fro > 0 else float(np.abs(diff).max())
    max_rel = float(np.abs(diff).max()) / ref_max if ref_max > 0 else float(np.abs(diff).max())
    finite = bool(np.all(np.isfinite(g)))
    print(f"[parity] {tag} d{name}: rel-Frobenius {rel_fro:.3e} | max/max|ref| {max_rel:.3e} "
          f"| max|ref| {ref_max:.3e} | finite {finite}", flush=True)
    return dict(rel_fro=rel_fro, max_rel=max_rel, finite=finite)


def assert_grad_parity(tag, grads, refs, bounds=None):
    """grads, refs: dicts name -> array (dQ, dK, dV).  With ``bounds`` (same
    keys, from grad_error_bounds) every element must also satisfy
    |G - G_ref| <= bound."""
    out = {}
    for name in refs:
        r = report_grad(tag, name, grads[name], refs[name])
        assert r["finite"], f"{tag} d{name}: non-finite"
        assert r["rel_fro"] <= GRAD_REL_FRO, f"{tag} d{name}: rel-Frobenius {r['rel_fro']:.3e}"
        assert r["max_rel"] <= GRAD_MAX_REL, f"{tag} d{name}: max rel {r['max_rel']:.3e}"
        if bounds is not None:
            err = np.abs(np.asarray(grads[name], np.float64) - np.asarray(refs[name], np.float64))
            bnd = np.asarray(bounds[name], np.float64)
            ratio = err / np.maximum(bnd, 1e-300)
            worst = float(ratio.max()) if ratio.size else 0.0
            print(f"[parity] {tag} d{name}: element bound: max |err|/bound {worst:.3f} "
                  f"(median bound {float(np.median(bnd)) if bnd.size else 0.0:.3e})", flush=True)
            r["bound_ratio"] = worst
            bad = np.argwhere(err > bnd)
            assert bad.size == 0, (f"{tag} d{name}: {len(bad)} elements exceed the element bound, "
                                   f"first at {tuple(bad[0])}: err {err[tuple(bad[0])]:.3e} > "
                                   f"{bnd[tuple(bad[0])]:.3e}")
        out[name] = r
    return out


# Element-wise gradient bound.  For one element of dQ, dK or dV the kernels'
# error is bounded by the roundings they make, each at most U_BF16 (bf16, 8
# significant bits) or U_F32 relative, taken with absolute values (every
# rounding aligned).  With P the exact probabilities, dP = dO V^T, Delta_i =
# rowsum(P * dP)_i, dS = P (dP - Delta):
#   p_err_ij  relative error of the kernel's fp32 P: its LSE input's error
#             |LSE_given - LSE|_i, the fp32 score sum (2 d U_F32 scale |q_i|.|k_j|),
#             the exponent's rounding (|s_ij| + |LSE_i|) U_F32 and the exp2
#             instruction (4 U_F32)
#   dd_i      error of the kernel's Delta = rowsum(dO * O_given) in fp32:
#             |rowsum(dO * (O_given - O))| + 2 d U_F32 rowsum(|dO| |O_given|)
#   ds_err_ij error of dS before its bf16 rounding: P (p_err |dP - Delta| + dd
#             + 2 d U_F32 |dO_i|.|v_j|)
#   dV_j      sum_i [(U_BF16 + 2 n U_F32 + p_err_ij) P_ij |dO_i|]    (P -> bf16)
#   dQ_i      scale sum_j [(U_BF16 |dS_ij| + ds_err_ij)(1 + 2 n U_F32) |k_j|]
#   dK_j      scale sum_i [(U_BF16 |dS_ij| + ds_err_ij)(1 + 2 n U_F32) |q_i|]
# (n = the number of products an fp32 accumulator sums; each fp32 sum term is
# taken as 2 n U_F32 Sum|terms|, one ulp per addition, since the MFMA's internal
# rounding is not specified), and the bf16 rounding of the output adds
# U_BF16 (|G_ref| + bound).  The sums run over the query heads that share a
# KV head for dK and dV.
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24
_BOUND_BLOCK_BYTES = 32 << 20


def _head_bound_terms(qh, kg, vg, doh, oh_given, lse_given, scale, causal, rows, keys, n_rows):
    """Bound terms of one (query head, KV head) pair: dQ terms for ``rows``,
    and this head's dK, dV terms for ``keys`` (summed over every row)."""
    from oracle.attention import allowed_keys
    Nq, d = qh.shape
    Nk = kg.shape[0]
    aq, ak, av, ado = np.abs(qh), np.abs(kg), np.abs(vg), np.abs(doh)
    gd = 2 * d * U_F32       # fp32 accumulation over d (S, dP, Delta)
    gk = 2 * Nk * U_F32      # fp32 accumulation over keys (dQ)
    gq = 2 * n_rows * U_F32  # fp32 accumulation over rows (dK, dV)
    step = max(1, _BOUND_BLOCK_BYTES // max(1, 8 * Nk))
    rsel = set(int(r) for r in rows)
    bq = {}
    bk = np.zeros((len(keys), d))
    bv = np.zeros((len(keys), vg.shape[1]))
    for r0 in range(0, Nq, step):
        rb = np.arange(r0, min(Nq, r0 + step), dtype=np.int64)
        s = scale * (qh[rb] @ kg.T)
        allowed = allowed_keys(rb, Nq, Nk, causal)
        s = np.where(allowed, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        p = np.exp(s - lse[:, None])
        o_ex = p @ vg
        dp = doh[rb] @ vg.T
        delta = (p * dp).sum(axis=1)
        ds = p * (dp - delta[:, None])
        s_abs = np.where(allowed, np.abs(s), 0.0)
        p_err = (np.abs(lse_given[rb] - lse)[:, None] + gd * scale * (aq[rb] @ ak.T)
                 + (s_abs + np.abs(lse)[:, None]) * U_F32 + 4 * U_F32)
        dd = (np.abs((doh[rb] * (oh_given[rb] - o_ex)).sum(axis=1))
              + gd * (ado[rb] * np.abs(oh_given[rb])).sum(axis=1))
        ds_err = p * (p_err * np.abs(dp - delta[:, None]) + dd[:, None]
                      + gd * (ado[rb] @ av.T))
        e = (U_BF16 * np.abs(ds) + ds_err)
        sel = [i for i, r in enumerate(rb) if int(r) in rsel]
        if sel:
            t = scale * (1 + gk) * (e[sel] @ ak)
            for i, ti in zip(sel, t):
                bq[int(rb[i])] = ti
        bk += scale * (1 + gq) * (e[:, keys].T @ aq[rb])
        bv += (((U_BF16 + gq) + p_err) * p)[:, keys].T @ ado[rb]
    bq = np.stack([bq[int(r)] for r in rows]) if len(rows) else np.zeros((0, d))
    return bq, bk, bv


def head_grad_error_bounds(qh, kg, vg, doh, oh_given, lseh_given, scale, causal, refs,
                           rows=None, keys=None):
    """grad_error_bounds for one query head whose KV head has no other query
    head (refs: dQ rows ``rows``, dK/dV keys ``keys`` of that pair)."""
    Nq = qh.shape[0]
    Nk = kg.shape[0]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    keys = np.arange(Nk) if keys is None else np.asarray(keys, np.int64)
    tq, tk, tv = _head_bound_terms(qh, kg, vg, doh, oh_given, lseh_given, scale, causal, rows,
                                   keys, Nq)
    return {name: (1 + U_BF16) * t + U_BF16 * np.abs(np.asarray(refs[name], np.float64))
            for name, t in (("Q", tq), ("K", tk), ("V", tv))}


def grad_error_bounds(q, k, v, do, o_given, lse_given, scale, causal, refs,
                      rows=None, keys=None):
    """Element bounds on |G - G_ref| for the kernels' dQ, dK, dV.

    q, do, o_given: [B][Hq][Nq][d]; k, v: [B][Hkv][Nk][d] (float64 values of
    the bf16 inputs; o_given and lse_given [B][Hq][Nq] are what the backward
    was fed); refs: dict Q, K, V of oracle gradients with the same row/key
    selection.  ``rows``/``keys`` (index arrays) select the dQ rows and the dK,
    dV keys compared, for every (b, head)."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    keys = np.arange(Nk) if keys is None else np.asarray(keys, np.int64)
    bQ = np.zeros((B, Hq, len(rows), d))
    bK = np.zeros((B, Hkv, len(keys), d))
    bV = np.zeros((B, Hkv, len(keys), v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            tq, tk, tv = _head_bound_terms(q[b, h], k[b, g], v[b, g], do[b, h], o_given[b, h],
                                           lse_given[b, h], scale, causal, rows, keys,
                                           Nq * grp)
            bQ[b, h] = tq
            bK[b, g] += tk
            bV[b, g] += tv
    out = {}
    for name, t in (("Q", bQ), ("K", bK), ("V", bV)):
        ref = np.abs(np.asarray(refs[name], np.float64)).reshape(t.shape)
        out[name] = ((1 + U_BF16) * t + U_BF16 * ref).reshape(np.shape(refs[name]))
    return out
