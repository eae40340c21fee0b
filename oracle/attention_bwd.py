"""Plain float64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP library and is deliberately slow and literal:
it materialises the score, probability and score-gradient matrices of each
block of query rows, which the fused kernels never do.

Pages cited (short names used below):
  [Comparison] "FlashAttention 1-4 generation comparison" (phantomic12.github.io,
               inference-research)
  [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
               posts/flashattention-evolution)

What is computed.  The pages state that the backward pass recomputes the
scores from the inputs instead of storing them ([Comparison] "Notes", the
FlashAttention-1 entry) and discuss the backward's speed and operand layouts
([Evolution] §4, §5), but print no gradient formulas.  The gradients are
therefore those of the forward function of ``oracle/attention.py`` (scaled,
optionally causal, grouped-query softmax attention) for a loss L whose
gradient with respect to the output O is the given dO.  By the chain rule,
per (batch b, query head h reading key/value head g):

  S  = scale * Q K^T,  masked entries excluded,  P = softmax over each row
  dV = P^T dO                                   (O = P V)
  dP = dO V^T
  dS = P * (dP - rowsum(P * dP))                (Jacobian of a row softmax)
  dQ = scale * dS K
  dK = scale * dS^T Q

A masked entry has P = 0 and therefore dS = 0.  A key/value head's gradients
are the sums over every query head that reads it.  ``tests/test_oracle_bwd.py``
pins these against PyTorch autograd (float64), central finite differences of
the forward oracle, closed forms and invariants.
"""

from __future__ import annotations

import numpy as np

from oracle.attention import allowed_keys

__all__ = ["attention_bwd_head_ref", "attention_bwd_ref"]

# Rows per block when materialising S, P, dP and dS (about 64 MB each).
_ROW_BLOCK_BYTES = 64 << 20


def _block_grads(qb, rb, kg, vg, dob, scale, causal, Nq):
    """P and dS for a block of query rows ``rb`` against all keys."""
    Nk = kg.shape[0]
    s = scale * (qb @ kg.T)                                   # scores
    s = np.where(allowed_keys(rb, Nq, Nk, causal), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)                      # row softmax
    dp = dob @ vg.T                                           # dP = dO V^T
    dsum = (p * dp).sum(axis=1, keepdims=True)                # rowsum(P * dP)
    ds = p * (dp - dsum)                                      # dS
    return p, ds


def attention_bwd_head_ref(qh, kg, vg, doh, scale, causal=False, rows=None,
                           keys=None, want_dq=True, want_dkv=True):
    """Gradients for one (batch, query head) pair, in float64.

    qh, doh: [Nq][d]; kg, vg: [Nk][d] (the key/value head that qh reads).
    ``rows`` selects the query rows whose dQ is returned (default all);
    ``keys`` selects the keys whose dK, dV are returned (default all).  dK and
    dV always sum over every query row.  Returns (dq [R][d] or None,
    dk [K][d] or None, dv [K][d] or None).
    """
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    vg = np.asarray(vg, dtype=np.float64)
    doh = np.asarray(doh, dtype=np.float64)
    Nq, d = qh.shape
    Nk = kg.shape[0]
    step = max(1, _ROW_BLOCK_BYTES // max(1, 8 * Nk))

    dq = None
    if want_dq:
        rsel = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
        dq = np.empty((rsel.shape[0], d), dtype=np.float64)
        for r0 in range(0, rsel.shape[0], step):
            rb = rsel[r0:r0 + step]
            _, ds = _block_grads(qh[rb], rb, kg, vg, doh[rb], scale, causal, Nq)
            dq[r0:r0 + step] = scale * (ds @ kg)             # dQ = scale dS K

    dk = dv = None
    if want_dkv:
        ksel = np.arange(Nk, dtype=np.int64) if keys is None else np.asarray(keys, np.int64)
        dk = np.zeros((ksel.shape[0], d), dtype=np.float64)
        dv = np.zeros((ksel.shape[0], vg.shape[1]), dtype=np.float64)
        for r0 in range(0, Nq, step):
            rb = np.arange(r0, min(Nq, r0 + step), dtype=np.int64)
            p, ds = _block_grads(qh[rb], rb, kg, vg, doh[rb], scale, causal, Nq)
            dv += p[:, ksel].T @ doh[rb]                     # dV = P^T dO
            dk += scale * (ds[:, ksel].T @ qh[rb])           # dK = scale dS^T Q
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, scale, causal=False):
    """Gradients over a batch, float64.

    q, do: [B][Hq][Nq][d]; k, v: [B][Hkv][Nk][d].  Returns dq [B][Hq][Nq][d]
    and dk, dv [B][Hkv][Nk][d]; query head h reads key/value head
    h // (Hq // Hkv), and each key/value head sums its query heads' gradients.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            dq_h, dk_h, dv_h = attention_bwd_head_ref(q[b, h], k[b, g], v[b, g], do[b, h],
                                                      scale, causal)
            dq[b, h] = dq_h
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv
