"""Plain float64 CPU oracle for exact attention and split-KV decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP library and is deliberately slow and literal:
it materialises the full score matrix S and probability matrix P, which the
fused kernels never do.

Pages cited (short names used below):
  [Evolution]  "FlashAttention evolution" (sandeep007734.github.io,
               posts/flashattention-evolution)
  [Kruglikov]  "Flash Attention" (vladislavkruglikov.com, articles/flash-attention)

What is computed, per batch b, query head h, query row i, key j:
  * [Evolution] §1 (the equation under "The Invariant and the Moving
    Bottleneck") defines the function as O = softmax(Q K^T) V; [Kruglikov]'s
    introduction calls it scaled dot-product attention with scores S and
    probabilities P.  The scale factor itself did not survive on the pages, so
    it is a caller argument; every workload passes 1/sqrt(d).
  * Causal masking is not defined on the pages.  Reading adopted: key j is
    allowed for row i iff j <= i + (Nk - Nq) (bottom-right aligned; the usual
    j <= i when Nq == Nk).  Masked keys get probability exactly 0.
  * Grouped-query attention (not on the pages): query head h reads key/value
    head h // (Hq // Hkv).
  * The per-row metadata written next to O ([Kruglikov], "The IO problem") is
    read as the natural-log log-sum-exp of the scaled, allowed scores.

The online recurrence ([Evolution] §2, §3, §5) and the split-KV merge
([Evolution] §6) are modelled separately in ``online_ref`` and
``merge_partials`` so that the tests can pin the identities the method relies
on; the reference result itself is always the two-pass definition.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "allowed_keys",
    "attention_ref",
    "attention_head_ref",
    "online_ref",
    "merge_partials",
    "merge_ref",
]

# Rows per block when materialising S, to keep each block near 64 MB.
_ROW_BLOCK_BYTES = 64 << 20


def allowed_keys(rows, Nq: int, Nk: int, causal: bool) -> np.ndarray:
    """Boolean [R][Nk]: key j allowed for query row i (reading of causal mask)."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Nk, dtype=np.int64)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Nk), dtype=bool)
    return j <= (rows[:, None] + (Nk - Nq))


def attention_head_ref(qh, kg, vg, scale, causal=False, rows=None,
                       return_p=False):
    """Exact attention for one (batch, head) pair, in float64.

    qh: [Nq][d] query rows; kg, vg: [Nk][d] keys and values of the KV head the
    query head reads.  ``rows`` selects a subset of query rows (indices into
    0..Nq-1); the mask still uses the full Nq.  Returns (O [R][d], LSE [R]) and
    optionally P [R][Nk].

    Steps, in the order of the definition:
      1. S = scale * Q K^T
      2. masked entries -> -inf
      3. m = row max of S
      4. E = exp(S - m)       (exp(-inf) = 0)
      5. l = row sum of E
      6. P = E / l
      7. O = P V,  LSE = m + ln l
    """
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    vg = np.asarray(vg, dtype=np.float64)
    Nq, d = qh.shape
    Nk = kg.shape[0]
    if rows is None:
        rows = np.arange(Nq, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    o = np.empty((R, vg.shape[1]), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    p_all = np.empty((R, Nk), dtype=np.float64) if return_p else None
    step = max(1, _ROW_BLOCK_BYTES // max(1, 8 * Nk))
    for r0 in range(0, R, step):
        rb = rows[r0:r0 + step]
        s = scale * (qh[rb] @ kg.T)                               # 1
        allowed = allowed_keys(rb, Nq, Nk, causal)
        s = np.where(allowed, s, -np.inf)                         # 2
        m = s.max(axis=1, keepdims=True)                          # 3
        e = np.exp(s - m)                                         # 4
        l = e.sum(axis=1, keepdims=True)                          # 5
        p = e / l                                                 # 6
        o[r0:r0 + step] = p @ vg                                  # 7
        lse[r0:r0 + step] = (m + np.log(l))[:, 0]
        if return_p:
            p_all[r0:r0 + step] = p
    if return_p:
        return o, lse, p_all
    return o, lse


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    """GQA reading: contiguous groups of Hq // Hkv query heads share a KV head."""
    return h // (Hq // Hkv)


def attention_ref(q, k, v, scale, causal=False, rows=None):
    """Exact attention over a batch, float64.

    q: [B][Hq][Nq][d]; k, v: [B][Hkv][Nk][d].  ``rows`` is None (all rows) or
    an index array applied to every (b, h), or a dict {h: rows} for per-head
    subsets.  Returns O [B][Hq][R][d] and LSE [B][Hq][R].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    outs_o, outs_l = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            r = rows.get(h) if isinstance(rows, dict) else rows
            o_h, l_h = attention_head_ref(q[b, h], k[b, g], v[b, g], scale,
                                          causal, r)
            ob.append(o_h)
            lb.append(l_h)
        outs_o.append(np.stack(ob))
        outs_l.append(np.stack(lb))
    return np.stack(outs_o), np.stack(outs_l)


def online_ref(qh, kg, vg, scale, causal=False, tile=64):
    """The tiled online-softmax recurrence for one (batch, head), float64.

    Follows the state the pages describe: a running maximum, a running
    normalisation sum and an unnormalised output accumulator, updated once per
    key/value tile ([Evolution] §2 and §3; the cheaper path when the maximum
    does not move is the same update with a rescale factor of one, §5), with
    the division by the sum deferred to the end ([Evolution] §3).

      m = -inf, l = 0, acc = 0
      for each key tile T:
          m_new = max(m, max over T of s)
          acc   = exp(m - m_new) * acc + sum over T of exp(s - m_new) * v
          l     = exp(m - m_new) * l   + sum over T of exp(s - m_new)
          m     = m_new
      O = acc / l,  LSE = m + ln l
    """
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    vg = np.asarray(vg, dtype=np.float64)
    Nq, _ = qh.shape
    Nk = kg.shape[0]
    rows = np.arange(Nq)
    m = np.full((Nq, 1), -np.inf)
    l = np.zeros((Nq, 1))
    acc = np.zeros((Nq, vg.shape[1]))
    for j0 in range(0, Nk, tile):
        kt, vt = kg[j0:j0 + tile], vg[j0:j0 + tile]
        s = scale * (qh @ kt.T)
        allowed = allowed_keys(rows, Nq, Nk, causal)[:, j0:j0 + tile]
        s = np.where(allowed, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1, keepdims=True))
        # A row with no allowed key yet keeps m = -inf; its factors are 0.
        safe = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - safe), 0.0)
        e = np.exp(s - safe)
        acc = alpha * acc + e @ vt
        l = alpha * l + e.sum(axis=1, keepdims=True)
        m = m_new
    return acc / l, (m + np.log(l))[:, 0]


def merge_partials(o_parts, lse_parts):
    """Merge per-chunk normalised partial outputs with the softmax identity.

    o_parts: [S][..., d] partial outputs, each normalised over its own chunk;
    lse_parts: [S][...] the chunk log-sum-exps (-inf for an empty chunk).
    [Evolution] §6: the partial maxima, sums and weighted outputs of the KV
    partitions are combined with the same identity the online softmax uses:
      M = max_s LSE_s,  w_s = exp(LSE_s - M),
      O = sum_s w_s O_s / sum_s w_s,  LSE = M + ln sum_s w_s.
    Chunks with LSE = -inf get weight 0.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - M), 0.0)
    wsum = w.sum(axis=0)
    o = (w[..., None] * np.nan_to_num(o_parts)).sum(axis=0) / wsum[..., None]
    return o, M + np.log(wsum)


def merge_ref(q, k, v, scale, bounds):
    """Split-KV decode: attention per key chunk, then ``merge_partials``.

    q: [B][Hq][d] (one query row per sequence); k, v: [B][Hkv][Nk][d].
    ``bounds`` is a list of (start, end) key ranges covering 0..Nk-1 (empty
    ranges allowed).  Returns O [B][Hq][d], LSE [B][Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    S = len(bounds)
    o_parts = np.zeros((S, B, Hq, v.shape[-1]))
    lse_parts = np.full((S, B, Hq), -np.inf)
    for s, (a, e) in enumerate(bounds):
        if e <= a:
            continue
        o_s, l_s = attention_ref(q[:, :, None, :], k[:, :, a:e], v[:, :, a:e],
                                 scale, causal=False)
        o_parts[s] = o_s[:, :, 0]
        lse_parts[s] = l_s[:, :, 0]
    return merge_partials(o_parts, lse_parts)
