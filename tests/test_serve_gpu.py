"""GPU parity tests of fa_decode_serve (serving-shaped split-KV decode).

Each sequence b has its own key count n_b <= Nk (the cache capacity) and Nq
query rows; with causal masking row i sees keys j <= n_b - Nq + i.  That is
the forward oracle's bottom-right causal mask on the sequence's first n_b
keys, so every expected row comes from ``oracle.attention_head_ref`` on
q[b, h] against k/v[b, g, :n_b].  Rows with no allowed key (n_b = 0, or
causal rows before the first key) are not computed by the oracle: their
result is the reading O = 0, LSE = -inf, checked directly.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import announce, assert_parity, dev_bf16, host_f64

import exact_attention_103_amd as fa

pytestmark = pytest.mark.gpu


def _expected(qb, kb, vb, lens, scale, causal):
    """Oracle O, LSE [B][Hq][Nq][d] / [B][Hq][Nq] and the mask of rows that
    have at least one allowed key."""
    B, Hq, Nq, d = qb.shape
    Hkv = kb.shape[1]
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    live = np.zeros((B, Hq, Nq), dtype=bool)
    for b in range(B):
        n = int(lens[b])
        rows = np.arange(Nq)
        if causal:
            rows = rows[n - Nq + rows >= 0]
        elif n == 0:
            rows = rows[:0]
        if rows.size == 0:
            continue
        for h in range(Hq):
            g = h // (Hq // Hkv)
            oh, lh = oracle.attention_head_ref(
                datagen.f64_from_bf16_bits(qb[b, h]), datagen.f64_from_bf16_bits(kb[b, g, :n]),
                datagen.f64_from_bf16_bits(vb[b, g, :n]), scale, causal, rows=rows)
            o[b, h, rows] = oh
            lse[b, h, rows] = lh
            live[b, h, rows] = True
    return o, lse, live


def _run(qb, kb, vb, lens, scale, causal, num_splits=0):
    import torch
    sl = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).to("cuda:0")
    o, lse = fa.decode_serve(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), sl, causal=causal,
                             scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


def _check(tag, qb, kb, vb, lens, scale, causal, num_splits=0):
    o, lse = _run(qb, kb, vb, lens, scale, causal, num_splits)
    o_ref, lse_ref, live = _expected(qb, kb, vb, lens, scale, causal)
    assert_parity(tag, o[live], lse[live], o_ref[live], lse_ref[live])
    dead = ~live
    if dead.any():
        assert np.all(o[dead] == 0.0), f"{tag}: rows without keys must be 0"
        assert np.all(np.isneginf(lse[dead])), f"{tag}: rows without keys must have LSE -inf"


# (B, Hq, Hkv, Nq, Nk capacity, d, causal, lengths)
CASES = [
    (4, 8, 2, 1, 2048, 128, False, [2048, 1, 700, 1500]),
    (4, 8, 2, 4, 2048, 128, True, [2048, 4, 701, 1499]),
    (3, 8, 2, 3, 1000, 64, True, [999, 64, 3]),
    (2, 4, 1, 16, 777, 64, True, [777, 300]),
    (2, 16, 1, 1, 513, 256, False, [513, 17]),
    (2, 6, 3, 5, 400, 32, False, [400, 129]),
    (3, 8, 8, 2, 300, 128, True, [0, 1, 2]),   # empty cache and rows before the first key
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_Nq{c[3]}_Nk{c[4]}_d{c[5]}_{'c' if c[6] else 'nc'}" for c in CASES])
def test_serve_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal, lens = case
    tag = f"serve B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} lens={lens}"
    announce(tag)
    qb, kb, vb = datagen.gaussian_bf16(900 + Nq + d, [(B, Hq, Nq, d), (B, Hkv, Nk, d),
                                                      (B, Hkv, Nk, d)])
    _check(tag, qb, kb, vb, np.array(lens, np.int32), 1 / np.sqrt(d), causal)


@pytest.mark.parametrize("splits", [0, 1, 7, 32])
def test_serve_workload(splits):
    """The serving workload (B=8, Hq=32, Hkv=8, 4 causal rows, caches of
    1k..32k tokens in a 32k capacity), every row checked."""
    cfg = datagen.CONFIGS["serve"]
    announce(f"serve workload splits={splits}")
    qb, kb, vb, lens = datagen.make_serve_inputs(cfg)
    _check(f"serve workload S={splits}", qb, kb, vb, lens, cfg.scale, cfg.causal, splits)


@pytest.mark.parametrize("splits", [0, 3, 16])
def test_serve_skewed_lengths(splits):
    """One full-capacity sequence next to short ones (and one of a single
    key): the long sequence's chunks are many times the short ones'."""
    B, Hq, Hkv, Nq, Nk, d = 8, 8, 2, 3, 4096, 128
    tag = f"serve skewed lengths S={splits}"
    announce(tag)
    lens = np.array([4096, 64, 65, 1, 100, 3000, 64, 129], np.int32)
    qb, kb, vb = datagen.gaussian_bf16(950 + splits, [(B, Hq, Nq, d), (B, Hkv, Nk, d),
                                                      (B, Hkv, Nk, d)])
    _check(tag, qb, kb, vb, lens, 1 / np.sqrt(d), True, splits)


def test_serve_matches_plain_decode_bitwise():
    """One row per sequence and no length array is the plain split-KV decode:
    same partition, same arithmetic, identical bits."""
    import torch
    announce("serve == decode")
    cfg = datagen.CONFIGS["decode"]
    qb, kb, vb = datagen.make_decode_inputs(cfg)
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o1, l1 = fa.decode(q, k, v, num_splits=16)
    o2, l2 = fa.decode_serve(q[:, :, None, :].contiguous(), k, v, None, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2[:, :, 0].view(torch.int16))
    assert torch.equal(l1, l2[:, :, 0])


def test_serve_deterministic():
    import torch
    announce("serve determinism")
    qb, kb, vb = datagen.gaussian_bf16(31, [(2, 8, 4, 128), (2, 2, 3000, 128), (2, 2, 3000, 128)])
    sl = torch.tensor([3000, 1234], dtype=torch.int32, device="cuda")
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    a = fa.decode_serve(q, k, v, sl, causal=True)
    b = fa.decode_serve(q, k, v, sl, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
