"""GPU parity tests of fa_bwd (dQ, dK, dV) against the float64 backward oracle.

Small and ragged shapes compare every gradient element; the inputs O and LSE
of those cases come from the float64 forward oracle (rounded to bf16 / fp32),
so the backward kernels are checked on their own.  The workload shapes run
the GPU forward first and feed its O and LSE to the backward, as a training
step does, and compare sampled heads, rows and keys against the oracle
gradients of the same q, k, v, dO.  The bar (tests/parity.py) is a relative
Frobenius error <= 1e-2 and a largest error <= 3e-2 of the largest reference
magnitude, per gradient, and for every compared element an error bound
derived from the kernels' bf16 and fp32 roundings (grad_error_bounds), given
the O and LSE the backward was fed.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import (announce, assert_grad_parity, dev_bf16, grad_error_bounds,
                    head_grad_error_bounds, host_f64)

import exact_attention_103_amd as fa

pytestmark = pytest.mark.gpu


def _oracle_fwd_outputs(q64, k64, v64, scale, causal):
    o, lse = oracle.attention_ref(q64, k64, v64, scale, causal)
    return datagen.bf16_bits_from_f32(o.astype(np.float32)), lse.astype(np.float32)


def _bwd_on_gpu(qb, kb, vb, dob, ob, lse32, scale, causal):
    import torch
    q, k, v, do, o = (dev_bf16(x) for x in (qb, kb, vb, dob, ob))
    lse = torch.from_numpy(np.ascontiguousarray(lse32)).to("cuda:0")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


# (B, Hq, Hkv, Nq, Nk, d, causal): ragged lengths, GQA, Nq != Nk, tiny sizes.
ODD = [
    (1, 2, 1, 200, 200, 128, False),
    (1, 2, 1, 200, 200, 128, True),
    (1, 4, 2, 77, 300, 128, True),
    (2, 2, 2, 130, 130, 64, True),
    (1, 4, 1, 257, 190, 64, False),
    (1, 2, 2, 100, 100, 32, True),
    (1, 2, 1, 64, 64, 32, False),
    (1, 1, 1, 1, 1, 128, False),
    (1, 2, 1, 3, 700, 128, True),
    (1, 8, 8, 129, 129, 128, True),
    (1, 8, 1, 150, 150, 64, False),   # eight query heads per KV head
    (2, 16, 2, 97, 161, 128, True),   # GQA 8, Nq < Nk, ragged in both
    (1, 2, 1, 100, 100, 256, True),   # d = 256: 32-key dQ tiles, one wave per SIMD
    (1, 4, 2, 77, 210, 256, True),
    (1, 2, 2, 130, 97, 256, False),
]


@pytest.mark.parametrize("shape", ODD, ids=[
    f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_Nq{s[3]}_Nk{s[4]}_d{s[5]}_{'c' if s[6] else 'nc'}" for s in ODD])
def test_bwd_full_parity(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    tag = f"bwd B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal}"
    announce(tag)
    cfg = datagen.fwd_config(tag, B, Hq, Nq, d, causal, seed=500 + Nq + Nk + d,
                             Hkv=Hkv, Nk=Nk)
    qb, kb, vb, dob = datagen.make_bwd_inputs(cfg)
    q64, k64, v64, do64 = (datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb, dob))
    ob, lse32 = _oracle_fwd_outputs(q64, k64, v64, cfg.scale, causal)
    dq, dk, dv = _bwd_on_gpu(qb, kb, vb, dob, ob, lse32, cfg.scale, causal)
    rq, rk, rv = oracle.attention_bwd_ref(q64, k64, v64, do64, cfg.scale, causal)
    refs = dict(Q=rq, K=rk, V=rv)
    bounds = grad_error_bounds(q64, k64, v64, do64, datagen.f64_from_bf16_bits(ob),
                               lse32.astype(np.float64), cfg.scale, causal, refs)
    assert_grad_parity(tag, dict(Q=host_f64(dq), K=host_f64(dk), V=host_f64(dv)), refs, bounds)


def _workload_case(name, heads, rows_per_head=None, keys_per_head=None):
    """GPU forward then backward on a whole workload; oracle gradients on
    sampled (b, h) pairs (all rows and keys, or seeded subsets)."""
    import torch
    cfg = datagen.CONFIGS[name]
    announce(f"bwd workload {name} heads {heads}")
    qb, kb, vb, dob = datagen.make_bwd_inputs(cfg)
    q, k, v, do = (dev_bf16(x) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=cfg.causal, scale=cfg.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=cfg.causal, scale=cfg.scale)
    torch.cuda.synchronize()
    assert cfg.Hq == cfg.Hkv, "the sampled comparison reads one query head per KV head"
    for b, h in heads:
        g = h // (cfg.Hq // cfg.Hkv)
        rows = None if rows_per_head is None else datagen.row_subset(cfg.Nq, rows_per_head, h)
        keys = None if keys_per_head is None else datagen.row_subset(cfg.Nk, keys_per_head, 100 + h)
        sel = lambda bits, bb, hh: datagen.f64_from_bf16_bits(bits[bb, hh])
        rq, rk, rv = oracle.attention_bwd_head_ref(sel(qb, b, h), sel(kb, b, g), sel(vb, b, g),
                                                   sel(dob, b, h), cfg.scale, cfg.causal,
                                                   rows=rows, keys=keys)
        gq = host_f64(dq[b, h])
        gk = host_f64(dk[b, g])
        gv = host_f64(dv[b, g])
        if rows is not None:
            gq = gq[rows]
        if keys is not None:
            gk, gv = gk[keys], gv[keys]
        refs = dict(Q=rq, K=rk, V=rv)
        bounds = head_grad_error_bounds(sel(qb, b, h), sel(kb, b, g), sel(vb, b, g),
                                        sel(dob, b, h), host_f64(o[b, h]), host_f64(lse[b, h]),
                                        cfg.scale, cfg.causal, refs, rows=rows, keys=keys)
        assert_grad_parity(f"{name} b{b} h{h}", dict(Q=gq, K=gk, V=gv), refs, bounds)


def test_bwd_train_noncausal_sampled():
    _workload_case("train_nc", [(0, 0), (5, 11)])


def test_bwd_train_causal_sampled():
    _workload_case("train_c", [(0, 3), (7, 15)])


def test_bwd_sweep_d64_sampled():
    _workload_case("sweep_d64", [(1, 9)])


def test_bwd_sweep_d256_sampled():
    _workload_case("sweep_d256", [(0, 2)], rows_per_head=512, keys_per_head=512)


def test_bwd_long_causal_sampled():
    # 256 seeded query rows (dQ) and 256 seeded keys (dK, dV) of one head.
    _workload_case("long", [(0, 5)], rows_per_head=256, keys_per_head=256)


def test_bwd_deterministic():
    import torch
    announce("bwd determinism")
    cfg = datagen.fwd_config("det", 1, 4, 300, 128, True, seed=77, Hkv=2)
    qb, kb, vb, dob = datagen.make_bwd_inputs(cfg)
    q, k, v, do = (dev_bf16(x) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_bwd_rejects_unsupported():
    import torch
    announce("bwd error paths")
    q = torch.zeros(1, 2, 64, 96, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
    assert e.value.status == -3
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.bwd(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), workspace=small)
    assert e.value.status == -5
