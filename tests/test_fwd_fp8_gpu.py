"""GPU parity tests of fa_fwd_fp8 (fp8 e4m3 inputs and products).

Inputs are the workloads' bf16 draws quantised per tensor to OCP fp8 e4m3
(datagen.make_fp8_fwd_inputs).  The oracle is the float64 forward on the
dequantised inputs (code value * descale, exact), so the comparison measures
the kernel's own arithmetic.  Bar, derived from that arithmetic: S is exact
up to fp32 accumulation, and each probability is rounded to e4m3 before the
PV product (relative error <= 2^-4, or absolute <= 2^-10 where it falls into
the e4m3 subnormal range), so for every output element
  |O - O_ref| <= 2^-4 * max|v| + 2^-8 * |O_ref| + 4e-3
(max|v| over the KV head's dequantised values; 2^-8 covers the bf16 output
rounding; 4e-3 the subnormal flush of tiny probabilities), and the LSE,
computed from the unrounded fp32 probabilities, keeps the bf16 path's bar of
1e-3.  Each report also prints the error against the oracle on the
unquantised bf16 inputs: the total quantisation effect, not a pass bar.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import announce, host_f64

import exact_attention_103_amd as fa

pytestmark = pytest.mark.gpu


def _dev_u8(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda:0")


def _check(tag, o, lse, o_ref, lse_ref, vmax, o_bf16_ref=None):
    err = np.abs(o - o_ref)
    tol = 2.0 ** -4 * vmax + 2.0 ** -8 * np.abs(o_ref) + 4e-3
    lse_err = float(np.abs(lse - lse_ref).max())
    extra = ""
    if o_bf16_ref is not None:
        extra = f" | vs bf16-input oracle: max {np.abs(o - o_bf16_ref).max():.3e} mean {np.abs(o - o_bf16_ref).mean():.3e}"
    print(f"[parity] {tag}: O max {err.max():.3e} mean {err.mean():.3e} | worst err/bound "
          f"{(err / tol).max():.3f} | LSE max {lse_err:.3e}{extra}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), tag
    assert np.all(err <= tol), f"{tag}: O error above the fp8 bound"
    assert lse_err <= 1e-3, f"{tag}: LSE error {lse_err:.3e}"


def _run(q8, k8, v8, scales, scale, causal):
    import torch
    o, lse = fa.fwd_fp8(_dev_u8(q8), _dev_u8(k8), _dev_u8(v8), *scales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


ODD = [
    (1, 2, 1, 200, 200, 128, False),
    (1, 2, 1, 200, 200, 128, True),
    (1, 4, 2, 77, 300, 128, True),
    (2, 2, 2, 130, 130, 64, True),
    (1, 4, 1, 257, 190, 64, False),
    (1, 1, 1, 1, 1, 128, False),
    (1, 8, 8, 300, 300, 128, True),
    # non-causal with B*Hq divisible by 8: head-major XCD order, query and key tails
    (1, 8, 4, 300, 1100, 128, False),
    (1, 8, 2, 1000, 2100, 128, False),
    (2, 4, 4, 129, 700, 64, False),
    # one, two and three key tiles: fewer tiles than the kernel's copy
    # pipeline is deep (the products of the last tile run after the loop)
    (1, 2, 1, 64, 64, 128, True),
    (1, 2, 2, 40, 120, 128, False),
    (1, 3, 1, 200, 130, 64, False),
    (1, 2, 1, 190, 190, 128, True),
    # d = 256 (four waves of 32 rows, one per SIMD): tails, GQA, Nq < Nk, one
    # valid row in the last query block, head-major non-causal order
    (1, 2, 1, 200, 200, 256, False),
    (1, 2, 1, 200, 200, 256, True),
    (1, 4, 2, 77, 300, 256, True),
    (1, 2, 1, 129, 190, 256, False),
    (2, 2, 2, 130, 130, 256, True),
    (1, 8, 4, 300, 1100, 256, False),
    # d = 32: one k-step with the upper lane half zero, 32-byte LDS rows;
    # tails, GQA, Nq < Nk, one and two key tiles, head-major order
    (1, 2, 1, 200, 200, 32, False),
    (1, 2, 1, 200, 200, 32, True),
    (1, 4, 2, 77, 300, 32, True),
    (2, 2, 2, 130, 130, 32, True),
    (1, 8, 4, 300, 1100, 32, False),
    (1, 2, 1, 64, 64, 32, True),
    (1, 3, 1, 40, 100, 32, False),
]


@pytest.mark.parametrize("shape", ODD, ids=[
    f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_Nq{s[3]}_Nk{s[4]}_d{s[5]}_{'c' if s[6] else 'nc'}" for s in ODD])
def test_fp8_full_parity(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    tag = f"fp8 B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal}"
    announce(tag)
    cfg = datagen.fwd_config(tag, B, Hq, Nq, d, causal, seed=700 + Nq + Nk + d, Hkv=Hkv, Nk=Nk)
    (q8, k8, v8), sc = datagen.make_fp8_fwd_inputs(cfg)
    qd, kd, vd = (datagen.f64_from_fp8_e4m3_bits(x) * s for x, s in zip((q8, k8, v8), sc))
    o, lse = _run(q8, k8, v8, sc, cfg.scale, causal)
    o_ref, lse_ref = oracle.attention_ref(qd, kd, vd, cfg.scale, causal)
    vmax = np.abs(vd).max(axis=(2, 3))                       # [B][Hkv]
    vmax = np.repeat(vmax, Hq // Hkv, axis=1)[:, :, None, None]
    qb, kb, vb = datagen.make_fwd_inputs(cfg)
    o_bf, _ = oracle.attention_ref(*(datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb)),
                                   cfg.scale, causal)
    _check(tag, o, lse, o_ref, lse_ref, vmax, o_bf)


def _workload(name, heads, rows_per_head):
    import torch
    cfg = datagen.CONFIGS[name]
    announce(f"fp8 workload {name}")
    (q8, k8, v8), sc = datagen.make_fp8_fwd_inputs(cfg)
    o, lse = fa.fwd_fp8(_dev_u8(q8), _dev_u8(k8), _dev_u8(v8), *sc, causal=cfg.causal,
                        scale=cfg.scale)
    torch.cuda.synchronize()
    for b, h in heads:
        g = h // (cfg.Hq // cfg.Hkv)
        rows = datagen.row_subset(cfg.Nq, rows_per_head, h)
        qd = datagen.f64_from_fp8_e4m3_bits(q8[b, h]) * sc[0]
        kd = datagen.f64_from_fp8_e4m3_bits(k8[b, g]) * sc[1]
        vd = datagen.f64_from_fp8_e4m3_bits(v8[b, g]) * sc[2]
        o_ref, lse_ref = oracle.attention_head_ref(qd, kd, vd, cfg.scale, cfg.causal, rows=rows)
        _check(f"fp8 {name} b{b} h{h}", host_f64(o[b, h])[rows], host_f64(lse[b, h])[rows],
               o_ref, lse_ref, np.abs(vd).max())


def test_fp8_long_sampled():
    _workload("long", [(0, 0), (0, 21)], 256)


def test_fp8_train_sampled():
    _workload("train_nc", [(0, 0), (7, 15)], 256)
    _workload("train_c", [(3, 5)], 256)


def test_fp8_sweep_d256_sampled():
    _workload("sweep_d256", [(0, 0), (1, 13)], 256)


def test_fp8_sweep_d32_sampled():
    _workload("sweep_d32", [(0, 0), (1, 9)], 256)


@pytest.mark.parametrize("slope", [0.2, 1.0, -1.0])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_fp8_drifting_scores(slope, d):
    """Rising scores exceed the reference maximum by far more than 2^8 in
    tile after tile, so the tile's probabilities are redone against a new
    reference in the middle of rows; falling scores never move it."""
    B, H, N = 1, 2, 300
    bits = datagen.drifting_bf16(60 + d, B, H, H, N, d, slope)
    quant = [datagen.quantize_fp8_e4m3(datagen.f64_from_bf16_bits(x)) for x in bits]
    q8, k8, v8 = (c for c, _ in quant)
    sc = tuple(s for _, s in quant)
    qd, kd, vd = (datagen.f64_from_fp8_e4m3_bits(c) * s for c, s in zip((q8, k8, v8), sc))
    for causal in (False, True):
        tag = f"fp8 drift slope={slope} d={d} causal={causal}"
        announce(tag)
        o, lse = _run(q8, k8, v8, sc, 1 / np.sqrt(d), causal)
        o_ref, lse_ref = oracle.attention_ref(qd, kd, vd, 1 / np.sqrt(d), causal)
        _check(tag, o, lse, o_ref, lse_ref, np.abs(vd).max())


def test_fp8_deterministic():
    import torch
    announce("fp8 determinism")
    cfg = datagen.fwd_config("det8", 1, 4, 300, 128, True, seed=9, Hkv=2)
    (q8, k8, v8), sc = datagen.make_fp8_fwd_inputs(cfg)
    q, k, v = _dev_u8(q8), _dev_u8(k8), _dev_u8(v8)
    a = fa.fwd_fp8(q, k, v, *sc, causal=True)
    b = fa.fwd_fp8(q, k, v, *sc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
