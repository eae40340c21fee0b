"""GPU parity of fa_fp8_quantize (incoherent processing + per-tensor e4m3
quantisation) and of the fp8 forward fed by it, against the float64 oracle.

Codes: the kernel rotates in fp32 (a fast Walsh-Hadamard transform) and
takes the rounding decision on its fp32 value of 448 * u / max|u|; the
oracle takes it on the exact value.  The two may therefore pick neighbouring
codes when the exact value lies within the fp32 error of a rounding midpoint,
so the comparison is exact everywhere except in such a window (|t - midpoint|
<= 1e-4 in code units with rotation, relative 1e-6 without), where the
kernel's code must be one of the two neighbours; -0 and +0 are the same
value.  Descale: relative 1e-5 (the fp32 maximum of the transform).

End to end: bf16 Q, K, V -> fa_fp8_quantize (Q and K rotated with the same
signs, V not) -> fa_fwd_fp8_devscale, against the float64 forward on the
oracle's own dequantised codes, at the fp8 forward's bound
|O - O_ref| <= 2^-4 max|v| + 2^-8 |O_ref| + 4e-3 and LSE 1e-3.  Since
(QR)(KR)^T = QK^T, the same outputs are also compared (reported, and for
outlier-channel inputs asserted to improve with the rotation) against the
unquantised bf16 oracle.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import announce, dev_bf16, host_f64

import exact_attention_103_amd as fa

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _quantize(xb, signs):
    import torch
    codes, ds = fa.fp8_quantize(dev_bf16(xb), _dev(signs) if signs is not None else None)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), float(ds.cpu().item())


def _check_codes(tag, got, y, descale_ref, rotated):
    """got: kernel codes; y: oracle values (rotated or not) of the same rows."""
    t = y / descale_ref
    want = oracle.e4m3_round_ref(t)
    w = 1e-4 + 1e-6 * np.abs(t) if rotated else 1e-6 * np.abs(t)
    lo, hi = oracle.e4m3_round_ref(t - w), oracle.e4m3_round_ref(t + w)
    zero = ((got & 0x7F) == 0) & ((want & 0x7F) == 0)
    same = (got == want) | zero
    near = ~same & ((got == lo) | (got == hi))
    bad = ~same & ~near
    print(f"[parity] {tag}: {got.size} codes, {int(near.sum())} neighbouring codes at "
          f"midpoints, {int(bad.sum())} wrong", flush=True)
    assert not bad.any(), f"{tag}: first wrong code at {np.argwhere(bad)[0]}: " \
        f"{got[bad][0]:#x} vs {want[bad][0]:#x} (t = {t[bad][0]!r})"
    assert near.sum() <= max(4, 1e-3 * got.size), f"{tag}: too many midpoint cases"


CASES = [  # (rows, d, rotated, outliers)
    (1, 128, True, False), (7, 64, True, False), (33, 128, True, True), (1000, 64, False, False),
    (1000, 128, False, True), (20000, 128, True, False), (4097, 64, True, True),
    (300, 128, True, True),
    # 8 rows: one wave's row group, the other waves idle; 50001 rows: the
    # grid's second row group per iteration ends partway.
    (8, 128, True, True), (50001, 128, True, False),
    # d = 256: a whole DPP row per tensor row (lane distance 8 is the row
    # rotation); 5 rows: part of one wave's row group
    (5, 256, True, False), (1000, 256, True, True), (3001, 256, False, False),
    (20000, 256, True, False),
    # d = 32: two lanes per row, one butterfly between lanes
    (3, 32, True, False), (1000, 32, True, True), (4099, 32, False, False),
    (50001, 32, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"rows{c[0]}_d{c[1]}_{'rot' if c[2] else 'plain'}{'_outl' if c[3] else ''}" for c in CASES])
def test_quantize_parity(case):
    rows, d, rotated, outliers = case
    tag = f"quantize rows={rows} d={d} rotated={rotated} outliers={outliers}"
    announce(tag)
    seed = 1000 + rows + d
    xb = (datagen.outlier_bf16(seed, (rows, d)) if outliers
          else datagen.gaussian_bf16(seed, [(rows, d)])[0])
    signs = datagen.random_signs(seed, d) if rotated else None
    got, ds = _quantize(xb, signs)
    x64 = datagen.f64_from_bf16_bits(xb)
    codes_ref, ds_ref = oracle.rotate_quantize_ref(x64, signs)
    assert ds == pytest.approx(ds_ref, rel=1e-5), (ds, ds_ref)
    y = oracle.rotate_ref(x64, signs) if rotated else x64
    _check_codes(tag, got, y, ds_ref, rotated)


def test_quantize_zero_and_repeat():
    import torch
    announce("quantize zeros / determinism")
    xb = np.zeros((64, 128), dtype=np.uint16)
    got, ds = _quantize(xb, datagen.random_signs(5, 128))
    assert ds == 1.0 and np.all((got & 0x7F) == 0)
    xb = datagen.gaussian_bf16(6, [(999, 128)])[0]
    s = _dev(datagen.random_signs(6, 128))
    x = dev_bf16(xb)
    a = fa.fp8_quantize(x, s)
    b = fa.fp8_quantize(x, s)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_quantize_long_workload_sampled():
    """Q of the 16k-token prefill (32 heads x 16384 rows x 128): descale
    from the oracle's full rotation, codes on 8192 seeded rows."""
    cfg = datagen.CONFIGS["long"]
    announce("quantize long workload")
    qb = datagen.make_fwd_inputs(cfg)[0]
    signs = datagen.random_signs(cfg.seed, cfg.d)
    got, ds = _quantize(qb, signs)
    x64 = datagen.f64_from_bf16_bits(qb).reshape(-1, cfg.d)
    R = oracle.rotate_ref(np.eye(cfg.d), signs)
    amax = 0.0
    for r0 in range(0, x64.shape[0], 65536):
        amax = max(amax, float(np.abs(x64[r0:r0 + 65536] @ R).max()))
    ds_ref = amax / 448.0
    assert ds == pytest.approx(ds_ref, rel=1e-5)
    rows = datagen.row_subset(x64.shape[0], 8192, 0)
    _check_codes("quantize long sampled", got.reshape(-1, cfg.d)[rows], x64[rows] @ R, ds_ref,
                 True)


def _pipeline(qb, kb, vb, signs, causal, scale):
    """GPU: quantise (Q, K rotated) and run the fp8 forward with device
    descales.  Returns host O, LSE."""
    import torch
    s = _dev(signs) if signs is not None else None
    q8, qd = fa.fp8_quantize(dev_bf16(qb), s)
    k8, kd = fa.fp8_quantize(dev_bf16(kb), s)
    v8, vd = fa.fp8_quantize(dev_bf16(vb), None)
    o, lse = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


def _oracle_pipeline(qb, kb, vb, signs, causal, scale):
    """Oracle: its own codes and descales, then the float64 forward on the
    dequantised values; also max|v| per KV head for the bound."""
    deq = []
    for x, sg in ((qb, signs), (kb, signs), (vb, None)):
        c, ds = oracle.rotate_quantize_ref(datagen.f64_from_bf16_bits(x), sg)
        deq.append(oracle.e4m3_decode_ref(c) * ds)
    o, lse = oracle.attention_ref(deq[0], deq[1], deq[2], scale, causal)
    return o, lse, deq[2]


E2E = [(1, 4, 2, 200, 200, 128, True), (1, 2, 2, 130, 300, 64, False),
       (2, 4, 4, 257, 257, 128, False), (1, 8, 2, 64, 1000, 128, True),
       (1, 2, 1, 200, 200, 256, True), (1, 4, 2, 130, 300, 256, False),
       (1, 2, 1, 200, 200, 32, True), (1, 4, 2, 130, 300, 32, False)]


@pytest.mark.parametrize("shape", E2E, ids=[
    f"B{s[0]}_Hq{s[1]}_Hkv{s[2]}_Nq{s[3]}_Nk{s[4]}_d{s[5]}_{'c' if s[6] else 'nc'}" for s in E2E])
def test_quantize_then_fp8_forward(shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    tag = f"rotate+fp8 B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal}"
    announce(tag)
    seed = 2000 + Nq + Nk + d
    # Outlier channels x6 in both Q and K (x20 puts scores of several hundred
    # into the LSE, whose fp32 accumulation then exceeds the 1e-3 bar).
    qb = datagen.outlier_bf16(seed, (B, Hq, Nq, d), gain=6.0)
    kb = datagen.outlier_bf16(seed + 1, (B, Hkv, Nk, d), gain=6.0)
    vb = datagen.gaussian_bf16(seed + 2, [(B, Hkv, Nk, d)])[0]
    signs = datagen.random_signs(seed, d)
    scale = 1.0 / np.sqrt(d)
    o, lse = _pipeline(qb, kb, vb, signs, causal, scale)
    o_ref, lse_ref, vd = _oracle_pipeline(qb, kb, vb, signs, causal, scale)
    err = np.abs(o - o_ref)
    tol = 2.0 ** -4 * np.abs(vd).max() + 2.0 ** -8 * np.abs(o_ref) + 4e-3
    lse_err = np.abs(lse - lse_ref).max()
    # Against the unquantised inputs, with and without the rotation.
    o_bf, _ = oracle.attention_ref(*(datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb)),
                                   scale, causal)
    o_plain, _ = _pipeline(qb, kb, vb, None, causal, scale)
    e_rot, e_plain = np.abs(o - o_bf).mean(), np.abs(o_plain - o_bf).mean()
    print(f"[parity] {tag}: O max {err.max():.3e} (worst err/bound {(err / tol).max():.3f}) "
          f"LSE max {lse_err:.3e} | vs bf16 inputs: rotated mean {e_rot:.3e}, "
          f"unrotated mean {e_plain:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(err <= tol), tag
    assert lse_err <= 1e-3, tag
    assert e_rot < e_plain, f"{tag}: rotation did not reduce the quantisation error"


def test_devscale_equals_value_scales():
    """Device descales and the same values passed as arguments give
    identical bits."""
    import torch
    announce("fp8 devscale == value scales")
    B, H, N, d = 1, 4, 300, 128
    qb, kb, vb = datagen.gaussian_bf16(77, [(B, H, N, d)] * 3)
    s = _dev(datagen.random_signs(77, d))
    q8, qd = fa.fp8_quantize(dev_bf16(qb), s)
    k8, kd = fa.fp8_quantize(dev_bf16(kb), s)
    v8, vd = fa.fp8_quantize(dev_bf16(vb))
    a = fa.fwd_fp8(q8, k8, v8, qd, kd, vd, causal=True)
    b = fa.fwd_fp8(q8, k8, v8, qd.item(), kd.item(), vd.item(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
