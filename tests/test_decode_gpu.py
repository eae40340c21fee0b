"""GPU parity of fa_decode_splitkv against the float64 oracle (through the C ABI).

The decode workload (8 sequences, 32 query heads over 8 KV heads, 32768
cached keys, d = 128) is checked on every output at split counts 16, 32, 64
and the heuristic's choice; small shapes cover ragged caches, every head
dimension, GQA group sizes that do and do not divide 8, and split counts from
1 to the maximum (which leaves empty chunks).
"""

import math

import numpy as np
import pytest

import datagen
import oracle
from parity import announce, assert_parity, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _fa():
    import exact_attention_103_amd as fa
    return fa


def _run(qb, kb, vb, scale, splits, keep_workspace=False):
    import torch
    fa = _fa()
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    B, Hq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    S = splits or fa.fa_decode_num_splits(B, Hq, Hkv, Nk, d)
    ws = torch.empty(fa.fa_decode_workspace_size(B, Hq, d, S), dtype=torch.uint8,
                     device="cuda")
    o, lse = fa.decode(q, k, v, scale=scale, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    if keep_workspace:
        return host_f64(o), host_f64(lse), ws, S
    return host_f64(o), host_f64(lse)


def _oracle(qb, kb, vb, scale):
    q, k, v = (datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb))
    o, lse = oracle.attention_ref(q[:, :, None, :], k, v, scale, causal=False)
    return o[:, :, 0], lse[:, :, 0]


@pytest.mark.parametrize("splits", [16, 32, 64, 0])
def test_decode_workload_full(splits):
    cfg = datagen.CONFIGS["decode"]
    announce(f"decode workload splits={splits}")
    qb, kb, vb = datagen.make_decode_inputs(cfg)
    o, lse = _run(qb, kb, vb, cfg.scale, splits)
    o_ref, lse_ref = _oracle(qb, kb, vb, cfg.scale)
    assert_parity(f"decode S={splits}", o, lse, o_ref, lse_ref)


ODD = [  # (B, Hq, Hkv, Nk, d, splits)
    (1, 1, 1, 1, 128, 1),
    (1, 4, 1, 17, 64, 0),
    (2, 8, 2, 63, 32, 1),
    (1, 2, 2, 65, 256, 2),
    (2, 16, 2, 129, 128, 3),
    (1, 6, 2, 1000, 128, 16),
    (3, 6, 1, 1000, 64, 5),
    (1, 16, 1, 1000, 32, 0),
    (2, 32, 4, 4097, 256, 0),
    (1, 4, 4, 640, 128, 10),
    (1, 8, 8, 200, 64, 4),
]


@pytest.mark.parametrize("shape", ODD, ids=[
    "B{}_H{}x{}_Nk{}_d{}_S{}".format(*s) for s in ODD])
def test_decode_odd_shapes_full(shape):
    B, Hq, Hkv, Nk, d, S = shape
    announce(f"decode odd shape {shape}")
    qb, kb, vb = datagen.gaussian_bf16(9000 + Nk + d + Hq,
                                       [(B, Hq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)])
    scale = 1 / math.sqrt(d)
    o, lse = _run(qb, kb, vb, scale, S)
    o_ref, lse_ref = _oracle(qb, kb, vb, scale)
    assert_parity(f"decode odd {shape}", o, lse, o_ref, lse_ref)


def test_decode_partials_match_chunked_oracle():
    """The split kernel's per-chunk (O_s, LSE_s), read back from the
    workspace ([B][Hq][S][d] then [B][Hq][S], fp32), against the oracle on
    each chunk; empty chunks must carry LSE = -inf."""
    import torch
    # 600 keys in 7 splits: chunks of 128 keys, so splits 5 and 6 are empty.
    B, Hq, Hkv, Nk, d, S = 2, 8, 2, 600, 128, 7
    announce("decode partial states")
    qb, kb, vb = datagen.gaussian_bf16(31, [(B, Hq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)])
    scale = 1 / math.sqrt(d)
    o, lse, ws, S = _run(qb, kb, vb, scale, S, keep_workspace=True)
    raw = ws.view(torch.float32).cpu().numpy().astype(np.float64)
    o_part = raw[:B * Hq * S * d].reshape(B, Hq, S, d)
    lse_part = raw[B * Hq * S * d:B * Hq * S * (d + 1)].reshape(B, Hq, S)
    q, k, v = (datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb))
    chunk = 64 * math.ceil(math.ceil(Nk / S) / 64)
    for s in range(S):
        a, e = s * chunk, min((s + 1) * chunk, Nk)
        if a >= e:
            assert np.all(lse_part[:, :, s] == -np.inf)
            continue
        o_s, l_s = oracle.attention_ref(q[:, :, None], k[:, :, a:e], v[:, :, a:e], scale)
        assert_parity(f"partial chunk {s}", o_part[:, :, s], lse_part[:, :, s],
                      o_s[:, :, 0], l_s[:, :, 0])
    o_m, l_m = oracle.merge_partials(np.moveaxis(o_part, 2, 0), np.moveaxis(lse_part, 2, 0))
    assert_parity("merge of GPU partials", o, lse, o_m, l_m)


def test_decode_chunk_rounding_and_empty_chunks():
    """Chunks are ceil(Nk/S) keys rounded up to 64: (130, 3) ends with a
    2-key chunk, (65, 2) with a 1-key chunk, (600, 7) and (1000, 9) leave
    empty chunks at the end, which must get weight 0."""
    for Nk, S in [(130, 3), (129, 3), (65, 2), (64, 1), (200, 4), (600, 7), (1000, 9)]:
        announce(f"decode chunking Nk={Nk} S={S}")
        qb, kb, vb = datagen.gaussian_bf16(40 + Nk, [(1, 4, 64), (1, 2, Nk, 64), (1, 2, Nk, 64)])
        o, lse = _run(qb, kb, vb, 0.125, S)
        o_ref, lse_ref = _oracle(qb, kb, vb, 0.125)
        assert_parity(f"chunking Nk={Nk} S={S}", o, lse, o_ref, lse_ref)


def test_decode_matches_forward_single_row_and_causal_last_row():
    import torch
    fa = _fa()
    announce("decode vs fwd consistency")
    B, Hq, Hkv, N, d = 2, 8, 2, 1000, 128
    qb, kb, vb = datagen.gaussian_bf16(50, [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o_c, l_c = fa.fwd(q, k, v, causal=True)
    q_last = q[:, :, -1].contiguous()
    o_1, l_1 = fa.fwd(q[:, :, -1:].contiguous(), k, v, causal=False)
    o_d, l_d = fa.decode(q_last, k, v, num_splits=7)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(qb[:, :, -1], kb, vb, 1 / math.sqrt(d))
    assert_parity("causal fwd last row", host_f64(o_c[:, :, -1]), host_f64(l_c[:, :, -1]),
                  o_ref, lse_ref)
    assert_parity("fwd Nq=1", host_f64(o_1[:, :, 0]), host_f64(l_1[:, :, 0]), o_ref, lse_ref)
    assert_parity("decode", host_f64(o_d), host_f64(l_d), o_ref, lse_ref)


def test_decode_repeat_runs_are_bit_identical():
    import torch
    fa = _fa()
    announce("decode determinism")
    qb, kb, vb = datagen.gaussian_bf16(60, [(4, 16, 128), (4, 4, 5000, 128), (4, 4, 5000, 128)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    o1, l1 = fa.decode(q, k, v)
    o2, l2 = fa.decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_decode_float32_workspace_counts_bytes():
    """A caller's workspace of another element type is sized in bytes: a
    float32 tensor of exactly workspace_size/4 elements must be accepted and
    give the same bits as the default uint8 workspace."""
    import torch
    fa = _fa()
    announce("decode float32 workspace")
    B, Hq, Hkv, Nk, d, S = 2, 8, 2, 3000, 128, 7
    qb, kb, vb = datagen.gaussian_bf16(77, [(B, Hq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    need = fa.fa_decode_workspace_size(B, Hq, d, S)
    assert need % 4 == 0
    ws32 = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    o1, l1 = fa.decode(q, k, v, num_splits=S, workspace=ws32)
    o2, l2 = fa.decode(q, k, v, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    with pytest.raises(fa.FAError) as ei:
        fa.decode(q, k, v, num_splits=S, workspace=ws32[:-1])
    assert ei.value.status == -5
