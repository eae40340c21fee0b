"""GPU test of fa_decode_splitkv_noalloc, the allocation-free decode entry point.

Its outputs must equal fa_decode_splitkv's (same kernels, same split count,
workspace from the caller) bit for bit, and meet the oracle's parity bar, on
two calls in a row: the decode workload (8 sequences, 32 query heads over 8 KV
heads, 32768 cached keys, d = 128) and then a smaller, ragged one, which finds
the fixed scratch still holding the first call's partials.  Everything goes
through the C ABI (ctypes); the outputs are preallocated, the entry point
itself allocates nothing.
"""

import numpy as np
import pytest

import datagen
import oracle
from parity import announce, assert_parity, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _oracle(qb, kb, vb, scale):
    q, k, v = (datagen.f64_from_bf16_bits(x) for x in (qb, kb, vb))
    o, lse = oracle.attention_ref(q[:, :, None, :], k, v, scale, causal=False)
    return o[:, :, 0], lse[:, :, 0]


def _both(qb, kb, vb, scale, splits):
    import torch
    import exact_attention_103_amd as fa
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    B, Hq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    o1 = torch.empty_like(q)
    l1 = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    rc = fa.fa_decode_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                                      l1.data_ptr(), B, Hq, Hkv, Nk, d, scale, splits, stream)
    assert rc == 0, fa.fa_strerror(rc)
    S = splits or fa.fa_decode_num_splits(B, Hq, Hkv, Nk, d)
    ws = torch.empty(fa.fa_decode_workspace_size(B, Hq, d, S), dtype=torch.uint8,
                     device=q.device)
    o2 = torch.empty_like(q)
    l2 = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    rc = fa.fa_decode_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                              l2.data_ptr(), B, Hq, Hkv, Nk, d, scale, S, ws.data_ptr(),
                              ws.numel(), stream)
    assert rc == 0, fa.fa_strerror(rc)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def _check(tag, qb, kb, vb, scale, splits):
    import torch
    announce(f"noalloc {tag} splits={splits} q={qb.shape} k={kb.shape}")
    o1, l1, o2, l2 = _both(qb, kb, vb, scale, splits)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{tag}: O differs"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{tag}: LSE differs"
    o_ref, lse_ref = _oracle(qb, kb, vb, scale)
    assert_parity(f"noalloc {tag}", host_f64(o1), host_f64(l1), o_ref, lse_ref)


def test_noalloc_decode_twice_then_smaller():
    cfg = datagen.CONFIGS["decode"]
    qb, kb, vb = datagen.make_decode_inputs(cfg)
    # first call: the decode workload with the most splits the scratch holds
    # for it (4*8*32*127*129 bytes of 16 MiB)
    _check("workload", qb, kb, vb, cfg.scale, 127)
    # second call: smaller and ragged, fewer heads, another head dim; the
    # scratch still holds the first call's partials
    qs, ks, vs = datagen.gaussian_bf16(4242, [(3, 6, 64), (3, 2, 1000, 64), (3, 2, 1000, 64)])
    _check("small", qs, ks, vs, 0.125, 0)


def test_noalloc_rejects_oversized_partials():
    import torch
    import exact_attention_103_amd as fa
    cfg = datagen.CONFIGS["decode"]
    B, Hq, Hkv, Nk, d = 8, 32, 8, 32768, 128
    assert cfg.B == B and cfg.Hq == Hq
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.decode_noalloc(q, k, k, o, lse, num_splits=128)
    assert e.value.status == -11
    # the torch-facing wrapper at a size that fits gives the C entry's result
    o_np = np.asarray(host_f64(fa.decode_noalloc(q, k, k, o, lse, num_splits=64)[0]))
    assert np.all(o_np == 0.0)
