"""Race check: the pipelined kernels against their serial build, bit for bit.

libfa_serial.so is compiled from the same sources with FA_SERIAL_PIPELINE:
around every staged copy into LDS each wave waits for all of its memory
operations and (for workgroup-shared buffers) for every other wave, so no
copy overlaps a read of its buffer or any compute.  The arithmetic and its
order are the same in both builds, so every output must agree exactly.  A
difference means a staged copy raced with the reads of its buffer (a missing
wait or barrier in the pipelined schedule), which a tolerance-based parity
test could miss when the stale data happens to be close.

Each case runs the pipelined library, then the serial one, on the same
device inputs, and compares the raw bits of every output.
"""

import numpy as np
import pytest

import datagen
from parity import announce, dev_bf16

import exact_attention_103_amd as fa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def serial_lib():
    assert fa.lib().fa_build_is_serial() == 0   # the pipelined build stays the default
    serial = fa.load_library(fa.SERIAL_LIB_PATH)
    assert serial.fa_build_is_serial() == 1, "libfa_serial.so is not the race-check build"
    return serial


def _bits(t):
    import torch
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _both(run, serial_lib, monkeypatch):
    """Outputs of run() with the pipelined build, then with the serial one."""
    import torch
    a = run()
    torch.cuda.synchronize()
    with monkeypatch.context() as m:
        m.setattr(fa, "_lib", serial_lib)
        b = run()
        torch.cuda.synchronize()
    return a, b


def _assert_same(tag, a, b):
    import torch
    for i, (x, y) in enumerate(zip(a, b)):
        bx, by = _bits(x), _bits(y)
        diff = int((bx != by).sum().item())
        assert diff == 0, f"{tag}: output {i} differs from the serial build in {diff} of " \
                          f"{bx.numel()} elements"
        assert torch.equal(bx, by)


FWD = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 4, 2, 1000, 1000, 32, True),
    (1, 4, 1, 333, 700, 32, False),
    (2, 4, 2, 1000, 1000, 64, True),
    (1, 2, 2, 129, 1000, 64, False),
    (1, 4, 2, 1000, 1000, 128, True),     # 128-row tile
    (1, 2, 1, 4500, 4500, 128, True),     # 256-row tile (long key range)
    (1, 2, 2, 700, 2100, 128, False),     # 256-row tile, non-causal
    (1, 8, 2, 300, 2100, 128, False),     # 256-row tile, head-major XCD order
    (1, 4, 4, 1000, 1000, 256, True),
    (1, 2, 1, 65, 1000, 256, False),
]


@pytest.mark.parametrize("shape", FWD, ids=[
    "B{}_H{}x{}_Nq{}_Nk{}_d{}_{}".format(*s[:6], "c" if s[6] else "nc") for s in FWD])
def test_fwd_matches_serial_build(shape, serial_lib, monkeypatch):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    announce(f"race fwd {shape} kernel {fa.fa_fwd_kernel_name(d, causal, Nq, Nk)}")
    qb, kb, vb = datagen.gaussian_bf16(500 + d, [(B, Hq, Nq, d), (B, Hkv, Nk, d),
                                                 (B, Hkv, Nk, d)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    a, b = _both(lambda: fa.fwd(q, k, v, causal=causal), serial_lib, monkeypatch)
    _assert_same(f"fwd {shape}", a, b)


FP8 = [(1, 4, 2, 1000, 1000, 64, True), (1, 2, 1, 3000, 3000, 128, True),
       (1, 2, 2, 300, 1100, 128, False),
       (1, 8, 4, 300, 1100, 128, False),    # head-major XCD order
       (1, 2, 1, 190, 190, 128, True), (1, 2, 2, 40, 120, 64, False),   # 2-3 key tiles
       (1, 4, 2, 700, 1000, 256, True), (1, 8, 4, 300, 1100, 256, False)]


@pytest.mark.parametrize("shape", FP8, ids=[
    "B{}_H{}x{}_Nq{}_Nk{}_d{}_{}".format(*s[:6], "c" if s[6] else "nc") for s in FP8])
def test_fwd_fp8_matches_serial_build(shape, serial_lib, monkeypatch):
    import torch
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    announce(f"race fwd_fp8 {shape}")
    qb, kb, vb = datagen.gaussian_bf16(600 + d, [(B, Hq, Nq, d), (B, Hkv, Nk, d),
                                                 (B, Hkv, Nk, d)])
    codes = [datagen.quantize_fp8_e4m3(datagen.f64_from_bf16_bits(x)) for x in (qb, kb, vb)]
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(c)).to("cuda:0") for c, _ in codes)
    sc = [s for _, s in codes]
    a, b = _both(lambda: fa.fwd_fp8(q8, k8, v8, *sc, causal=causal), serial_lib, monkeypatch)
    _assert_same(f"fwd_fp8 {shape}", a, b)


DEC = [  # (B, Hq, Hkv, Nk, d, splits)
    (2, 8, 2, 5000, 128, 0),
    (2, 8, 2, 5000, 128, 7),
    (1, 16, 1, 3333, 64, 5),
    (3, 4, 4, 999, 32, 3),
    (1, 8, 8, 2048, 256, 4),
]


@pytest.mark.parametrize("shape", DEC, ids=["B{}_H{}x{}_Nk{}_d{}_S{}".format(*s) for s in DEC])
def test_decode_matches_serial_build(shape, serial_lib, monkeypatch):
    B, Hq, Hkv, Nk, d, S = shape
    announce(f"race decode {shape}")
    qb, kb, vb = datagen.gaussian_bf16(700 + d, [(B, Hq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    a, b = _both(lambda: fa.decode(q, k, v, num_splits=S), serial_lib, monkeypatch)
    _assert_same(f"decode {shape}", a, b)


def test_decode_serve_matches_serial_build(serial_lib, monkeypatch):
    import torch
    B, Hq, Hkv, Nq, Nk, d = 4, 8, 2, 4, 3000, 128
    announce(f"race decode_serve B{B} H{Hq}x{Hkv} Nq{Nq} Nk{Nk} d{d}")
    qb, kb, vb = datagen.gaussian_bf16(800, [(B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)])
    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    seqlens = torch.tensor([3000, 17, 1234, 4], dtype=torch.int32, device="cuda:0")
    a, b = _both(lambda: fa.decode_serve(q, k, v, seqlens, causal=True, num_splits=5),
                 serial_lib, monkeypatch)
    _assert_same("decode_serve", a, b)


BWD = [  # (B, Hq, Hkv, Nq, Nk, d, causal)
    (1, 4, 2, 1000, 1000, 32, True),
    (1, 2, 2, 700, 1000, 64, False),
    (1, 4, 2, 1000, 1000, 128, True),
    (1, 2, 1, 333, 1111, 128, False),
    (1, 4, 2, 700, 1000, 256, True),
]


@pytest.mark.parametrize("shape", BWD, ids=[
    "B{}_H{}x{}_Nq{}_Nk{}_d{}_{}".format(*s[:6], "c" if s[6] else "nc") for s in BWD])
def test_bwd_matches_serial_build(shape, serial_lib, monkeypatch):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    announce(f"race bwd {shape}")
    qb, kb, vb, dob = datagen.gaussian_bf16(900 + d, [(B, Hq, Nq, d), (B, Hkv, Nk, d),
                                                      (B, Hkv, Nk, d), (B, Hq, Nq, d)])
    q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(dob)
    o, lse = fa.fwd(q, k, v, causal=causal)
    a, b = _both(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal), serial_lib, monkeypatch)
    _assert_same(f"bwd {shape}", a, b)
