"""Throughput table for every workload shape (one GPU).

    python -m exact_attention_103_amd.perf [--iters 20] [--warmup 5]

Prints one JSON line per workload: the kernel that ran, the median launch
time (HIP events on the launch stream) and TFLOP/s for the forward (flop =
4*B*H*Nq*Nk*d, halved when causal), for the backward (the algorithmic five
products, 2.5x the forward's flop) or GB/s for the decode (K + V cache read
once, plus q, O and LSE; for the serving decode only each sequence's first
seqlens[b] keys count; for the fp8 quantisation 3 bytes per element).  Inputs are random bf16 tensors of the workload's
shape and scaling; the forward's speed does not depend on the values.
"""

from __future__ import annotations

import argparse
import json
import time

import torch

import exact_attention_103_amd as fa

FWD = [  # name, B, H, N, d, causal, input scale
    ("train_nc", 8, 16, 2048, 128, False, 1.0),
    ("train_c", 8, 16, 2048, 128, True, 1.0),
    ("long", 1, 32, 16384, 128, True, 1.0),
    ("sweep_d32", 2, 16, 4096, 32, True, 32 ** -0.5),
    ("sweep_d64", 2, 16, 4096, 64, True, 64 ** -0.5),
    ("sweep_d128", 2, 16, 4096, 128, True, 128 ** -0.5),
    ("sweep_d256", 2, 16, 4096, 256, True, 256 ** -0.5),
]
DECODE = [(8, 32, 8, 32768, 128, s) for s in (0, 16, 32, 64)]
SERVE = [(8, 32, 8, 4, 32768, 128, True, 6, S) for S in (0, 32, 64)] + \
        [(8, 32, 8, 1, 32768, 128, False, 6, 0)]


def _time(fn, iters, warmup, warm_ms=200.0):
    """Median launch time after `warmup` launches and at least `warm_ms` of
    back-to-back launches of the same call (the clocks settle only after
    ~50 ms of sustained work)."""
    st = torch.cuda.current_stream()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(max(warmup, 1)):
            fn()
        n += max(warmup, 1)
        torch.cuda.synchronize()
    ev = []
    for _ in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        fn()
        b.record(st)
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in ev)
    return ms[len(ms) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    args = ap.parse_args()
    torch.manual_seed(0)
    for name, B, H, N, d, causal, sc in FWD:
        q = (torch.randn(B, H, N, d, device="cuda") * sc).to(torch.bfloat16)
        k = (torch.randn(B, H, N, d, device="cuda") * sc).to(torch.bfloat16)
        v = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, device="cuda", dtype=torch.float32)
        ms = _time(lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse), args.iters, args.warmup)
        flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
        print(json.dumps({"workload": name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                          "kernel": fa.fa_fwd_kernel_name(d, int(causal), N, N), "ms": round(ms, 4),
                          "tflops": round(flop / ms / 1e9, 1),
                          "pct_of_2500": round(100 * flop / ms / 1e9 / 2500, 1)}), flush=True)
        del q, k, v, o, lse
    for name, B, H, N, d, causal, sc in FWD:
        q = (torch.randn(B, H, N, d, device="cuda") * sc).to(torch.bfloat16)
        k = (torch.randn(B, H, N, d, device="cuda") * sc).to(torch.bfloat16)
        v = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
        do = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
        o, lse = fa.fwd(q, k, v, causal=causal)
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N), dtype=torch.uint8, device="cuda")
        ms = _time(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=ws),
                   args.iters, args.warmup)
        flop = 2.5 * 4.0 * B * H * N * N * d / (2 if causal else 1)
        print(json.dumps({"workload": name + "_bwd", "B": B, "H": H, "N": N, "d": d,
                          "causal": causal,
                          "kernels": [fa.fa_bwd_kernel_name(d, int(causal), 0),
                                      fa.fa_bwd_kernel_name(d, int(causal), 1)],
                          "ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                          "pct_of_2500": round(100 * flop / ms / 1e9 / 2500, 1)}), flush=True)
        del q, k, v, do, o, lse, ws
    for name, B, H, N, d, causal, sc in FWD:
        # fp8 forward on random e4m3 codes of magnitude <= 2 (speed only).
        q8 = torch.randint(0, 0x41, (B, H, N, d), dtype=torch.uint8, device="cuda")
        k8 = torch.randint(0, 0x41, (B, H, N, d), dtype=torch.uint8, device="cuda")
        v8 = torch.randint(0, 0x41, (B, H, N, d), dtype=torch.uint8, device="cuda")
        o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, H, N, device="cuda", dtype=torch.float32)
        ms = _time(lambda: fa.fwd_fp8(q8, k8, v8, 1.0, 1.0, 1.0, causal=causal, out=o, lse=lse),
                   args.iters, args.warmup)
        flop = 4.0 * B * H * N * N * d / (2 if causal else 1)
        print(json.dumps({"workload": name + "_fp8", "B": B, "H": H, "N": N, "d": d,
                          "causal": causal, "kernel": fa.fa_fwd_fp8_kernel_name(d, int(causal)),
                          "ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                          "pct_of_5000": round(100 * flop / ms / 1e9 / 5000, 1)}), flush=True)
        del q8, k8, v8, o, lse
    for name, B, H, N, d in (("long", 1, 32, 16384, 128), ("train", 8, 16, 2048, 128),
                             ("sweep_d32", 2, 16, 4096, 32), ("sweep_d64", 2, 16, 4096, 64),
                             ("sweep_d256", 2, 16, 4096, 256)):
        # fp8 input step on one bf16 tensor: rotated (Q, K) and plain (V);
        # GB/s over 3 bytes per element (bf16 read, e4m3 code written).
        x = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
        signs = torch.where(torch.rand(d, device="cuda") < 0.5, -1, 1).to(torch.int8)
        codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
        dsc = torch.empty(1, dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_fp8_quantize_workspace_size(B * H * N, d), dtype=torch.uint8,
                         device="cuda")
        for rot in (True, False):
            ms = _time(lambda: fa.fp8_quantize(x, signs if rot else None, codes, dsc, ws),
                       args.iters, args.warmup)
            nbytes = 3 * x.numel()
            print(json.dumps({"workload": name + "_quantize", "B": B, "H": H, "N": N, "d": d,
                              "rotated": rot, "kernels": [fa.fa_fp8_quantize_kernel_name(d, 0),
                                                          fa.fa_fp8_quantize_kernel_name(d, 1)],
                              "ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                              "pct_of_8000": round(100 * nbytes / ms / 1e6 / 8000, 1)}),
                  flush=True)
        del x, codes, ws
    for B, Hq, Hkv, Nk, d, S in DECODE:
        q = torch.randn(B, Hq, d, device="cuda").to(torch.bfloat16)
        kc = torch.randn(B, Hkv, Nk, d, device="cuda").to(torch.bfloat16)
        vc = torch.randn(B, Hkv, Nk, d, device="cuda").to(torch.bfloat16)
        splits = S or fa.fa_decode_num_splits(B, Hq, Hkv, Nk, d)
        ws = torch.empty(fa.fa_decode_workspace_size(B, Hq, d, splits), dtype=torch.uint8,
                         device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, device="cuda", dtype=torch.float32)
        ms = _time(lambda: fa.decode(q, kc, vc, num_splits=splits, out=o, lse=lse, workspace=ws),
                   args.iters, args.warmup)
        nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * Hq * d * 2 + 4 * B * Hq
        print(json.dumps({"workload": "decode", "B": B, "Hq": Hq, "Hkv": Hkv, "Nk": Nk, "d": d,
                          "splits": splits, "kernels": [fa.fa_decode_kernel_name(d, Hq // Hkv, 0),
                                                        fa.fa_decode_kernel_name(d, Hq // Hkv, 1)],
                          "ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                          "pct_of_8000": round(100 * nbytes / ms / 1e6 / 8000, 1)}), flush=True)
        del q, kc, vc, ws, o, lse
    import numpy as np
    for B, Hq, Hkv, Nq, Nk, d, causal, seed, S in SERVE:
        # Per-sequence lengths as in the serving workload: uniform in 1024..Nk.
        lens = np.random.default_rng(seed + 1).integers(1024, Nk + 1, size=B).astype(np.int32)
        q = torch.randn(B, Hq, Nq, d, device="cuda").to(torch.bfloat16)
        kc = torch.randn(B, Hkv, Nk, d, device="cuda").to(torch.bfloat16)
        vc = torch.randn(B, Hkv, Nk, d, device="cuda").to(torch.bfloat16)
        sl = torch.from_numpy(lens).to("cuda")
        splits = S or fa.fa_decode_serve_num_splits(B, Hq, Hkv, Nq, Nk, d)
        ws = torch.empty(fa.fa_decode_serve_workspace_size(B, Hq, Nq, d, splits),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, Nq, device="cuda", dtype=torch.float32)
        ms = _time(lambda: fa.decode_serve(q, kc, vc, sl, causal=causal, num_splits=splits,
                                           out=o, lse=lse, workspace=ws), args.iters, args.warmup)
        nbytes = 2 * Hkv * int(lens.sum()) * d * 2 + 2 * B * Hq * Nq * d * 2 + 4 * B * Hq * Nq
        print(json.dumps({"workload": "serve", "B": B, "Hq": Hq, "Hkv": Hkv, "Nq": Nq, "Nk": Nk,
                          "d": d, "causal": causal, "mean_len": float(lens.mean()),
                          "splits": splits,
                          "kernels": [fa.fa_decode_serve_kernel_name(d, Hq // Hkv, Nq, 0),
                                      fa.fa_decode_serve_kernel_name(d, Hq // Hkv, Nq, 1)],
                          "ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                          "pct_of_8000": round(100 * nbytes / ms / 1e6 / 8000, 1)}), flush=True)
        del q, kc, vc, ws, o, lse, sl


if __name__ == "__main__":
    main()
