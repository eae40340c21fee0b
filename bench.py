"""Benchmark of the exact-attention hot path on one MI355X.

One step = one causal prefill forward over the long-context workload
(B=1, H=32, N=16384, d=128) followed by one split-KV decode over the decode
workload (B=8, Hq=32, Hkv=8, Nk=32768, d=128), both through the C ABI on the
same stream, inputs already resident in HBM.  Prints one JSON line:

  value     prefill TFLOP/s, flop = 4*B*H*N*N*d / 2 (causal), over the median
            forward launch duration (HIP events on the launch stream around
            each launch); the mean is reported next to it
  decode    split-KV decode GB/s, bytes = K + V cache read once + q + O + LSE
  roofline  the forward kernel against the dense bf16 MFMA peak (2.5 PFLOP/s);
            decode carries its own roofline against 8 TB/s HBM
  cpu_baseline  the float64 oracle on a bounded sample of the same workload,
            timed on the host cores (rank 0, one GPU)
  fp8       after the timed steps: fa_fwd_fp8 on the same prefill quantised
            per tensor to fp8 e4m3, timed per call; its own roofline against
            the 5 PFLOP/s dense fp8 MFMA peak
  bwd       after the timed steps: the backward pass (fa_bwd) of the same
            prefill, fed the last step's O and LSE and a seeded dO, timed
            over its own launches; TFLOP/s counts the algorithmic 5 products
            of the backward (10*B*H*N*N*d / 2 flop, causal), not the 7 the
            recomputation performs
  workloads after the timed steps: the forward on the training shape
            (B=8 H=16 N=2048 d=128, causal and not) and on the head-dim sweep
            (B=2 H=16 N=4096 causal, d = 32, 64, 128, 256), each with its
            kernel name, median TFLOP/s and roofline: the MFMA peak for
            d >= 128, the VALU softmax bound (see alu_peak_tflops) for d <= 64
  sclk      shader clock samples (amd-smi) taken during a sustained run of
            the prefill after the timed steps; amd-smi's reading lags the
            load (it can still show the idle clock in the first second), so
            only samples from the second half of a 3 s run count

Every timed series is preceded by a warm-up of at least 200 ms of the same
launches (and at least --warmup steps): the clock ramps up over the first
tens of milliseconds of sustained work.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bwd]
                      [--no-fp8] [--no-workloads] [--no-sclk]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import datagen  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
METRIC = "fused attn fwd TFLOP/s (% bf16 MFMA peak); split-KV decode HBM GB/s"
WARM_MS = 200.0             # minimum warm-up of every timed series

# VALU bound of the softmax (head dims whose MFMA work is too small to hide
# it).  Per (query, key) pair the online softmax needs at least one exponential
# and three other wave64 VALU instructions per 64 pairs: the FMA that applies
# scale*log2(e) and subtracts the running maximum, the add into the row sum,
# half a v_max3 for the row maximum and half a v_cvt_pk_bf16_f32 for the bf16
# probabilities.  A wave64 fp32 VALU instruction occupies a 16-lane SIMD for 4
# cycles; v_exp_f32 was measured on MI355X to issue every 9.5 cycles (8 waves
# per SIMD, independent chains).  So one SIMD turns at most 64 pairs into
# probabilities every 9.5 + 3*4 = 21.5 cycles; 1024 SIMDs at 2.4 GHz give
# 7.3e12 pairs/s, i.e. 4d flop per pair -> 935 TFLOP/s at d = 32, 1871 at
# d = 64 (and 3741 at d = 128, above the MFMA peak, which then binds).
EXP_ISSUE_CYCLES = 9.5
VALU_ISSUE_CYCLES = 4.0
MIN_VALU_PER_64_PAIRS = 3.0
SIMDS = 1024
CLOCK_HZ = 2.4e9


def alu_peak_tflops(d):
    pairs_per_s = SIMDS * CLOCK_HZ * 64 / (EXP_ISSUE_CYCLES + MIN_VALU_PER_64_PAIRS * VALU_ISSUE_CYCLES)
    return 4 * d * pairs_per_s / 1e12


def roofline_for(d, tflops):
    """The binding roofline of a bf16 forward at head dim d."""
    alu = alu_peak_tflops(d)
    if alu < PEAK_BF16_TFLOPS:
        return {"bound": "alu", "achieved": round(tflops, 2), "peak": round(alu, 1),
                "unit": "TFLOP/s", "frac": round(tflops / alu, 4),
                "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    return {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}


def warm(calls, steps):
    """Run the launch sequence `calls` at least `steps` times and for at least
    WARM_MS of wall time, then synchronise."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < steps or (time.perf_counter() - t0) * 1e3 < WARM_MS:
        calls()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_launches(call, stream, steps, warmup=10):
    """Per-launch durations (ms) of `call`, from HIP events recorded on the
    launch stream around each launch, after a time-based warm-up."""
    import torch
    warm(call, warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in evs]


def stats(ms):
    return {"ms": round(float(np.median(ms)), 5), "ms_mean": round(float(np.mean(ms)), 5),
            "ms_min": round(float(np.min(ms)), 5)}


def _dev(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0").contiguous()


def _traffic(kernel, source_files):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when no summary exists or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for s in source_files:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline_fwd(cfg, qb, kb, vb, rows_per_head=4096, heads=32):
    """Oracle on `heads` heads x `rows_per_head` seeded rows of the prefill
    workload; throughput counts the algorithmic (causal) flop of those rows."""
    import oracle
    q = datagen.f64_from_bf16_bits(qb[:, :heads])
    k = datagen.f64_from_bf16_bits(kb[:, :heads])
    v = datagen.f64_from_bf16_bits(vb[:, :heads])
    rows = {h: datagen.row_subset(cfg.Nq, rows_per_head, h) for h in range(heads)}
    t0 = time.perf_counter()
    oracle.attention_ref(q, k, v, cfg.scale, cfg.causal, rows=rows)
    dt = time.perf_counter() - t0
    pairs = sum(int((r + 1).sum()) for r in rows.values()) if cfg.causal else \
        heads * rows_per_head * cfg.Nk
    flop = 4.0 * cfg.d * pairs * cfg.B
    return dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=_blas_threads(),
                kind="oracle", seconds=round(dt, 3),
                sample=f"float64 oracle, {heads} of {cfg.Hq} heads x {rows_per_head} seeded "
                       f"query rows of the causal B={cfg.B} H={cfg.Hq} N={cfg.Nq} d={cfg.d} "
                       f"prefill, scores materialised then masked")


def cpu_baseline_decode(cfg, qb, kb, vb, batches=8):
    import oracle
    q = datagen.f64_from_bf16_bits(qb[:batches])
    k = datagen.f64_from_bf16_bits(kb[:batches])
    v = datagen.f64_from_bf16_bits(vb[:batches])
    t0 = time.perf_counter()
    oracle.attention_ref(q[:, :, None, :], k, v, cfg.scale, False)
    dt = time.perf_counter() - t0
    nbytes = 2 * batches * cfg.Hkv * cfg.Nk * cfg.d * 2
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=_blas_threads(), kind="oracle",
                seconds=round(dt, 3),
                sample=f"float64 oracle, {batches} of {cfg.B} sequences of the decode workload")


def cpu_baseline_bwd(cfg, qb, kb, vb, dob, head=0):
    """Oracle gradients (dQ of every row, dK and dV of every key) of one head
    of the prefill workload; throughput counts the algorithmic backward flop
    of that head."""
    import oracle
    sel = lambda bits: datagen.f64_from_bf16_bits(bits[0, head])
    t0 = time.perf_counter()
    oracle.attention_bwd_head_ref(sel(qb), sel(kb), sel(vb), sel(dob), cfg.scale, cfg.causal)
    dt = time.perf_counter() - t0
    flop = 10.0 * cfg.Nq * cfg.Nk * cfg.d / (2 if cfg.causal else 1)
    return dict(value=flop / dt / 1e12, unit="TFLOP/s", cores=_blas_threads(), kind="oracle",
                seconds=round(dt, 3),
                sample=f"float64 oracle gradients of head {head} of the causal B={cfg.B} "
                       f"H={cfg.Hq} N={cfg.Nq} d={cfg.d} prefill (all rows and keys), "
                       f"score, probability and gradient blocks materialised")


def _blas_threads():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        if os.environ.get(var):
            try:
                return int(os.environ[var])
            except ValueError:
                pass
    return os.cpu_count()


def fp8_leg(fa, cfg, stream, steps, warmup=20):
    """fa_fwd_fp8 on the prefill quantised per tensor to fp8 e4m3 (the same
    draws as the bf16 leg), timed per call with HIP events."""
    import torch
    (q8, k8, v8), sc = datagen.make_fp8_fwd_inputs(cfg)
    dq, dk, dv = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0") for x in (q8, k8, v8))
    o8 = torch.empty((cfg.B, cfg.Hq, cfg.Nq, cfg.d), dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty((cfg.B, cfg.Hq, cfg.Nq), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream

    def call():
        rc = fa.fa_fwd_fp8(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), o8.data_ptr(), l8.data_ptr(),
                           cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.scale, sc[0], sc[1],
                           sc[2], int(cfg.causal), sp)
        if rc:
            raise fa.FAError(rc, "fa_fwd_fp8")

    ms = time_launches(call, stream, steps, warmup)
    f_ms = float(np.median(ms))
    tf = cfg.flops() / (f_ms * 1e-3) / 1e12
    srcs = ["exact_attention_103_amd/csrc/fa_fwd_fp8.hip", "exact_attention_103_amd/csrc/fa_internal.h"]
    kname = fa.fa_fwd_fp8_kernel_name(cfg.d, int(cfg.causal))
    return {"value": round(tf, 2), "unit": "TFLOP/s", **stats(ms),
            "dtype": "fp8 e4m3 (per-tensor scales), fp32 accumulate",
            "kernel": kname,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                         "traffic": _traffic(kname, srcs)},
            "quantize": quantize_leg(fa, cfg, stream, steps)}


def quantize_leg(fa, cfg, stream, steps, warmup=20):
    """fa_fp8_quantize of the prefill's bf16 Q (rotated), K (rotated) and V
    (not rotated), timed per call; GB/s over the algorithmic 3 bytes per
    element (read bf16, write the e4m3 code)."""
    import torch
    qb, kb, vb = datagen.make_fwd_inputs(cfg)
    xs = [_dev(x) for x in (qb, kb, vb)]
    signs = torch.from_numpy(datagen.random_signs(cfg.seed, cfg.d)).to("cuda:0")
    rows = [x.numel() // cfg.d for x in xs]
    codes = [torch.empty(x.shape, dtype=torch.uint8, device="cuda") for x in xs]
    ds = torch.empty(3, dtype=torch.float32, device="cuda")
    wss = [torch.empty(fa.fa_fp8_quantize_workspace_size(r, cfg.d), dtype=torch.uint8,
                       device="cuda") for r in rows]
    sp = stream.cuda_stream

    def call(i):
        rc = fa.fa_fp8_quantize(xs[i].data_ptr(), codes[i].data_ptr(), ds[i:].data_ptr(),
                                signs.data_ptr() if i < 2 else None, rows[i], cfg.d,
                                wss[i].data_ptr(), wss[i].numel() * wss[i].element_size(), sp)
        if rc:
            raise fa.FAError(rc, "fa_fp8_quantize")

    warm(lambda: [call(i) for i in range(3)], warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        e[0].record(stream)
        call(0)
        e[1].record(stream)
        call(1)
        call(2)
    torch.cuda.synchronize()
    ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    nbytes = 3 * xs[0].numel()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"tensor": f"Q [{cfg.B}][{cfg.Hq}][{cfg.Nq}][{cfg.d}] bf16, rotated",
            "ms": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
            "kernels": [fa.fa_fp8_quantize_kernel_name(cfg.d, 0),
                        fa.fa_fp8_quantize_kernel_name(cfg.d, 1)],
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic(f"fa_fp8_quantize_d{cfg.d}",
                                             ["exact_attention_103_amd/csrc/fa_fp8_quant.hip",
                                              "exact_attention_103_amd/csrc/fa_internal.h"])}}


def bwd_leg(fa, cfg, q, k, v, o, lse, stream, steps, warmup=10):
    """Backward of the prefill: fa_bwd fed the forward's O and LSE and a
    seeded dO, timed per call with HIP events on the launch stream."""
    import torch
    _, _, _, dob = datagen.make_bwd_inputs(cfg)
    do = _dev(dob)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(cfg.B, cfg.Hq, cfg.Nq), dtype=torch.uint8,
                     device="cuda")
    sp = stream.cuda_stream

    def call():
        rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cfg.B,
                       cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.scale, int(cfg.causal),
                       ws.data_ptr(), ws.numel() * ws.element_size(), sp)
        if rc:
            raise fa.FAError(rc, "fa_bwd")

    ms = time_launches(call, stream, steps, warmup)
    b_ms = float(np.median(ms))
    flop = 2.5 * cfg.flops()
    tf = flop / (b_ms * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", **stats(ms), "flop": flop,
            "kernels": [fa.fa_bwd_kernel_name(cfg.d, int(cfg.causal), 0),
                        fa.fa_bwd_kernel_name(cfg.d, int(cfg.causal), 1)],
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": _bwd_traffic(cfg)}}


def _bwd_traffic(cfg):
    """HBM bytes of one fa_bwd call (both kernels) from the committed counter
    summaries, or None (missing, or the sources changed since)."""
    srcs = ["exact_attention_103_amd/csrc/fa_bwd.hip", "exact_attention_103_amd/csrc/fa_internal.h"]
    tag = "causal" if cfg.causal else "nomask"
    parts = [_traffic(f"fa_bwd_{k}_d{cfg.d}_{tag}", srcs) for k in ("dq", "dkdv")]
    return None if any(x is None for x in parts) else sum(parts)


def workload_legs(fa, stream, steps, names=("train_nc", "train_c", "sweep_d32", "sweep_d64",
                                             "sweep_d128", "sweep_d256")):
    """The forward on the training shape and the head-dim sweep, one timed
    series each (median of per-launch HIP-event durations)."""
    import torch
    out = []
    sp = stream.cuda_stream
    for name in names:
        cfg = datagen.CONFIGS[name]
        q, k, v = (_dev(x) for x in datagen.make_fwd_inputs(cfg))
        o = torch.empty_like(q)
        lse = torch.empty((cfg.B, cfg.Hq, cfg.Nq), dtype=torch.float32, device="cuda")

        def call():
            rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.scale,
                           int(cfg.causal), sp)
            if rc:
                raise fa.FAError(rc, "fa_fwd")

        ms = time_launches(call, stream, steps)
        st = stats(ms)
        tf = cfg.flops() / (st["ms"] * 1e-3) / 1e12
        out.append({"workload": name, "B": cfg.B, "H": cfg.Hq, "N": cfg.Nq, "d": cfg.d,
                    "causal": cfg.causal, "input_scale": cfg.input_scale,
                    "kernel": fa.fa_fwd_kernel_name(cfg.d, int(cfg.causal), cfg.Nq, cfg.Nk),
                    "flop": cfg.flops(), **st, "value": round(tf, 2), "unit": "TFLOP/s",
                    "roofline": roofline_for(cfg.d, tf)})
        del q, k, v, o, lse
    return out


def _under_profiler():
    """True inside a rocprofv3 run (its tool library is preloaded)."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


def sample_sclk(call, seconds=3.0):
    """Shader clock (MHz) samples from amd-smi while `call` runs back to back
    for about `seconds`.  amd-smi's value lags the load, so only the samples
    taken in the second half of the run count.  Returns their median/min/max
    (and how many samples were dropped), or a note with the start of
    amd-smi's reply when no clock could be read from it."""
    import re
    import subprocess
    import threading
    import torch
    samples, raw, stop = [], [], threading.Event()
    cmd = ["amd-smi", "metric", "-g", "0", "-c", "--json"]

    def poll():
        while not stop.is_set():
            try:
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=5)
            except Exception as e:  # amd-smi missing or hung
                raw.append(repr(e))
                return
            text = r.stdout
            # the graphics clock block ("gfx_0" / "GFX_0"): first "clk" value in it
            m = re.search(r'"gfx_0"\s*:\s*\{.*?"clk"\s*:\s*\{\s*"value"\s*:\s*(\d+)', text,
                          re.S | re.I)
            if m:
                samples.append((time.perf_counter(), int(m.group(1))))
            elif not raw:
                raw.append((text or r.stderr)[:300])

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=10)
    late = [v for t, v in samples if t >= t0 + seconds / 2]
    if not late:
        return {"mhz_median": None, "note": "no clock parsed", "reply": raw[:1]}
    return {"mhz_median": float(np.median(late)), "mhz_min": min(late),
            "mhz_max": max(late), "samples": len(late),
            "samples_dropped_first_half": len(samples) - len(late), "source": " ".join(cmd)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)   # ~70 ms: the clocks ramp up first
    ap.add_argument("--splits", type=int, default=0, help="decode splits (0 = heuristic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward leg")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the training-shape and head-dim-sweep forward legs")
    ap.add_argument("--no-sclk", action="store_true", help="skip the shader clock samples")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="instead of the benchmark, run three plain device-to-device "
                         "copies of BYTES bytes (reference dispatches for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the kernels are single-GPU and this build has "
              "no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_103_amd as fa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.calibrate_copy:
        n = args.calibrate_copy
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 3}), flush=True)
        return

    fcfg = datagen.CONFIGS["long"]
    dcfg = datagen.CONFIGS["decode"]
    fq, fk, fv = datagen.make_fwd_inputs(fcfg)
    dq, dk, dv = datagen.make_decode_inputs(dcfg)
    q, k, v = _dev(fq), _dev(fk), _dev(fv)
    o = torch.empty_like(q)
    lse = torch.empty((fcfg.B, fcfg.Hq, fcfg.Nq), dtype=torch.float32, device="cuda")
    qd, kc, vc = _dev(dq), _dev(dk), _dev(dv)
    od = torch.empty_like(qd)
    lsed = torch.empty((dcfg.B, dcfg.Hq), dtype=torch.float32, device="cuda")
    S = args.splits or fa.fa_decode_num_splits(dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.Nk, dcfg.d)
    ws = torch.empty(fa.fa_decode_workspace_size(dcfg.B, dcfg.Hq, dcfg.d, S),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       fcfg.B, fcfg.Hq, fcfg.Hkv, fcfg.Nq, fcfg.Nk, fcfg.d, fcfg.scale,
                       int(fcfg.causal), sp)
        if rc:
            raise fa.FAError(rc, "fa_fwd")
        if ev is not None:
            ev[1].record(stream)
        rc = fa.fa_decode_splitkv(qd.data_ptr(), kc.data_ptr(), vc.data_ptr(), od.data_ptr(),
                                  lsed.data_ptr(), dcfg.B, dcfg.Hq, dcfg.Hkv, dcfg.Nk, dcfg.d,
                                  dcfg.scale, S, ws.data_ptr(), ws.numel() * ws.element_size(),
                                  sp)
        if rc:
            raise fa.FAError(rc, "fa_decode_splitkv")
        if ev is not None:
            ev[2].record(stream)

    warm_steps = warm(step, args.warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    f_ms = float(np.median(fwd_ms))
    d_ms = float(np.median(dec_ms))

    flop = fcfg.flops()
    tflops = flop / (f_ms * 1e-3) / 1e12
    dec_bytes = (2 * dcfg.B * dcfg.Hkv * dcfg.Nk * dcfg.d * 2 + 2 * dcfg.B * dcfg.Hq * dcfg.d * 2
                 + 4 * dcfg.B * dcfg.Hq)
    gbs = dec_bytes / (d_ms * 1e-3) / 1e9
    fwd_bytes = 4 * fcfg.B * fcfg.Hq * fcfg.Nq * fcfg.d * 2 + 4 * fcfg.B * fcfg.Hq * fcfg.Nq
    srcs = ["exact_attention_103_amd/csrc/fa_fwd.hip", "exact_attention_103_amd/csrc/fa_internal.h"]
    dsrcs = ["exact_attention_103_amd/csrc/fa_decode.hip", "exact_attention_103_amd/csrc/fa_internal.h"]

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) float32 rounded to bf16",
        "config": {
            "workload": "causal prefill B=1 H=32 N=16384 d=128 + split-KV decode B=8 Hq=32 "
                        "Hkv=8 Nk=32768 d=128",
            "fwd": {"B": fcfg.B, "H": fcfg.Hq, "N": fcfg.Nq, "d": fcfg.d, "causal": True,
                    "scale": fcfg.scale, "kernel": fa.fa_fwd_kernel_name(fcfg.d, 1, fcfg.Nq, fcfg.Nk),
                    "flop": flop, **stats(fwd_ms)},
            "decode": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "Nk": dcfg.Nk, "d": dcfg.d,
                       "splits": S,
                       "kernels": [fa.fa_decode_kernel_name(dcfg.d, dcfg.Hq // dcfg.Hkv, 0),
                                   fa.fa_decode_kernel_name(dcfg.d, dcfg.Hq // dcfg.Hkv, 1)],
                       "bytes": dec_bytes, **stats(dec_ms)},
            "parallelism": "1 GPU",
            "warmup_steps_run": warm_steps,
            "timing": "median of per-launch HIP-event durations on the launch stream",
        },
        "fwd_pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic("fa_fwd_d128_causal", srcs),
            "kernel": fa.fa_fwd_kernel_name(fcfg.d, 1, fcfg.Nq, fcfg.Nk),
            "algorithmic_bytes": fwd_bytes,
        },
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s", "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic("fa_decode_split_d128_g4", dsrcs)},
        },
        "cpu_baseline": None,
    }
    if not args.no_sclk and _under_profiler():
        # amd-smi would start inside the profiler's preloaded library and
        # replace itself with its interpreter after that library touched the
        # GPU; profiled runs take no clock samples.
        out["sclk"] = {"mhz_median": None, "note": "skipped under a profiler"}
    elif not args.no_sclk:
        def fwd_only():
            fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      fcfg.B, fcfg.Hq, fcfg.Hkv, fcfg.Nq, fcfg.Nk, fcfg.d, fcfg.scale,
                      int(fcfg.causal), sp)
        out["sclk"] = sample_sclk(fwd_only)
    if not args.no_workloads:
        out["workloads"] = workload_legs(fa, stream, args.steps)
    if not args.no_fp8:
        out["fp8"] = fp8_leg(fa, fcfg, stream, args.steps)
    if not args.no_bwd:
        out["bwd"] = bwd_leg(fa, fcfg, q, k, v, o, lse, stream, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_fwd(fcfg, fq, fk, fv)
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(dcfg, dq, dk, dv)
        if not args.no_bwd:
            _, _, _, fdo = datagen.make_bwd_inputs(fcfg)
            out["bwd"]["cpu_baseline"] = cpu_baseline_bwd(fcfg, fq, fk, fv, fdo)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
