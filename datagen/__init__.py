"""Seeded synthetic inputs shared by the oracle-side checks and the HIP path.

This module holds no attention arithmetic.  It only draws Gaussian samples,
rounds them to bfloat16 and names the workload shapes, so that both sides of a
parity test consume the exact same bit patterns.

Recipe (the pages name no dataset; every workload is synthetic):
  * ``numpy.random.default_rng(seed)`` (PCG64);
  * ``standard_normal(shape, dtype=float32)`` drawn in the order q, k, v
    (and, for the backward pass, the output gradient dO after them, so q, k
    and v equal the forward inputs of the same workload);
  * optionally multiplied by ``input_scale`` in float32 (the head-dim sweep
    scales by 1/sqrt(d) before rounding);
  * rounded to bfloat16 by round-to-nearest-even on the float32 bit pattern.

Tensors are laid out ``[B][H][N][d]`` with d fastest.  Decode queries are
``[B][Hq][d]`` (one query row per sequence).
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f64_from_bf16_bits",
    "f32_from_bf16_bits",
    "gaussian_bf16",
    "AttnConfig",
    "CONFIGS",
    "fwd_config",
    "decode_config",
    "make_fwd_inputs",
    "make_decode_inputs",
    "make_bwd_inputs",
    "make_serve_inputs",
    "fp8_e4m3_bits",
    "f64_from_fp8_e4m3_bits",
    "quantize_fp8_e4m3",
    "make_fp8_fwd_inputs",
    "serve_config",
    "row_subset",
]


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs are finite Gaussian
    samples, so NaN handling is not needed; infinities round to themselves.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_from_bf16_bits(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return f32_from_bf16_bits(bits).astype(np.float64)


def gaussian_bf16(seed: int, shapes, input_scale: float = 1.0):
    """Draw one bf16 tensor per shape from N(0,1), in order, from one generator."""
    rng = np.random.default_rng(seed)
    out = []
    s32 = np.float32(input_scale)
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if input_scale != 1.0:
            x = (x * s32).astype(np.float32)
        out.append(bf16_bits_from_f32(x))
    return out


@dataclass(frozen=True)
class AttnConfig:
    """One synthetic workload.  ``kind`` is "fwd", "decode" or "serve"."""

    name: str
    kind: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    input_scale: float = 1.0
    splits: tuple = field(default_factory=tuple)
    min_len: int = 1            # serving decode: shortest per-sequence cache

    @property
    def scale(self) -> float:
        """Softmax scale: 1/sqrt(d) for every workload."""
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic flop: 4*B*Hq*Nq*Nk*d, halved when causal (Nq == Nk)."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f / 2.0 if self.causal else f


def fwd_config(name, B, H, N, d, causal, seed, input_scale=1.0, Hkv=None, Nk=None):
    return AttnConfig(name, "fwd", B, H, Hkv or H, N, Nk or N, d, causal, seed,
                      input_scale)


def decode_config(name, B, Hq, Hkv, Nk, d, seed, splits=()):
    return AttnConfig(name, "decode", B, Hq, Hkv, 1, Nk, d, False, seed, 1.0,
                      tuple(splits))


def serve_config(name, B, Hq, Hkv, Nq, Nk, d, causal, seed, min_len=1):
    """Serving-shaped decode: Nq query rows per sequence, cache capacity Nk,
    per-sequence lengths drawn uniformly from min_len..Nk."""
    return AttnConfig(name, "serve", B, Hq, Hkv, Nq, Nk, d, causal, seed, 1.0, (),
                      min_len)


# The five workloads: a tiny non-causal case, a training-shape prefill (both
# mask modes), a long-context causal prefill, a head-dim sweep and a GQA
# split-KV decode over a 32k-token cache.
CONFIGS = {
    "tiny": fwd_config("tiny", 1, 2, 256, 64, False, seed=1),
    "train_nc": fwd_config("train_nc", 8, 16, 2048, 128, False, seed=2),
    "train_c": fwd_config("train_c", 8, 16, 2048, 128, True, seed=2),
    "long": fwd_config("long", 1, 32, 16384, 128, True, seed=3),
    "sweep_d32": fwd_config("sweep_d32", 2, 16, 4096, 32, True, seed=72,
                            input_scale=1 / math.sqrt(32)),
    "sweep_d64": fwd_config("sweep_d64", 2, 16, 4096, 64, True, seed=104,
                            input_scale=1 / math.sqrt(64)),
    "sweep_d128": fwd_config("sweep_d128", 2, 16, 4096, 128, True, seed=168,
                             input_scale=1 / math.sqrt(128)),
    "sweep_d256": fwd_config("sweep_d256", 2, 16, 4096, 256, True, seed=296,
                             input_scale=1 / math.sqrt(256)),
    "decode": decode_config("decode", 8, 32, 8, 32768, 128, seed=5,
                            splits=(16, 32, 64)),
    # Serving-shaped decode (a NEXT row): 4 new tokens per sequence, causal
    # among themselves, over per-sequence caches of 1k..32k tokens.
    "serve": serve_config("serve", 8, 32, 8, 4, 32768, 128, True, seed=6, min_len=1024),
}


def make_fwd_inputs(cfg: AttnConfig):
    """bf16 bits for q [B][Hq][Nq][d], k and v [B][Hkv][Nk][d]."""
    return gaussian_bf16(
        cfg.seed,
        [(cfg.B, cfg.Hq, cfg.Nq, cfg.d), (cfg.B, cfg.Hkv, cfg.Nk, cfg.d),
         (cfg.B, cfg.Hkv, cfg.Nk, cfg.d)],
        cfg.input_scale)


def make_bwd_inputs(cfg: AttnConfig):
    """bf16 bits for q, k, v (as make_fwd_inputs) and dO [B][Hq][Nq][d]."""
    return gaussian_bf16(
        cfg.seed,
        [(cfg.B, cfg.Hq, cfg.Nq, cfg.d), (cfg.B, cfg.Hkv, cfg.Nk, cfg.d),
         (cfg.B, cfg.Hkv, cfg.Nk, cfg.d), (cfg.B, cfg.Hq, cfg.Nq, cfg.d)],
        cfg.input_scale)


def make_serve_inputs(cfg: AttnConfig):
    """bf16 bits for q [B][Hq][Nq][d], k_cache and v_cache [B][Hkv][Nk][d], and
    int32 lengths [B] drawn from default_rng(seed + 1) in min_len..Nk."""
    q, k, v = gaussian_bf16(
        cfg.seed,
        [(cfg.B, cfg.Hq, cfg.Nq, cfg.d), (cfg.B, cfg.Hkv, cfg.Nk, cfg.d),
         (cfg.B, cfg.Hkv, cfg.Nk, cfg.d)],
        cfg.input_scale)
    lens = np.random.default_rng(cfg.seed + 1).integers(cfg.min_len, cfg.Nk + 1, size=cfg.B)
    return q, k, v, lens.astype(np.int32)


# OCP fp8 e4m3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
# bits; codes 0x7F and 0xFF are NaN, there is no infinity, 448 is the largest
# finite value.  Input preparation only: the encoder rounds to nearest, ties
# to the even code, and saturates at +-448.
def _e4m3_positive_values():
    codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))


_E4M3_POS = _e4m3_positive_values()


def fp8_e4m3_bits(x) -> np.ndarray:
    """float array -> uint8 e4m3 codes (round to nearest even, saturate)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), _E4M3_POS[-1])
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x) & (code != 0), code | 0x80, code).astype(np.uint8)


def f64_from_fp8_e4m3_bits(bits) -> np.ndarray:
    """uint8 e4m3 codes (no NaN codes) -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint8)
    v = _E4M3_POS[(bits & 0x7F).astype(np.int64)]
    return np.where(bits & 0x80, -v, v)


def quantize_fp8_e4m3(x):
    """Per-tensor quantisation: descale = max|x| / 448, bytes = e4m3(x / descale).
    Returns (uint8 codes, descale as a Python float)."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.abs(x).max()) if x.size else 0.0
    descale = amax / 448.0 if amax > 0 else 1.0
    return fp8_e4m3_bits(x / descale), descale


def make_fp8_fwd_inputs(cfg: AttnConfig):
    """The forward inputs of a workload (the same bf16 draws) quantised per
    tensor to fp8 e4m3: ((q8, k8, v8), (q_descale, k_descale, v_descale))."""
    out, scales = [], []
    for bits in make_fwd_inputs(cfg):
        codes, ds = quantize_fp8_e4m3(f64_from_bf16_bits(bits))
        out.append(codes)
        scales.append(ds)
    return tuple(out), tuple(scales)


def drifting_bf16(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, slope: float,
                  noise: float = 0.1):
    """Inputs whose scores drift along the key axis: q = 0.5 + noise*z and
    k_j = slope*j/(0.5*sqrt(d)*log2 e) + noise*z per element, v ~ N(0,1), all
    rounded to bf16.  With the softmax scale 1/sqrt(d) the score of key j in
    base-2 units is then about slope*j (negative slope: falling scores), so a
    row's largest score keeps moving as its keys are scanned."""
    rng = np.random.default_rng(seed)
    q = 0.5 + noise * rng.standard_normal((B, Hq, N, d))
    t = slope * np.arange(N) / (0.5 * np.sqrt(d) * np.log2(np.e))
    k = t[None, None, :, None] + noise * rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    return [bf16_bits_from_f32(x.astype(np.float32)) for x in (q, k, v)]


def random_signs(seed: int, d: int) -> np.ndarray:
    """The random ±1 signs of the incoherent-processing rotation, int8 [d]
    (drawn here and passed to both sides as an input)."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)


def outlier_bf16(seed: int, shape, channels=(3, 77), gain: float = 20.0):
    """N(0,1) bf16 bits with a few head-dim channels scaled by `gain`: the
    outlier pattern that incoherent processing is meant for."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    for c in channels:
        if c < shape[-1]:
            x[..., c] *= np.float32(gain)
    return bf16_bits_from_f32(x)


def make_decode_inputs(cfg: AttnConfig):
    """bf16 bits for q [B][Hq][d], k_cache and v_cache [B][Hkv][Nk][d]."""
    return gaussian_bf16(
        cfg.seed,
        [(cfg.B, cfg.Hq, cfg.d), (cfg.B, cfg.Hkv, cfg.Nk, cfg.d),
         (cfg.B, cfg.Hkv, cfg.Nk, cfg.d)],
        cfg.input_scale)


def row_subset(N: int, count: int, head: int) -> np.ndarray:
    """Seeded sorted subset of query rows checked for one head of a long case."""
    rng = np.random.default_rng(1000 + head)
    return np.sort(rng.choice(N, size=min(count, N), replace=False))
