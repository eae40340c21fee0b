"""Helpers for the GPU parity tests: device marshalling and the parity bar.

The bar (float inputs rounded to bf16, compared against the float64 oracle):
  O   max-abs error <= 1.5e-2 and mean-abs error <= 2e-3
  LSE max-abs error <= 1e-3
Next to the primary error the report prints the error against the oracle
rounded to bf16 (the output format's own rounding) and the count of outputs
with |O| >= 4, where one bf16 half-ulp (2^-6) already exceeds 1.5e-2.
"""

from __future__ import annotations

import sys

import numpy as np

from datagen import bf16_bits_from_f32, f64_from_bf16_bits

O_MAX_ABS = 1.5e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def dev_bf16(bits):
    """uint16 bf16 bit patterns -> contiguous torch.bfloat16 tensor on cuda:0."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0").contiguous()


def host_f64(t):
    """Device tensor (bf16 or fp32) -> float64 numpy array (exact widening)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def report(tag, o, lse, o_ref, lse_ref):
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o - o_ref)
    e_max = float(err.max()) if err.size else 0.0
    e_mean = float(err.mean()) if err.size else 0.0
    e_lse = float(np.abs(np.asarray(lse, dtype=np.float64) - lse_ref).max()) if np.size(lse) else 0.0
    o_ref_bf = f64_from_bf16_bits(bf16_bits_from_f32(o_ref.astype(np.float32)))
    e_bf = float(np.abs(o - o_ref_bf).max()) if err.size else 0.0
    big = int((np.abs(o_ref) >= 4).sum())
    finite = bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse)))
    print(f"[parity] {tag}: O max {e_max:.3e} mean {e_mean:.3e} | vs bf16(oracle) "
          f"max {e_bf:.3e} | LSE max {e_lse:.3e} | |O_ref|>=4: {big} | finite {finite}",
          flush=True)
    return dict(o_max=e_max, o_mean=e_mean, lse_max=e_lse, o_max_bf16=e_bf, big=big,
                finite=finite)


def assert_parity(tag, o, lse, o_ref, lse_ref):
    r = report(tag, o, lse, o_ref, lse_ref)
    assert r["finite"], f"{tag}: non-finite output"
    assert r["o_max"] <= O_MAX_ABS, f"{tag}: O max-abs {r['o_max']:.3e}"
    assert r["o_mean"] <= O_MEAN_ABS, f"{tag}: O mean-abs {r['o_mean']:.3e}"
    assert r["lse_max"] <= LSE_MAX_ABS, f"{tag}: LSE max-abs {r['lse_max']:.3e}"
    return r


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


# Gradients.  Each element of dQ, dK, dV is a sum over keys or query rows of
# products whose bf16 operands (P, dS) carry independent rounding of relative
# size <= 2^-9, plus the bf16 rounding of the result and of the forward
# output O that Delta = rowsum(dO * O) is computed from.  Those roundings give
# a relative Frobenius error of a few times 2^-9 / sqrt(3) ~ 1e-3; the bar
# allows about 5 * 2^-9:
GRAD_REL_FRO = 1e-2      # ||G - G_ref||_F / ||G_ref||_F
GRAD_MAX_REL = 3e-2      # max |G - G_ref| / max |G_ref|


def report_grad(tag, name, g, g_ref):
    g = np.asarray(g, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    diff = g - g_ref
    ref_fro = float(np.sqrt((g_ref ** 2).sum()))
    ref_max = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    rel_fro = float(np.sqrt((diff ** 2).sum())) / ref_fro if ref_fro > 0 else float(np.abs(diff).max())
    max_rel = float(np.abs(diff).max()) / ref_max if ref_max > 0 else float(np.abs(diff).max())
    finite = bool(np.all(np.isfinite(g)))
    print(f"[parity] {tag} d{name}: rel-Frobenius {rel_fro:.3e} | max/max|ref| {max_rel:.3e} "
          f"| max|ref| {ref_max:.3e} | finite {finite}", flush=True)
    return dict(rel_fro=rel_fro, max_rel=max_rel, finite=finite)


def assert_grad_parity(tag, grads, refs):
    """grads, refs: dicts name -> array (dQ, dK, dV)."""
    out = {}
    for name in refs:
        r = report_grad(tag, name, grads[name], refs[name])
        assert r["finite"], f"{tag} d{name}: non-finite"
        assert r["rel_fro"] <= GRAD_REL_FRO, f"{tag} d{name}: rel-Frobenius {r['rel_fro']:.3e}"
        assert r["max_rel"] <= GRAD_MAX_REL, f"{tag} d{name}: max rel {r['max_rel']:.3e}"
        out[name] = r
    return out
