"""Shared helpers of the GPU parity tests (inputs, oracle plumbing)."""
import numpy as np
import pytest
import torch

import synth
from oracle import rope as orope


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import scaled_rope_tiled_amd as srt    # fails loudly if the library is missing
    return srt


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact host fp64 copy (bf16 and fp32 upcast exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_freq(rp: synth.Rope, D: int):
    return orope.inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)


def device_table(srt, rp: synth.Rope, D: int, npos: int):
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    return srt.rope_cos_sin(th, D, ms, npos, "cuda"), ms


def qkv(B, Hq, Hkv, Nq, Nk, D, dtype, seed, device="cuda"):
    q = synth.randn((B, Hq, Nq, D), dtype, seed, synth.Q_ID, device)
    k = synth.randn((B, Hkv, Nk, D), dtype, seed, synth.K_ID, device)
    v = synth.randn((B, Hkv, Nk, D), dtype, seed, synth.V_ID, device)
    return q, k, v


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_ninf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_ninf, 0.0, a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0
