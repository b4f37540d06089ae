"""GPU parity of the frequency-step variants vs the fp64 oracle: half-split
pairs (x_i, x_{i+D/2}) in every kernel that rotates, and tables built from the
Dynamic-NTK and per-pair-factor frequencies.

Bars as elsewhere: fp32 path 1e-4 max-abs, bf16 path 2e-2 max-abs."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import f64, max_abs, need_gpu, qkv
from oracle import attention as A
from oracle import rope as orope

pytestmark = pytest.mark.gpu

YARN_SMALL = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)


def _table(srt, D, npos, rp=YARN_SMALL):
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    oth, oms, _ = orope.inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    return srt.rope_cos_sin(th, D, ms, npos, "cuda"), oth, oms


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_apply_half(dtype, D):
    srt = need_gpu()
    B, H, N, pos0 = 2, 3, 301, 777
    x = synth.randn((B, H, N, D), dtype, 12, 0, "cuda")
    table, th, ms = _table(srt, D, pos0 + N)
    y = srt.rope_apply(x, table, pos0=pos0, pairing="half")
    ref = orope.rotate_half(f64(x), pos0 + np.arange(N), th, ms)
    got = f64(y)
    if dtype == torch.float32:
        assert max_abs(got, ref) <= 1e-5
    else:
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    # the interleaved kernel gives a different answer on the same input
    assert max_abs(f64(srt.rope_apply(x, table, pos0=pos0)), ref) > 1e-2


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("k_on_load", [True, False])
def test_prefill_f32_half(D, k_on_load):
    srt = need_gpu()
    q, k, v = qkv(1, 4, 2, 150, 150, D, torch.float32, 21)
    table, th, ms = _table(srt, D, 150)
    flags = srt.ROTATE_Q | srt.PAIR_HALF
    kin = k
    if k_on_load:
        flags |= srt.ROTATE_K
    else:
        kin = srt.rope_apply(k, table, pairing="half")
    o, l = srt.attn_prefill(q, kin, v, table=table, rope_flags=flags)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), theta=th, mscale=ms, pairing="half")
    assert max_abs(f64(o), ro) <= 1e-4 and max_abs(f64(l), rl) <= 1e-4


@pytest.mark.parametrize("k_on_load", [True, False])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_bf16_half(k_on_load, G):
    srt = need_gpu()
    D = 128
    q, k, v = qkv(1, 2 * G, 2, 200, 260, D, torch.bfloat16, 22)
    table, th, ms = _table(srt, D, 300)
    flags = srt.ROTATE_Q | srt.PAIR_HALF
    kin = k
    if k_on_load:
        flags |= srt.ROTATE_K
    else:
        kin = srt.rope_apply(k, table, pos0=30, pairing="half")
    o, l = srt.attn_prefill(q, kin, v, q_pos0=90, k_pos0=30, table=table, rope_flags=flags)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), q_pos0=90, k_pos0=30, theta=th,
                         mscale=ms, pairing="half")
    assert max_abs(f64(o), ro) <= 2e-2 and max_abs(f64(l), rl) <= 2e-2


def test_decode_half():
    srt = need_gpu()
    D, B, Hq, Hkv, Nk = 128, 3, 8, 2, 900
    q = synth.randn((B, Hq, D), torch.bfloat16, 23, synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 23, synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 23, synth.V_ID, "cuda")
    table, th, ms = _table(srt, D, Nk, synth.Rope(synth.PI, 10000.0, 16.0))
    kc = srt.rope_apply(k, table, pairing="half")
    lens = [900, 17, 450]
    o, l = srt.attn_decode_splitk(q, kc, v, num_splits=6, table=table, pairing="half",
                                  seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    kref = np.stack([orope.rotate_half(f64(k[b]), np.arange(Nk), th, ms) for b in range(B)])
    ro, rl = A.decode(f64(q), kref, f64(v), sm_scale=1 / math.sqrt(D), seq_lens=lens, theta=th, mscale=ms,
                      pairing="half")
    assert max_abs(f64(o), ro) <= 2e-2 and max_abs(f64(l), rl) <= 1e-2


@pytest.mark.parametrize("variant", ["dynamic_ntk", "factors"])
def test_prefill_with_variant_tables(variant):
    """Tables from the other frequency rules drive the bf16 kernel like any other."""
    srt = need_gpu()
    D, N = 128, 333
    if variant == "dynamic_ntk":
        th, _ = srt.rope_inv_freq_dynamic_ntk(10000.0, N, 64.0, D)
        oth = orope.inv_freq_dynamic_ntk(10000.0, N, 64.0, D)
    else:
        lam = 1.0 + np.linspace(0.0, 15.0, D // 2) ** 1.5 / 4.0
        th = srt.rope_inv_freq_factors(10000.0, lam, D)
        oth = orope.inv_freq_factors(10000.0, lam, D)
    table = srt.rope_cos_sin(th, D, 1.0, N, "cuda")
    q, k, v = qkv(1, 4, 1, N, N, D, torch.bfloat16, 24)
    o, l = srt.attn_prefill(q, k, v, table=table)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), theta=oth, mscale=1.0)
    assert max_abs(f64(o), ro) <= 2e-2 and max_abs(f64(l), rl) <= 2e-2
