"""GPU parity of the fp32 prefill kernel vs the fp64 oracle (bar: max-abs 1e-4 on O)."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import attention as A

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _run(srt, rp, B, Hq, Hkv, Nq, Nk, D, *, causal=True, q_pos0=0, k_pos0=0, seed=1, flags=None):
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, D, torch.float32, seed)
    npos = max(q_pos0 + Nq, k_pos0 + Nk)
    table, _ = device_table(srt, rp, D, npos)
    o, l = srt.attn_prefill(q, k, v, causal=causal, q_pos0=q_pos0, k_pos0=k_pos0, table=table, rope_flags=flags)
    th, ms, _ = oracle_freq(rp, D)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), causal=causal, q_pos0=q_pos0,
                         k_pos0=k_pos0, theta=th, mscale=ms)
    return f64(o), f64(l), ro, rl


def test_tiny_fp32_full_parity():
    """B=1, H=1, N=512, D=64, fp32, causal, plain RoPE base 1e4, scale 1/sqrt(D), seed 1."""
    srt = need_gpu()
    w = synth.WORKLOADS["tiny_fp32"]
    o, l, ro, rl = _run(srt, w.rope, w.B, w.Hq, w.Hkv, w.N, w.N, w.D, seed=w.seed)
    assert max_abs(o, ro) <= TOL
    assert max_abs(l, rl) <= TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_gqa_yarn(D, causal):
    srt = need_gpu()
    rp = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)
    o, l, ro, rl = _run(srt, rp, 2, 4, 2, 77, 77, D, causal=causal, seed=3)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


def test_offsets_and_fully_masked_rows():
    """q positions 100.., k positions 130..: the first 30 query rows see no key (O = 0, lse = -inf)."""
    srt = need_gpu()
    o, l, ro, rl = _run(srt, synth.Rope(synth.NTK, 10000.0, 4.0), 1, 2, 1, 70, 45, 64, q_pos0=100, k_pos0=130,
                        seed=4)
    assert np.isneginf(l[:, :, :30]).all() and (o[:, :, :30] == 0).all()
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


def test_single_row_and_prerotated_k():
    srt = need_gpu()
    rp = synth.Rope(synth.PI, 10000.0, 8.0)
    o, l, ro, rl = _run(srt, rp, 1, 1, 1, 1, 1, 64, seed=6)
    assert max_abs(o, ro) <= TOL
    # K rotated by rope_apply first, prefill rotates q only
    q, k, v = qkv(1, 2, 1, 90, 90, 64, torch.float32, 8)
    table, _ = device_table(srt, rp, 64, 90)
    kr = srt.rope_apply(k, table)
    o1, l1 = srt.attn_prefill(q, kr, v, table=table, rope_flags=srt.ROTATE_Q)
    o2, l2 = srt.attn_prefill(q, k, v, table=table)
    assert max_abs(f64(o1), f64(o2)) <= 1e-5
