"""GPU parity of the sliding-window and sink masks vs the fp64 oracle.

Key j stays visible to query i iff j <= i and (i - j < W or j < S), absolute
positions.  Bars: fp32 path 1e-4, bf16 paths 2e-2 max-abs (O and lse).  Cases
span several tiles, windows shorter and longer than a tile, sinks inside one
tile and across two, ring-chunk offsets (sinks are absolute positions), W = 1
and W past the sequence length."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import attention as A
from oracle import rope as orope

pytestmark = pytest.mark.gpu

YARN_SMALL = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W,S", [(1, 0), (16, 0), (50, 4), (300, 4), (40, 45)])
def test_prefill_f32_window(D, W, S):
    srt = need_gpu()
    q, k, v = qkv(1, 4, 2, 200, 200, D, torch.float32, 31)
    table, _ = device_table(srt, YARN_SMALL, D, 200)
    o, l = srt.attn_prefill(q, k, v, table=table, window=W, sink=S)
    th, ms, _ = oracle_freq(YARN_SMALL, D)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), theta=th, mscale=ms, window=W, sink=S)
    assert max_abs(f64(o), ro) <= 1e-4 and max_abs(f64(l), rl) <= 1e-4


def _bf16_case(srt, B, Hq, Hkv, Nq, Nk, W, S, *, q_pos0=0, k_pos0=0, seed=32, rows=None, rotate_k_on_load=False):
    D = 128
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, D, torch.bfloat16, seed)
    table, _ = device_table(srt, YARN_SMALL, D, max(q_pos0 + Nq, k_pos0 + Nk))
    if rotate_k_on_load:
        o, l = srt.attn_prefill(q, k, v, table=table, q_pos0=q_pos0, k_pos0=k_pos0, window=W, sink=S)
    else:
        kr = srt.rope_apply(k, table, pos0=k_pos0)
        o, l = srt.attn_prefill(q, kr, v, table=table, rope_flags=srt.ROTATE_Q, q_pos0=q_pos0, k_pos0=k_pos0,
                                window=W, sink=S)
    th, ms, _ = oracle_freq(YARN_SMALL, D)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), q_pos0=q_pos0, k_pos0=k_pos0,
                         theta=th, mscale=ms, window=W, sink=S, rows=rows)
    o, l = f64(o), f64(l)
    if rows is not None:
        o, l = o[:, :, rows], l[:, :, rows]
    return o, l, ro, rl


@pytest.mark.parametrize("W,S", [(1, 0), (64, 0), (100, 4), (257, 4), (130, 70), (1000, 4)])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_prefill_bf16_window(W, S, G):
    srt = need_gpu()
    o, l, ro, rl = _bf16_case(srt, 1, 2 * G if G < 8 else 8, 2 if G < 8 else 1, 700, 700, W, S)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2


@pytest.mark.parametrize("rot_k", [False, True])
def test_prefill_bf16_window_ring_offsets(rot_k):
    """One ring chunk pair: queries at 600.., keys at 100..; sinks are absolute
    positions, so this chunk holds none of them and a 64-position window leaves
    the early keys invisible to every query."""
    srt = need_gpu()
    for W, S in [(64, 4), (550, 4), (300, 150)]:
        o, l, ro, rl = _bf16_case(srt, 2, 8, 2, 300, 450, W, S, q_pos0=600, k_pos0=100, rotate_k_on_load=rot_k)
        assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2
    # keys wholly outside every query's window and past the sinks: identity state
    o, l, ro, rl = _bf16_case(srt, 1, 4, 1, 100, 200, 64, 4, q_pos0=5000, k_pos0=1000)
    assert np.isneginf(l).all() and (o == 0).all()


def test_prefill_bf16_window_32k_sampled():
    """32K-token GQA 32/8, W = 4096, S = 4: sampled rows from the first window,
    around each tile edge and the last rows."""
    srt = need_gpu()
    N = 32768
    rows = np.unique(np.concatenate([[0, 1, 3, 4, 63, 64, 4095, 4096, 4097, 4100, 8191, 8192, 16383],
                                     np.arange(N - 5, N),
                                     np.random.default_rng(1).integers(0, N, 12)]))
    o, l, ro, rl = _bf16_case(srt, 1, 32, 8, N, N, 4096, 4, seed=33, rows=rows)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2


@pytest.mark.parametrize("W,S", [(1, 0), (100, 0), (300, 4), (5000, 4)])
def test_decode_window(W, S):
    srt = need_gpu()
    D, B, Hq, Hkv, Nk = 128, 6, 8, 2, 2000
    rp = synth.Rope(synth.PI, 10000.0, 16.0)
    q = synth.randn((B, Hq, D), torch.bfloat16, 34, synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 34, synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 34, synth.V_ID, "cuda")
    table, _ = device_table(srt, rp, D, Nk)
    kc = srt.rope_apply(k, table)
    lens = [0, 1, 3, 302, 1500, 2000]
    o, l = srt.attn_decode_splitk(q, kc, v, num_splits=7, table=table, window=W, sink=S,
                                  seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    th, ms, _ = oracle_freq(rp, D)
    kref = np.stack([orope.rotate(f64(k[b]), np.arange(Nk), th, ms) for b in range(B)])
    ro, rl = A.decode(f64(q), kref, f64(v), sm_scale=1 / math.sqrt(D), seq_lens=lens, theta=th, mscale=ms,
                      window=W, sink=S)
    o, l = f64(o), f64(l)
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 1e-2
