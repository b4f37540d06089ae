"""GPU parity of split-K decode vs the fp64 oracle (bar: max-abs 2e-2 on O, bf16)."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq
from oracle import attention as A
from oracle import rope as orope

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _case(srt, B, Hq, Hkv, Nk, splits, seq_lens=None, seed=5, rp=synth.Rope(synth.PI, 10000.0, 16.0)):
    D = 128
    q = synth.randn((B, Hq, D), torch.bfloat16, seed, synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, Nk, D), torch.bfloat16, seed, synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, Nk, D), torch.bfloat16, seed, synth.V_ID, "cuda")
    table, _ = device_table(srt, rp, D, Nk)
    kc = srt.rope_apply(k, table)                       # rotated cache at positions 0..Nk-1
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    o, l = srt.attn_decode_splitk(q, kc, v, num_splits=splits, table=table, seq_lens=sl)
    th, ms, _ = oracle_freq(rp, D)
    kref = np.stack([orope.rotate(f64(k[b]), np.arange(Nk), th, ms) for b in range(B)])
    ro, rl = A.decode(f64(q), kref, f64(v), sm_scale=1 / math.sqrt(D), seq_lens=seq_lens, theta=th, mscale=ms)
    return f64(o), f64(l), ro, rl


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_small(G):
    srt = need_gpu()
    o, l, ro, rl = _case(srt, 3, 2 * G, 2, 1000, 7)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= 1e-2


def test_decode_seq_lens_edge_cases():
    """Lengths 0 (no key: O = 0, lse = -inf), 1, a ragged one, and the full cache."""
    srt = need_gpu()
    o, l, ro, rl = _case(srt, 4, 8, 2, 777, 5, seq_lens=[0, 1, 300, 777])
    assert (o[0] == 0).all() and np.isneginf(l[0]).all()
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= 1e-2


def test_decode_one_split_and_many_splits():
    srt = need_gpu()
    for splits in (1, 64, 200):
        o, l, ro, rl = _case(srt, 2, 4, 1, 2000, splits, seed=7)
        assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= 1e-2


def test_decode_given_q_is_exact_at_large_scores():
    """Without a table q is used as given, exactly (the dot products are
    scaled in fp32, as the prefill kernel does), so at sm_scale = 0.5 (scores
    near 30 in log2 units) lse stays within fp32 accuracy of the oracle; a
    bf16 rounding of q * sm_scale log2(e) would move it by about 2^-9 of the
    score (~0.04)."""
    srt = need_gpu()
    B, Hq, Hkv, Nk, D = 2, 8, 2, 1500, 128
    q = synth.randn((B, Hq, D), torch.bfloat16, 71, synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 71, synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, Nk, D), torch.bfloat16, 71, synth.V_ID, "cuda")
    o, l = srt.attn_decode_splitk(q, k, v, num_splits=16, sm_scale=0.5)
    ro, rl = A.decode(f64(q), f64(k), f64(v), sm_scale=0.5)
    print(f"max|err| O {max_abs(f64(o), ro):.3g} lse {max_abs(f64(l), rl):.3g}", flush=True)
    assert max_abs(f64(l), rl) <= 1e-3
    assert max_abs(f64(o), ro) <= TOL
