"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times, on sampled output rows the oracle computes one by one.

Row samples per head: the first and last rows, both sides of every 64-row
kernel tile edge near the sample points, both sides of every ring chunk edge,
and seeded random rows.  Bar: max-abs <= 1e-4 (fp32) / 2e-2 (bf16) on O and lse."""
import math
import os

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq
from oracle import attention as A
from oracle import rope as orope

pytestmark = pytest.mark.gpu
TOL = 2e-2
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _row_ranges(N, seed, chunk=None, n_random=24):
    rng = np.random.default_rng(seed)
    ranges = [(0, 8), (N - 8, N), (63, 66), (N // 2 - 1, N // 2 + 1)]
    if chunk:
        for j in range(1, N // chunk):
            ranges.append((j * chunk - 2, j * chunk + 2))
    for r in rng.integers(0, N - 2, n_random):
        ranges.append((int(r), int(r) + 2))
    return sorted(set(ranges))


def _inputs(w, device="cuda"):
    D = w.D
    q = synth.randn((w.B, w.Hq, w.N, D), w.dtype, w.seed, synth.Q_ID, device)
    k = synth.randn((w.B, w.Hkv, w.N, D), w.dtype, w.seed, synth.K_ID, device)
    v = synth.randn((w.B, w.Hkv, w.N, D), w.dtype, w.seed, synth.V_ID, device)
    return q, k, v


def _check_rows(w, q, k, v, outs, ranges):
    """Oracle on the sampled rows: rotate each KV head once (fp64), then plain
    softmax attention for each contiguous row range at its absolute position.
    ``outs`` is a list of (O, lse) results of the same problem; returns the
    worst (O error, lse error) of each."""
    th, ms, _ = oracle_freq(w.rope, w.D)
    G = w.Hq // w.Hkv
    worst = [[0.0, 0.0] for _ in outs]
    for b in range(w.B):
        for hk in range(w.Hkv):
            kr = orope.rotate(f64(k[b, hk]), np.arange(w.N), th, ms)[None, None]
            vv = f64(v[b, hk])[None, None]
            for h in range(hk * G, (hk + 1) * G):
                for a, e in ranges:
                    qr = orope.rotate(f64(q[b, h, a:e]), np.arange(a, e), th, ms)[None, None]
                    ro, rl = A.attention(qr, kr[:, :, :e], vv[:, :, :e], sm_scale=w.sm_scale, causal=True,
                                         q_pos0=a, k_pos0=0, theta=None)
                    for i, (o, l) in enumerate(outs):
                        worst[i][0] = max(worst[i][0], max_abs(f64(o[b, h, a:e]), ro[0, 0]))
                        worst[i][1] = max(worst[i][1], max_abs(f64(l[b, h, a:e]), rl[0, 0]))
    return worst


@pytest.mark.parametrize("name", ["gqa_8k_bf16", "yarn_32k_bf16"])
def test_prefill_full_size(name):
    """Two launches of the full-size problem against the oracle on the same
    rows: K rotated once by rope_apply and q rotated on load (the launch the
    benchmark times), and q and k both rotated on load."""
    srt = need_gpu()
    w = synth.WORKLOADS[name]
    q, k, v = _inputs(w)
    table, _ = device_table(srt, w.rope, w.D, w.N)
    kr = srt.rope_apply(k, table)
    o_b, l_b = srt.attn_prefill(q, kr, v, table=table, rope_flags=srt.ROTATE_Q)   # the benchmark's launch
    del kr
    o_r, l_r = srt.attn_prefill(q, k, v, table=table)                           # q and k rotated on load
    torch.cuda.synchronize()
    (wo_b, wl_b), (wo_r, wl_r) = _check_rows(w, q, k, v, [(o_b, l_b), (o_r, l_r)], _row_ranges(w.N, w.seed))
    print(f"{name} rope_apply(k) + ROTATE_Q: max|dO|={wo_b:.3g} max|dlse|={wl_b:.3g}; "
          f"ROTATE_Q|ROTATE_K: max|dO|={wo_r:.3g} max|dlse|={wl_r:.3g}", flush=True)
    assert wo_b <= TOL and wl_b <= TOL
    assert wo_r <= TOL and wl_r <= TOL


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
def test_ring_128k_full_size(partition):
    """NTK 128K as a ring of 8 devices (the benchmark's ring leg): contiguous
    shards of 16384, zig-zag shards (chunks r and 15 - r of 8192) and striped
    shards (positions r + 8t)."""
    srt = need_gpu()
    from oracle import ring as R
    w = synth.WORKLOADS["ntk_128k_ring_bf16"]
    q, k, v = _inputs(w)
    table, _ = device_table(srt, w.rope, w.D, w.N)
    pos = torch.from_numpy(R.partition_positions(w.N, w.chunks, partition)).cuda()
    if partition == "contiguous":
        o, l = srt.attn_ring_prefill(q, k, v, num_devices=w.chunks, partition=partition, table=table)
    else:
        qs, ks, vs = (t.index_select(2, pos).contiguous() for t in (q, k, v))
        os_, ls_ = srt.attn_ring_prefill(qs, ks, vs, num_devices=w.chunks, partition=partition, table=table)
        del qs, ks, vs
        o, l = torch.empty_like(os_), torch.empty_like(ls_)
        o.index_copy_(2, pos, os_)                 # back to natural order
        l.index_copy_(2, pos, ls_)
    torch.cuda.synchronize()
    C = w.N // w.chunks
    ranges = _row_ranges(w.N, w.seed, chunk=C // 2 if partition == "zigzag" else C, n_random=8)
    [(wo, wl)] = _check_rows(w, q, k, v, [(o, l)], ranges)
    print(f"ntk 128k ring {partition}: max|dO|={wo:.3g} max|dlse|={wl:.3g}", flush=True)
    assert wo <= TOL and wl <= TOL


def test_decode_full_size():
    """B=16 sequences, 131072-position rotated cache (PI s=16), 64 splits; one
    (b, kv head) group of every sequence, each KV head twice."""
    srt = need_gpu()
    w = synth.WORKLOADS["decode_128k_bf16"]
    D, N = w.D, w.N
    q = synth.randn((w.B, w.Hq, D), w.dtype, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, N, D), w.dtype, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, N, D), w.dtype, w.seed, synth.V_ID, "cuda")
    table, _ = device_table(srt, w.rope, D, N)
    kc = srt.rope_apply(k, table)
    o, l = srt.attn_decode_splitk(q, kc, v, num_splits=w.splits, table=table)
    torch.cuda.synchronize()
    th, ms, _ = oracle_freq(w.rope, D)
    G = w.Hq // w.Hkv
    worst_o = worst_l = 0.0
    for b in range(w.B):
        hk = b % w.Hkv
        kr = orope.rotate(f64(k[b, hk]), np.arange(N), th, ms)
        hs = slice(hk * G, (hk + 1) * G)
        ro, rl = A.decode(f64(q[b:b + 1, hs]), kr[None, None], f64(v[b, hk])[None, None],
                          sm_scale=w.sm_scale, theta=th, mscale=ms)
        worst_o = max(worst_o, max_abs(f64(o[b, hs]), ro[0]))
        worst_l = max(worst_l, max_abs(f64(l[b, hs]), rl[0]))
    print(f"decode 128k: max|dO|={worst_o:.3g} max|dlse|={worst_l:.3g}", flush=True)
    assert worst_o <= TOL and worst_l <= TOL
