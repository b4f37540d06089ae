"""GPU parity of srt_attn_ring_prefill (Ring Attention over P devices run on
one GPU, contiguous / striped / zig-zag shards) vs the fp64 oracle.

Inputs are drawn in natural order and moved to the partition's shard-major
order; the oracle's whole-sequence attention, moved the same way, is the
reference (the ring is exact).  Bars: fp32 1e-4, bf16 2e-2 max-abs."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import attention as A
from oracle import ring as R

pytestmark = pytest.mark.gpu

YARN_SMALL = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)


def _case(srt, mode, P, *, dtype=torch.bfloat16, D=128, B=1, Hq=8, Hkv=2, N=1024, window=0, sink=0,
          prerotate=False, half=False, seed=41):
    q, k, v = qkv(B, Hq, Hkv, N, N, D, dtype, seed)
    table, _ = device_table(srt, YARN_SMALL, D, N)
    pos = R.partition_positions(N, P, mode)
    ip = torch.from_numpy(pos).cuda()
    qs, ks, vs = (t.index_select(2, ip).contiguous() for t in (q, k, v))
    pairing = "half" if half else "interleaved"
    flags = srt.ROTATE_Q | srt.ROTATE_K | (srt.PAIR_HALF if half else 0)
    if prerotate:
        ks = srt.rope_apply(k, table, pairing=pairing).index_select(2, ip).contiguous()
        flags &= ~srt.ROTATE_K
    o, l = srt.attn_ring_prefill(qs, ks, vs, num_devices=P, partition=mode, table=table, rope_flags=flags,
                                 window=window, sink=sink)
    th, ms, _ = oracle_freq(YARN_SMALL, D)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), theta=th, mscale=ms, window=window,
                         sink=sink, pairing=pairing)
    return f64(o), f64(l), ro[:, :, pos], rl[:, :, pos]


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("P", [1, 4, 8])
def test_ring_bf16(mode, P):
    srt = need_gpu()
    o, l, ro, rl = _case(srt, mode, P)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
def test_ring_fp32(mode):
    srt = need_gpu()
    o, l, ro, rl = _case(srt, mode, 4, dtype=torch.float32, D=64, Hq=4, Hkv=2, N=512)
    assert max_abs(o, ro) <= 1e-4 and max_abs(l, rl) <= 1e-4


@pytest.mark.parametrize("mode", ["contiguous", "striped", "zigzag"])
def test_ring_prerotated_k_and_half_pairs(mode):
    srt = need_gpu()
    o, l, ro, rl = _case(srt, mode, 4, prerotate=True, seed=42)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2
    o, l, ro, rl = _case(srt, mode, 4, half=True, seed=43)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2


@pytest.mark.parametrize("mode", ["contiguous", "zigzag"])
@pytest.mark.parametrize("W,S", [(100, 4), (300, 70)])
def test_ring_window(mode, W, S):
    srt = need_gpu()
    o, l, ro, rl = _case(srt, mode, 4, window=W, sink=S, seed=44)
    assert max_abs(o, ro) <= 2e-2 and max_abs(l, rl) <= 2e-2


def test_ring_one_device_share_and_errors():
    """device=r writes exactly shard r's rows, with the same bits as the full ring."""
    srt = need_gpu()
    P, N, D = 4, 1024, 128
    q, k, v = qkv(1, 8, 2, N, N, D, torch.bfloat16, 45)
    table, _ = device_table(srt, YARN_SMALL, D, N)
    o_all, l_all = srt.attn_ring_prefill(q, k, v, num_devices=P, partition="zigzag", table=table)
    o = torch.full_like(q, float("nan"))
    l = torch.full((1, 8, N), float("nan"), device="cuda")
    srt.attn_ring_prefill(q, k, v, num_devices=P, partition="zigzag", device=2, table=table, out=o, lse=l)
    C = N // P
    assert torch.equal(o[:, :, 2 * C:3 * C], o_all[:, :, 2 * C:3 * C])
    assert torch.equal(l[:, :, 2 * C:3 * C], l_all[:, :, 2 * C:3 * C])
    assert torch.isnan(o[:, :, :2 * C]).all() and torch.isnan(o[:, :, 3 * C:]).all()
    from scaled_rope_tiled_amd._lib import SrtError
    with pytest.raises(SrtError, match="striped"):
        srt.attn_ring_prefill(q, k, v, num_devices=P, partition="striped", table=table, window=64)
    with pytest.raises(SrtError, match="multiple"):
        srt.attn_ring_prefill(q[:, :, :1004].contiguous(), k[:, :, :1004].contiguous(), v[:, :, :1004].contiguous(),
                              num_devices=P, partition="zigzag", table=table)
