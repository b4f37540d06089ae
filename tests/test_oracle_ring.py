"""Pins of the oracle's Ring Attention and its partitions (CPU only).

"8.3 长上下文技术" §8.3.5: the printed Striped and Zig-Zag shards; the ring
result equals attention over the whole sequence (exactness of the online
softmax); Zig-Zag gives every device the same work at every step."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import ring as R
from oracle import rope

RNG = np.random.default_rng(11)


def test_partitions_match_printed_shards(golden):
    for mode, N, P, shard, *positions in golden("ring_partitions.txt"):
        N, P, shard = int(N), int(P), int(shard)
        C = N // P
        got = R.partition_positions(N, P, mode)[shard * C:(shard + 1) * C]
        assert got.tolist() == [int(x) for x in positions]


@pytest.mark.parametrize("mode", R.PARTITIONS)
@pytest.mark.parametrize("N,P", [(16, 4), (96, 3), (64, 8), (8, 1)])
def test_partition_is_a_permutation(mode, N, P):
    pos = R.partition_positions(N, P, mode)
    assert sorted(pos.tolist()) == list(range(N))
    if mode == "contiguous":
        assert pos.tolist() == list(range(N))


def test_ring_order_follows_the_ring():
    """Step 0 is the device's own shard; each step the shard of the previous device arrives."""
    P = 5
    order = R.ring_order(P)
    for r in range(P):
        js = [j for (rr, s, j) in order if rr == r]
        assert js[0] == r and sorted(js) == list(range(P))
        for s in range(1, P):
            assert js[s] == (js[s - 1] - 1) % P


@pytest.mark.parametrize("mode", R.PARTITIONS)
@pytest.mark.parametrize("P", [1, 2, 4])
def test_ring_equals_unchunked_attention(mode, P):
    B, Hq, Hkv, N, D = 1, 4, 2, 48, 8
    q = RNG.standard_normal((B, Hq, N, D))
    k = RNG.standard_normal((B, Hkv, N, D))
    v = RNG.standard_normal((B, Hkv, N, D))
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 8.0, 16.0, 1.0, 32.0, D)
    pos = R.partition_positions(N, P, mode)
    o, l = R.ring_attention(q[:, :, pos], k[:, :, pos], v[:, :, pos], P=P, mode=mode, sm_scale=0.3, theta=th,
                            mscale=msc)
    ro, rl = A.attention(q, k, v, sm_scale=0.3, theta=th, mscale=msc)
    np.testing.assert_allclose(o, ro[:, :, pos], atol=1e-12)
    np.testing.assert_allclose(l, rl[:, :, pos], atol=1e-12)


@pytest.mark.parametrize("mode", R.PARTITIONS)
def test_ring_with_window_and_sinks(mode):
    B, Hq, Hkv, N, D, P = 1, 2, 1, 64, 8, 4
    q = RNG.standard_normal((B, Hq, N, D))
    k = RNG.standard_normal((B, Hkv, N, D))
    v = RNG.standard_normal((B, Hkv, N, D))
    pos = R.partition_positions(N, P, mode)
    o, l = R.ring_attention(q[:, :, pos], k[:, :, pos], v[:, :, pos], P=P, mode=mode, sm_scale=0.5, window=9,
                            sink=3)
    ro, rl = A.attention(q, k, v, sm_scale=0.5, window=9, sink=3)
    np.testing.assert_allclose(o, ro[:, :, pos], atol=1e-12)
    np.testing.assert_allclose(l, rl[:, :, pos], atol=1e-12)


def test_zigzag_balances_every_step():
    """§8.3.5: with Zig-Zag every device does the same work at every step."""
    for N, P in [(16, 4), (64, 8), (1024, 8)]:
        w = R.step_work(N, P, "zigzag")
        assert (w == w[:1, :]).all(), w
        h = N // (2 * P)
        assert w[0, 0] == 2 * h * h + h and (w[:, 1:] == 2 * h * h).all()
        assert w.sum() == N * (N + 1) // 2


def test_contiguous_is_unbalanced_striped_nearly_balanced():
    """Contiguous: device r does r full blocks plus a diagonal; Striped: per-step
    work differs across devices by at most one diagonal (C pairs)."""
    N, P = 256, 8
    C = N // P
    wc = R.step_work(N, P, "contiguous").sum(axis=1)
    assert wc.tolist() == [r * C * C + C * (C + 1) // 2 for r in range(P)]
    ws = R.step_work(N, P, "striped")
    assert (ws.max(axis=0) - ws.min(axis=0) <= C).all()
    assert ws.sum() == wc.sum() == N * (N + 1) // 2
    tot = ws.sum(axis=1)                    # device r: r + 1 diagonal blocks, the rest strictly below
    assert tot.tolist() == [P * C * (C - 1) // 2 + (r + 1) * C for r in range(P)]
    assert wc.max() / wc.mean() > 1.8
