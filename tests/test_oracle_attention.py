"""Pins of the oracle's attention, merge and decode (CPU only).

The row-block oracle is checked against: a brute force that uses explicit
rotation matrices and the full score matrix; torch's scaled_dot_product
attention and scipy's logsumexp in float64 (library routines); closed-form
special cases of the softmax; GQA by explicit K/V head repetition; chunking
with the log-sum-exp merge (FlashAttention / Ring Attention exactness).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as A
from oracle import rope

RNG = np.random.default_rng(7)


def _qkv(B, Hq, Hkv, Nq, Nk, D):
    return (RNG.standard_normal((B, Hq, Nq, D)), RNG.standard_normal((B, Hkv, Nk, D)),
            RNG.standard_normal((B, Hkv, Nk, D)))


@pytest.mark.parametrize("D", [4, 8, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_row_block_equals_brute_force(D, causal):
    """"Long Context..." §2.4 definition; brute force with blkdiag R_m (§2.2)."""
    B, Hq, Hkv, N = 1, 4, 2, 37
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 16.0, 64.0, 1.0, 32.0, D)
    kw = dict(sm_scale=1 / math.sqrt(D), causal=causal, theta=th, mscale=msc)
    o1, l1 = A.attention(q, k, v, block=5, **kw)
    o2, l2 = A.brute_force(q, k, v, **kw)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_offsets_brute_force_and_fully_masked_rows():
    """Absolute-position causal mask with q_pos0 < k_pos0: early rows see nothing (O = 0, lse = -inf)."""
    D = 8
    q, k, v = _qkv(1, 2, 1, 12, 10, D)
    th = rope.base_inv_freq(D, 1e4)
    kw = dict(sm_scale=0.3, causal=True, q_pos0=100, k_pos0=105, theta=th)
    o1, l1 = A.attention(q, k, v, **kw)
    o2, l2 = A.brute_force(q, k, v, **kw)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(l1), np.isinf(l2))
    assert np.isneginf(l1[0, :, :5]).all() and (o1[0, :, :5] == 0).all()
    np.testing.assert_allclose(l1[np.isfinite(l1)], l2[np.isfinite(l2)], atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_float64(causal):
    """Library check: torch SDPA (float64, CPU) on the rotated q, k; lse vs scipy logsumexp."""
    B, Hq, Hkv, N, D = 2, 4, 4, 70, 64
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th = rope.base_inv_freq(D, 500000.0)
    pos = np.arange(N)
    qr = rope.rotate(q, pos, th)
    kr = rope.rotate(k, pos, th)
    sc = 1 / math.sqrt(D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr), torch.from_numpy(kr), torch.from_numpy(v), is_causal=causal, scale=sc).numpy()
    o, l = A.attention(q, k, v, sm_scale=sc, causal=causal, theta=th, block=16)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    S = sc * np.einsum("bhqd,bhkd->bhqk", qr, kr)
    if causal:
        S = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf)
    np.testing.assert_allclose(l, logsumexp(S, axis=-1), atol=1e-12)


def test_gqa_equals_repeated_heads():
    """GQA: query head h reads kv head h // (Hq/Hkv); equal to MHA over repeated K/V."""
    B, Hq, Hkv, N, D = 1, 8, 2, 33, 16
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th = rope.base_inv_freq(D, 1e4)
    o1, l1 = A.attention(q, k, v, sm_scale=0.25, theta=th)
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).numpy()
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).numpy()
    o2, l2 = A.attention(q, kk, vv, sm_scale=0.25, theta=th)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_softmax_special_cases():
    """Closed forms of softmax attention: single visible key, constant V, q = 0."""
    B, H, N, D = 1, 1, 20, 8
    q, k, v = _qkv(B, H, H, N, N, D)
    th = rope.base_inv_freq(D, 1e4)
    o, l = A.attention(q, k, v, sm_scale=0.5, theta=th)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-14)        # row 0 sees key 0 only
    kr0 = rope.rotate(k[0, 0, :1], [0], th)[0]
    assert l[0, 0, 0] == pytest.approx(0.5 * float(q[0, 0, 0] @ kr0), abs=1e-13)
    vc = np.broadcast_to(RNG.standard_normal(D), (B, H, N, D)).copy()
    o, _ = A.attention(q, k, vc, sm_scale=0.5, theta=th)
    np.testing.assert_allclose(o, vc, atol=1e-13)                         # constant V
    o, l = A.attention(np.zeros_like(q), k, v, sm_scale=0.5, theta=th)
    means = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], means, atol=1e-13)                # uniform weights
    np.testing.assert_allclose(l[0, 0], np.log(np.arange(1, N + 1)), atol=1e-13)


def test_temperature_folding_equivalence():
    """"Long Context..." §6.4 / "8.3 长上下文技术" §8.3.3: scaling rotated q and k by
    sqrt(1/t) equals dividing the logits by t (sm_scale * mscale^2)."""
    B, H, N, D = 1, 2, 25, 16
    q, k, v = _qkv(B, H, H, N, N, D)
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 16.0, 64.0, 1.0, 32.0, D)
    o1, l1 = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=msc)
    o2, l2 = A.attention(q, k, v, sm_scale=0.25 * msc * msc, theta=th, mscale=1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    o3, _ = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=1.0)
    assert np.abs(o1 - o3).max() > 1e-3                                   # the factor matters


@pytest.mark.parametrize("chunks", [1, 2, 3, 8])
def test_chunked_merge_equals_unchunked(chunks):
    """Ring step on one device ("8.3 长上下文技术" §8.3.5): K/V split into chunks at
    absolute offsets, partial (O, lse) merged in any order == full attention."""
    B, Hq, Hkv, N, D = 1, 4, 2, 48, 8
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th = rope.base_inv_freq(D, 1e4)
    full_o, full_l = A.attention(q, k, v, sm_scale=0.35, theta=th)
    edges = np.linspace(0, N, chunks + 1).astype(int)
    order = RNG.permutation(chunks)
    acc = None
    for j in order:
        a, b = edges[j], edges[j + 1]
        part = A.attention(q, k[:, :, a:b], v[:, :, a:b], sm_scale=0.35, k_pos0=int(a), theta=th)
        acc = part if acc is None else A.merge(*acc, *part)
    np.testing.assert_allclose(acc[0], full_o, atol=1e-12)
    np.testing.assert_allclose(acc[1], full_l, atol=1e-12)


def test_merge_identity_and_associativity():
    """-inf state is the identity; (-inf, -inf) -> (0, -inf); merge is associative and commutative."""
    shp = (2, 3, 5)
    oa, ob, oc = (RNG.standard_normal(shp + (4,)) for _ in range(3))
    la, lb, lc = (RNG.standard_normal(shp) * 3 for _ in range(3))
    ninf = np.full(shp, -np.inf)
    o, l = A.merge(oa, la, np.zeros_like(oa), ninf)
    np.testing.assert_allclose(o, oa, atol=1e-15)
    np.testing.assert_allclose(l, la, atol=1e-15)
    o, l = A.merge(oa, ninf, ob, ninf)
    assert (o == 0).all() and np.isneginf(l).all()
    x1 = A.merge(*A.merge(oa, la, ob, lb), oc, lc)
    x2 = A.merge(oa, la, *A.merge(ob, lb, oc, lc))
    x3 = A.merge(oc, lc, *A.merge(ob, lb, oa, la))
    for x in (x2, x3):
        np.testing.assert_allclose(x[0], x1[0], atol=1e-13)
        np.testing.assert_allclose(x[1], x1[1], atol=1e-13)
    # explicit definition at one point: log of summed exponentials
    i = (0, 0, 0)
    assert x1[1][i] == pytest.approx(math.log(math.exp(la[i]) + math.exp(lb[i]) + math.exp(lc[i])), abs=1e-12)


def test_decode_equals_last_row_of_causal_prefill_and_split():
    """Decode (one query at position Nk-1, cache already rotated) == last row of full causal
    attention; splitting the cache into blocks and merging gives the same result."""
    B, Hq, Hkv, N, D = 2, 4, 2, 40, 16
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th, msc, _ = rope.inv_freq(rope.PI, 1e4, 16.0, D=D)
    full_o, full_l = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=msc)
    kc = np.stack([rope.rotate(k[b], np.arange(N), th, msc) for b in range(B)])
    o, l = A.decode(q[:, :, -1], kc, v, sm_scale=0.25, theta=th, mscale=msc)
    np.testing.assert_allclose(o, full_o[:, :, -1], atol=1e-12)
    np.testing.assert_allclose(l, full_l[:, :, -1], atol=1e-12)
    # split-K over 4 blocks, rotated query, merged
    qr = np.stack([rope.rotate(q[b, :, -1][:, None], [N - 1], th, msc)[:, 0] for b in range(B)])
    acc = None
    for a in range(0, N, 10):
        part = A.attention(qr[:, :, None], kc[:, :, a:a + 10], v[:, :, a:a + 10], sm_scale=0.25, causal=False)
        acc = part if acc is None else A.merge(*acc, *part)
    np.testing.assert_allclose(acc[0][:, :, 0], o, atol=1e-12)
    # per-sequence lengths: a shorter sequence sees only its first n keys
    o2, l2 = A.decode(q[:, :, -1], kc, v, sm_scale=0.25, seq_lens=[N, 17], theta=th, mscale=msc)
    np.testing.assert_allclose(o2[0], o[0], atol=1e-13)
    r17, l17 = A.attention(q[1:2, :, -1:], k[1:2, :, :17], v[1:2, :, :17], sm_scale=0.25, q_pos0=16,
                           theta=th, mscale=msc)
    np.testing.assert_allclose(o2[1], r17[0, :, 0], atol=1e-12)


def test_row_subset_matches_full():
    q, k, v = _qkv(1, 2, 1, 300, 300, 8)
    th = rope.base_inv_freq(8, 1e4)
    o, l = A.attention(q, k, v, sm_scale=0.3, theta=th)
    rows = np.array([0, 1, 255, 256, 299])
    o2, l2 = A.attention(q, k, v, sm_scale=0.3, theta=th, rows=rows)
    np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(l2, l[:, :, rows], atol=1e-14)


def test_half_split_attention_is_interleaved_on_permuted_dims():
    """"Long Context..." §2.4: the half-split rule is the interleaved one on permuted
    dimensions, and q.k is invariant under one permutation of both q and k."""
    B, Hq, Hkv, N, D = 1, 4, 2, 30, 16
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 8.0, 64.0, 1.0, 32.0, D)
    perm = np.empty(D, dtype=int)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    o1, l1 = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=msc, pairing="half")
    o2, l2 = A.attention(q[..., perm], k[..., perm], v, sm_scale=0.25, theta=th, mscale=msc)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    o3, _ = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=msc)
    assert np.abs(o1 - o3).max() > 1e-3
    kc = np.stack([rope.rotate_half(k[0], np.arange(N), th, msc)])
    od, ld = A.decode(q[:, :, -1], kc, v, sm_scale=0.25, theta=th, mscale=msc, pairing="half")
    np.testing.assert_allclose(od, o1[:, :, -1], atol=1e-12)


# --------------------------------------------------------------------------- sliding window and sinks

def test_sliding_window_mask_matches_printed(golden):
    """"Long Context..." §10.1: the printed L = 8, W = 4 mask, row by row."""
    want = np.array([[c == "T" for c in row[1:]] for row in golden("sliding_window_mask_L8_W4.txt")])
    got = A.visible(np.arange(8), np.arange(8), window=4)
    np.testing.assert_array_equal(got, want)
    # no window: the plain causal mask; a window as long as the sequence changes nothing
    np.testing.assert_array_equal(A.visible(np.arange(8), np.arange(8)), np.tri(8, dtype=bool))
    np.testing.assert_array_equal(A.visible(np.arange(8), np.arange(8), window=8), np.tri(8, dtype=bool))
    with pytest.raises(ValueError):
        A.visible(np.arange(8), np.arange(8), causal=False, window=4)


def test_streaming_sinks_keep_first_s_and_last_w(golden):
    """"Long Context..." §10.2: the last query sees the first S tokens and the last W: S + W keys."""
    (_, S, W, n_keys), = [r for r in golden("sliding_window_work.txt") if r[0] == "streaming_cache"]
    S, W, n_keys = int(S), int(W), int(n_keys)
    N = 10000
    row = A.visible([N - 1], np.arange(N), window=W, sink=S)[0]
    assert row.sum() == n_keys == S + W
    assert row[:S].all() and row[N - W:].all() and not row[S:N - W].any()
    # rows still inside the first S + W positions see every earlier key
    early = A.visible(np.arange(S + W), np.arange(S + W), window=W, sink=S)
    assert early.sum(axis=1).tolist() == [min(i + 1, W) + min(S, max(0, i - W + 1)) for i in range(S + W)]


def test_visible_pair_counts(golden):
    """O(N W) work: the row-by-row count equals the mask's count on small cases and
    reproduces the printed 16B -> 524M (97 % fewer) at N = 128K, W = 4096."""
    for N, W, S in [(1, 0, 0), (50, 0, 0), (50, 7, 0), (50, 7, 4), (50, 60, 4), (33, 1, 3)]:
        m = A.visible(np.arange(N), np.arange(N), window=W, sink=S)
        assert A.visible_pairs(N, W, S) == int(m.sum())
    rows = {r[0]: r for r in golden("sliding_window_work.txt")}
    N, W = int(rows["window_dots"][1]), int(rows["window_dots"][2])
    full, win = A.visible_pairs(N), A.visible_pairs(N, W)
    assert abs(N * N - float(rows["full_dots"][3])) <= float(rows["full_dots"][4]) * float(rows["full_dots"][3])
    assert abs(win - float(rows["window_dots"][3])) <= float(rows["window_dots"][4]) * float(rows["window_dots"][3])
    assert win == N * W - W * (W - 1) // 2              # closed form of the ramp
    assert full == N * (N + 1) // 2
    pct = 100.0 * (1.0 - (N * W) / (N * N))
    assert abs(pct - float(rows["reduction_pct"][3])) <= float(rows["reduction_pct"][4])


@pytest.mark.parametrize("W,S", [(1, 0), (5, 0), (5, 3), (16, 4), (40, 2)])
def test_window_attention_equals_brute_force(W, S):
    B, Hq, Hkv, N, D = 1, 4, 2, 37, 8
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 16.0, 64.0, 1.0, 32.0, D)
    kw = dict(sm_scale=1 / math.sqrt(D), theta=th, mscale=msc, window=W, sink=S)
    o1, l1 = A.attention(q, k, v, block=6, **kw)
    o2, l2 = A.brute_force(q, k, v, **kw)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    # offsets (one ring chunk): sinks are absolute positions, so a chunk past them has none
    kw2 = dict(kw, q_pos0=30, k_pos0=0)
    o3, l3 = A.attention(q[:, :, :7], k, v, **kw2)
    o4, l4 = A.brute_force(q[:, :, :7], k, v, **kw2)
    np.testing.assert_allclose(o3, o4, atol=1e-12)


def test_window_special_cases():
    """W = 1, no sink: each query sees only itself (O = v_i, lse = its own score);
    W >= N: plain causal attention; window attention == full attention over the kept keys."""
    B, H, N, D = 1, 2, 20, 8
    q, k, v = _qkv(B, H, H, N, N, D)
    o, l = A.attention(q, k, v, sm_scale=0.5, window=1)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(l, 0.5 * np.einsum("bhnd,bhnd->bhn", q, k), atol=1e-12)
    o1, l1 = A.attention(q, k, v, sm_scale=0.5, window=N, sink=3)
    o2, l2 = A.attention(q, k, v, sm_scale=0.5)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    W, S, i = 6, 2, 15
    keep = sorted(set(range(S)) | set(range(i - W + 1, i + 1)))
    o3, l3 = A.attention(q[:, :, i:i + 1], k[:, :, keep], v[:, :, keep], sm_scale=0.5, causal=False)
    o4, l4 = A.attention(q, k, v, sm_scale=0.5, window=W, sink=S, rows=[i])
    np.testing.assert_allclose(o4, o3, atol=1e-13)
    np.testing.assert_allclose(l4, l3, atol=1e-13)


def test_decode_window_equals_last_row():
    B, Hq, Hkv, N, D = 2, 4, 2, 40, 16
    q, k, v = _qkv(B, Hq, Hkv, N, N, D)
    th, msc, _ = rope.inv_freq(rope.PI, 1e4, 16.0, D=D)
    kc = np.stack([rope.rotate(k[b], np.arange(N), th, msc) for b in range(B)])
    for W, S in [(8, 0), (8, 4), (100, 4)]:
        full_o, full_l = A.attention(q, k, v, sm_scale=0.25, theta=th, mscale=msc, window=W, sink=S)
        o, l = A.decode(q[:, :, -1], kc, v, sm_scale=0.25, theta=th, mscale=msc, window=W, sink=S)
        np.testing.assert_allclose(o, full_o[:, :, -1], atol=1e-12)
        np.testing.assert_allclose(l, full_l[:, :, -1], atol=1e-12)


@pytest.mark.parametrize("window,sink", [(0, 0), (5, 2)])
def test_empty_key_set_equals_invisible_keys(window, sink):
    """Nk = 0 is the limit of a key set no row can see: every row has O = 0 and
    lse = -inf (the convention for a row without a visible key), exactly what
    keys placed after every query position give under the causal mask; the
    backward of such rows is zero."""
    from oracle import backward as BW
    D = 8
    q, k, v = _qkv(2, 4, 2, 9, 6, D)
    th = rope.base_inv_freq(D, 1e4)
    kw = dict(sm_scale=0.3, causal=True, theta=th, window=window, sink=sink, q_pos0=40)
    o0, l0 = A.attention(q, k[:, :, :0], v[:, :, :0], **kw)
    o1, l1 = A.attention(q, k, v, k_pos0=50, **kw)        # keys at 50.., queries at 40..48
    assert o0.shape == q.shape and (o0 == 0).all() and np.isneginf(l0).all()
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    dq, dk, dv, _ = BW.attention_backward(q, k[:, :, :0], v[:, :, :0], np.ones_like(q), **kw)
    assert (dq == 0).all() and dk.shape[2] == 0 and dv.shape[2] == 0
