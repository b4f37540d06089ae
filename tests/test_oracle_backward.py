"""Pins of the oracle's attention backward (CPU only).

Central finite differences of the oracle's own forward (loss = sum O * dO)
check every gradient entry; torch autograd in float64 on an independent
complex-number forward is a library check; N = 1 is a closed form
(O = v: dv = dO, dq = dk = 0)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import backward as BW
from oracle import rope

RNG = np.random.default_rng(21)


def _fd(fn, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = fn()
        x[i] = old - h
        fm = fn()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("kw", [
    dict(),
    dict(q_pos0=7, k_pos0=3),
    dict(window=3, sink=1),
    dict(pairing="half"),
    dict(causal=False),
])
def test_gradients_match_finite_differences(kw):
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 5, 6 if "q_pos0" in kw else 5, 4
    q = RNG.standard_normal((B, Hq, Nq, D))
    k = RNG.standard_normal((B, Hkv, Nk, D))
    v = RNG.standard_normal((B, Hkv, Nk, D))
    do = RNG.standard_normal((B, Hq, Nq, D))
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 8.0, 16.0, 1.0, 32.0, D)
    common = dict(sm_scale=0.7, theta=th, mscale=msc, **kw)

    def loss():
        o, _ = A.attention(q, k, v, **common)
        return float((o * do).sum())

    dq, dk, dv, _ = BW.attention_backward(q, k, v, do, **common)
    np.testing.assert_allclose(dq, _fd(loss, q), atol=2e-8)
    np.testing.assert_allclose(dk, _fd(loss, k), atol=2e-8)
    np.testing.assert_allclose(dv, _fd(loss, v), atol=2e-8)


def test_matches_torch_autograd_float64():
    """Library check: autograd through a torch forward that rotates with complex multiplication."""
    B, Hq, Hkv, N, D = 1, 4, 2, 23, 8
    q = RNG.standard_normal((B, Hq, N, D))
    k = RNG.standard_normal((B, Hkv, N, D))
    v = RNG.standard_normal((B, Hkv, N, D))
    do = RNG.standard_normal((B, Hq, N, D))
    th, msc, _ = rope.inv_freq(rope.NTK, 1e4, 4.0, D=D)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ang = torch.tensor(np.arange(N)[:, None] * th[None, :])
    e = torch.polar(torch.ones_like(ang), ang) * msc

    def rot(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2).contiguous())
        return torch.view_as_real(z * e).reshape(x.shape)

    kr = rot(tk).repeat_interleave(Hq // Hkv, dim=1)
    vr = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = 0.4 * rot(tq) @ kr.transpose(-1, -2)
    s = s.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv, _ = BW.attention_backward(q, k, v, do, sm_scale=0.4, theta=th, mscale=msc)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_single_key_closed_form():
    """N = 1: O = v, so dv = sum of dO over the group, dq = dk = 0; delta = dO . v."""
    q = RNG.standard_normal((1, 4, 1, 8))
    k = RNG.standard_normal((1, 2, 1, 8))
    v = RNG.standard_normal((1, 2, 1, 8))
    do = RNG.standard_normal((1, 4, 1, 8))
    th = rope.base_inv_freq(8, 1e4)
    dq, dk, dv, delta = BW.attention_backward(q, k, v, do, sm_scale=0.3, theta=th, mscale=1.2)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, 0], do[0, 0] + do[0, 1], atol=1e-15)
    np.testing.assert_allclose(delta[0, 2], (do[0, 2] * v[0, 1]).sum(axis=-1), atol=1e-14)


def test_rotate_back_is_the_transpose():
    D = 16
    th = rope.base_inv_freq(D, 1e4)
    x, g = RNG.standard_normal((5, D)), RNG.standard_normal((5, D))
    pos = np.array([0, 3, 100, 4095, 65000])
    for pairing, fn in (("interleaved", rope.rotate), ("half", rope.rotate_half)):
        lhs = (fn(x, pos, th, 1.3) * g).sum(axis=1)
        rhs = (x * BW.rotate_back(g, pos, th, 1.3, pairing)).sum(axis=1)
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


@pytest.mark.parametrize("kw", [dict(), dict(causal=False), dict(window=9, sink=2), dict(q_pos0=3, k_pos0=11),
                                dict(pairing="half"), dict(rotate=False)],
                         ids=["causal", "noncausal", "window", "masked_rows", "half", "given"])
def test_sampled_backward_equals_full(kw):
    """attention_backward_sampled (the form full-size GPU tests use) returns exactly the entries of the full
    oracle backward at the chosen rows and keys, GQA 4/2, YaRN rotation."""
    kw = dict(kw)
    rotate = kw.pop("rotate", True)
    rng = np.random.default_rng(7)
    B, Hq, Hkv, N, D = 1, 4, 2, 40, 8
    q, k, v, do = (rng.standard_normal(s) for s in [(B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D), (B, Hq, N, D)])
    th, ms, _ = rope.inv_freq(rope.YARN, 10000.0, 4.0, 16.0, 1.0, 32.0, D)
    rk = dict(theta=th if rotate else None, mscale=ms if rotate else 1.0)
    full = BW.attention_backward(q, k, v, do, sm_scale=0.3, **rk, **kw)
    rows, keys = [0, 7, 23, 39], [0, 1, 20, 39]
    for hk in range(Hkv):
        dq, dk, dv = BW.attention_backward_sampled(q, k, v, do, hk=hk, rows=rows, keys=keys, sm_scale=0.3, **rk, **kw)
        np.testing.assert_allclose(dq, full[0][0, 2 * hk:2 * hk + 2][:, rows], atol=1e-12)
        np.testing.assert_allclose(dk, full[1][0, hk][keys], atol=1e-12)
        np.testing.assert_allclose(dv, full[2][0, hk][keys], atol=1e-12)
