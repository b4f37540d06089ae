"""GPU parity of the bf16 matrix-core prefill kernel vs the fp64 oracle.

Bar: max-abs error <= 2e-2 on O and on lse (bf16 inputs; the oracle consumes
the same bf16 values upcast to fp64).  Small problems are compared element by
element; they span several 64-key tiles, a ragged tail, GQA group sizes 1, 2,
4 and 8, every RoPE method, offsets with fully masked rows, fp32 output and
K pre-rotated by rope_apply."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import attention as A

pytestmark = pytest.mark.gpu
TOL = 2e-2

YARN_SMALL = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)
ROPES = [synth.Rope(synth.NONE, 500000.0), synth.Rope(synth.PI, 10000.0, 16.0),
         synth.Rope(synth.NTK, 10000.0, 16.0), YARN_SMALL]


def _run(srt, rp, B, Hq, Hkv, Nq, Nk, *, causal=True, q_pos0=0, k_pos0=0, seed=2, flags=None,
         out_dtype=None, prerotate_k=False):
    D = 128
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, D, torch.bfloat16, seed)
    table, _ = device_table(srt, rp, D, max(q_pos0 + Nq, k_pos0 + Nk))
    kin = k
    if prerotate_k:
        kin = srt.rope_apply(k.contiguous(), table, pos0=k_pos0)
        flags = srt.ROTATE_Q
    o, l = srt.attn_prefill(q, kin, v, causal=causal, q_pos0=q_pos0, k_pos0=k_pos0, table=table,
                            rope_flags=flags, out_dtype=out_dtype)
    th, ms, _ = oracle_freq(rp, D)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=1 / math.sqrt(D), causal=causal, q_pos0=q_pos0,
                         k_pos0=k_pos0, theta=th, mscale=ms)
    return f64(o), f64(l), ro, rl


@pytest.mark.parametrize("rp", ROPES, ids=lambda r: f"m{r.method}")
def test_methods_gqa4_ragged(rp):
    srt = need_gpu()
    o, l, ro, rl = _run(srt, rp, 1, 8, 2, 200, 200)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_group_sizes(G, causal):
    srt = need_gpu()
    o, l, ro, rl = _run(srt, YARN_SMALL, 2, 2 * G, 2, 150, 150, causal=causal, seed=3)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


def test_offsets_fully_masked_rows_fp32_out():
    """q at positions 300.., k at 340..: the first 40 rows see nothing (O = 0, lse = -inf)."""
    srt = need_gpu()
    o, l, ro, rl = _run(srt, YARN_SMALL, 1, 4, 1, 130, 257, q_pos0=300, k_pos0=340, out_dtype=torch.float32)
    assert np.isneginf(l[:, :, :40]).all() and (o[:, :, :40] == 0).all()
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


def test_prerotated_k_and_rectangular():
    srt = need_gpu()
    o, l, ro, rl = _run(srt, ROPES[2], 1, 4, 1, 96, 320, q_pos0=400, k_pos0=100, prerotate_k=True, seed=9)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL
    o, l, ro, rl = _run(srt, ROPES[2], 1, 4, 1, 96, 320, q_pos0=400, k_pos0=100, causal=False, seed=9)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


def test_tiny_and_empty_keys():
    srt = need_gpu()
    o, l, ro, rl = _run(srt, ROPES[0], 1, 4, 4, 1, 1)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL
    q, k, v = qkv(1, 4, 1, 10, 0, 128, torch.bfloat16, 1)
    o, l = srt.attn_prefill(q, k, v, causal=False)
    assert (f64(o) == 0).all() and np.isneginf(f64(l)).all()


def test_repeat_is_bitwise_deterministic():
    """Same inputs twice -> identical bits (catches LDS races and unwritten tiles)."""
    srt = need_gpu()
    q, k, v = qkv(1, 8, 2, 700, 700, 128, torch.bfloat16, 4)
    table, _ = device_table(srt, YARN_SMALL, 128, 700)
    o1 = torch.full((1, 8, 700, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o1, l1 = srt.attn_prefill(q, k, v, table=table, out=o1)
    o2, l2 = srt.attn_prefill(q, k, v, table=table)
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# sm_scale * log2(e) = 1/8 exactly: the kernel's scaling of q is then a power
# of two (no rounding), so large scores stay comparable at the bf16 bar.
SM_POW2 = 0.125 * math.log(2.0)


def _plain(srt, q, k, v, causal):
    """q, k taken as already rotated (no table) against the oracle with no rotation."""
    o, l = srt.attn_prefill(q, k, v, causal=causal, sm_scale=SM_POW2)
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=SM_POW2, causal=causal)
    return f64(o), f64(l), ro, rl


@pytest.mark.parametrize("causal", [True, False])
def test_reference_moves_as_scores_grow(causal):
    """Key c is scaled by 1 + 5c/N, so the row maxima keep rising along the key
    walk (from ~7 to ~40 in log2 units) and the exponentials' reference must
    move several times; each move rescales O and the partial sums."""
    srt = need_gpu()
    N, D = 640, 128
    g = torch.Generator().manual_seed(11)
    q = (2.0 * torch.randn(1, 4, N, D, generator=g)).to(torch.bfloat16).cuda()
    ramp = 1.0 + 5.0 * torch.arange(N, dtype=torch.float32) / N
    k = (torch.randn(1, 1, N, D, generator=g) * ramp[None, None, :, None]).to(torch.bfloat16).cuda()
    v = torch.randn(1, 1, N, D, generator=g).to(torch.bfloat16).cuda()
    o, l, ro, rl = _plain(srt, q, k, v, causal)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL


@pytest.mark.parametrize("causal", [True, False])
def test_reference_far_below_zero(causal):
    """Every score is near -256 in log2 units: taken against the starting
    reference 0 the exponentials underflow to 0, so the first visible half of
    each row must set the reference from its maximum."""
    srt = need_gpu()
    N, D = 300, 128
    g = torch.Generator().manual_seed(12)
    q = (-4.0 * (1.0 + 0.1 * torch.randn(1, 4, N, D, generator=g))).to(torch.bfloat16).cuda()
    k = (4.0 * (1.0 + 0.1 * torch.randn(1, 2, N, D, generator=g))).to(torch.bfloat16).cuda()
    v = torch.randn(1, 2, N, D, generator=g).to(torch.bfloat16).cuda()
    o, l, ro, rl = _plain(srt, q, k, v, causal)
    assert np.all(rl < -150)
    assert max_abs(o, ro) <= TOL and max_abs(l, rl) <= TOL
