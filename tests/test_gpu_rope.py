"""GPU parity: cos/sin table and standalone rotation vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq
from oracle import rope as orope

pytestmark = pytest.mark.gpu

ROPES = [synth.Rope(synth.NONE, 10000.0), synth.Rope(synth.NONE, 500000.0), synth.Rope(synth.PI, 10000.0, 16.0),
         synth.Rope(synth.NTK, 10000.0, 16.0), synth.Rope(synth.YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0)]


@pytest.mark.parametrize("rp", ROPES, ids=lambda r: f"m{r.method}_b{int(r.base)}")
@pytest.mark.parametrize("D", [64, 128])
def test_table_matches_fp64(rp, D):
    """Entry (p, i) = mscale (cos, sin)(p theta'_i); fp64 angle, one fp32 rounding: error <= 1 ulp-ish."""
    srt = need_gpu()
    npos = 131072
    table, ms = device_table(srt, rp, D, npos)
    th, oms, _ = oracle_freq(rp, D)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(npos - 64, npos),
                                     np.random.default_rng(0).integers(0, npos, 512)]))
    got = table[torch.from_numpy(rows).cuda()].cpu().double().numpy()
    a = rows[:, None] * th[None, :]
    ref = np.stack([oms * np.cos(a), oms * np.sin(a)], axis=-1)
    assert max_abs(got, ref) <= 2.0 ** -23 * oms * 1.01


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_rope_apply_matches_oracle(dtype, D):
    srt = need_gpu()
    rp = synth.Rope(synth.YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0)
    B, H, N, pos0 = 2, 3, 301, 777
    x = synth.randn((B, H, N, D), dtype, 11, 0, "cuda")
    table, _ = device_table(srt, rp, D, pos0 + N)
    y = srt.rope_apply(x, table, pos0=pos0)
    th, ms, _ = oracle_freq(rp, D)
    ref = orope.rotate(f64(x), pos0 + np.arange(N), th, ms)
    got = f64(y)
    if dtype == torch.float32:
        assert max_abs(got, ref) <= 1e-5
    else:
        # one bf16 rounding of the result: |err| <= 2^-9 |y| (+ fp32 slack)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    # in place gives the same bits
    x2 = x.clone()
    srt.rope_apply(x2, table, pos0=pos0, out=x2)
    assert torch.equal(x2, y)


def test_rope_apply_empty_and_position_errors():
    srt = need_gpu()
    table, _ = device_table(srt, synth.Rope(), 64, 10)
    x = torch.zeros((1, 1, 0, 64), device="cuda")
    assert srt.rope_apply(x, table).shape == x.shape
    from scaled_rope_tiled_amd._lib import SrtError
    with pytest.raises(SrtError):
        srt.rope_apply(torch.zeros((1, 1, 11, 64), device="cuda"), table)
