"""GPU parity: log-sum-exp merge of partial states vs the fp64 oracle."""
import numpy as np
import pytest
import torch

from gpu_helpers import f64, max_abs, need_gpu
from oracle import attention as A

pytestmark = pytest.mark.gpu


def _states(B, H, N, D, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    oa = torch.randn((B, H, N, D), generator=g).to(dtype).cuda()
    ob = torch.randn((B, H, N, D), generator=g).to(dtype).cuda()
    la = (torch.randn((B, H, N), generator=g) * 4).cuda()
    lb = (torch.randn((B, H, N), generator=g) * 4).cuda()
    la[..., ::7] = -float("inf")            # rows with no visible key in part a
    lb[..., ::5] = -float("inf")            # ... in part b; rows 0, 35, ... in both
    return oa, la, ob, lb


@pytest.mark.parametrize("in_dt,out_dt", [(torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                                          (torch.bfloat16, torch.bfloat16)])
def test_merge_matches_oracle(in_dt, out_dt):
    srt = need_gpu()
    oa, la, ob, lb = _states(2, 3, 333, 128, in_dt, 5)
    o, l = srt.attn_merge_states(oa, la, ob, lb, out_dtype=out_dt)
    ro, rl = A.merge(f64(oa), f64(la), f64(ob), f64(lb))
    tol = 1e-5 if out_dt == torch.float32 else 2e-2
    assert max_abs(f64(o), ro) <= tol
    assert max_abs(f64(l), rl) <= 1e-5
    assert np.array_equal(np.isneginf(f64(l)), np.isneginf(rl))
    both = (np.isneginf(f64(la)) & np.isneginf(f64(lb)))
    assert (f64(o)[both] == 0).all()


def test_merge_in_place_and_strided_out():
    srt = need_gpu()
    oa, la, ob, lb = _states(1, 4, 100, 64, torch.float32, 9)
    ro, rl = A.merge(f64(oa), f64(la), f64(ob), f64(lb))
    srt.attn_merge_states(oa, la, ob, lb, out=oa, lse_out=la)
    assert max_abs(f64(oa), ro) <= 1e-5 and max_abs(f64(la), rl) <= 1e-5
    big = torch.zeros((1, 4, 300, 64), device="cuda", dtype=torch.bfloat16)
    biglse = torch.zeros((1, 4, 300), device="cuda")
    oa2, la2, ob2, lb2 = _states(1, 4, 100, 64, torch.float32, 9)
    srt.attn_merge_states(oa2, la2, ob2, lb2, out=big[:, :, 100:200], lse_out=biglse[:, :, 100:200])
    assert max_abs(f64(big[:, :, 100:200]), ro) <= 2e-2
    assert (f64(big[:, :, :100]) == 0).all() and (f64(big[:, :, 200:]) == 0).all()
    assert max_abs(f64(biglse[:, :, 100:200]), rl) <= 1e-5
