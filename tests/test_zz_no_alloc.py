"""The allocation-free decode entry point (srt_attn_decode_splitk_noalloc),
called through the C ABI, against srt_attn_decode_splitk with a caller
workspace: the same kernels on the same inputs, so the outputs must agree bit
for bit.  Two calls in a row, the second on a smaller problem (fewer
sequences, fewer splits, a shorter cache), check that the static scratch
carries nothing from one call into the next; the last case is the 128K decode
workload's own shape (16.9 MB of partials)."""
import ctypes as C
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq
from oracle import attention as A
from oracle import rope as orope

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, N, seed):
    q = synth.randn((B, Hq, 128), torch.bfloat16, seed, synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, N, 128), torch.bfloat16, seed, synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, N, 128), torch.bfloat16, seed, synth.V_ID, "cuda")
    return q, k, v


def _noalloc_abi(srt, q, kc, v, splits, table, seq_lens=None):
    """srt_attn_decode_splitk_noalloc called directly through ctypes."""
    lib = srt.lib()
    B, Hq, D = q.shape
    _, Hkv, Nk, _ = kc.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    st = lib.srt_attn_decode_splitk_noalloc(
        C.c_void_p(q.data_ptr()), C.c_void_p(kc.data_ptr()), C.c_void_p(v.data_ptr()), srt.BF16, B, Hq, Hkv, Nk, D,
        None if seq_lens is None else C.c_void_p(seq_lens.data_ptr()), splits, 1.0 / math.sqrt(D),
        C.c_void_p(table.data_ptr()), table.shape[0], 0, 0, 0, C.c_void_p(out.data_ptr()),
        C.c_void_p(lse.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.srt_last_error()
    return out, lse


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, N, splits, seed): a large call, then a smaller one on the same scratch
    ((8, 32, 8, 4096, 64, 21), (3, 16, 4, 1000, 7, 22)),
    ((16, 32, 8, 131072, 64, 5), (2, 8, 8, 300, 3, 23)),
])
def test_noalloc_matches_workspace_entry_point(case):
    srt = need_gpu()
    rp = synth.Rope(synth.PI, 10000.0, 16.0)
    for (B, Hq, Hkv, N, splits, seed) in case:
        print(f"noalloc decode B={B} Hq={Hq} Hkv={Hkv} N={N} splits={splits}", flush=True)
        q, k, v = _inputs(B, Hq, Hkv, N, seed)
        table, _ = device_table(srt, rp, 128, N)
        kc = srt.rope_apply(k, table)
        seq_lens = torch.tensor([N - (7 * b) % max(1, N // 3) for b in range(B)], dtype=torch.int32, device="cuda")
        o_ref, l_ref = srt.attn_decode_splitk(q, kc, v, num_splits=splits, table=table, seq_lens=seq_lens)
        o, l = _noalloc_abi(srt, q, kc, v, splits, table, seq_lens)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
        # and to the oracle's bar on the first sequence
        th, ms, _ = oracle_freq(rp, 128)
        n = int(seq_lens[0])
        G = Hq // Hkv
        kr = orope.rotate(f64(k[0, 0, :n]), np.arange(n), th, ms)
        ro, rl = A.decode(f64(q[0:1, :G]), kr[None, None], f64(v[0, 0, :n])[None, None],
                          sm_scale=1 / math.sqrt(128), theta=th, mscale=ms)
        assert max_abs(f64(o[0, :G]), ro[0]) <= 2e-2 and max_abs(f64(l[0, :G]), rl[0]) <= 2e-2
        del q, k, v, kc
        torch.cuda.empty_cache()
