"""GPU parity of srt_attn_backward (dq, dk, dv) vs the fp64 oracle.

The forward pass (srt_attn_prefill) supplies out and lse; the oracle
recomputes everything in fp64 from the same inputs.  Bars: fp32 kernels
1e-4 max-abs; bf16 kernels 2e-2 max-abs after each gradient is scaled to its
largest entry (max|err| <= 2e-2 max(1, max|ref|)).  The gradients reach ~10
here (dv of an early key sums P dO over every later query), and the bf16
kernels round rotated q~, k~ (so S moves by ~2^-8 |S| and P with it), P and
dS: errors are a fixed fraction of the gradient's scale, not of 1.
Cases span several tiles, a ragged tail, GQA 1/2/4/8, both pairings, windows
and sinks, offsets with fully masked rows, non-causal, inputs used as given."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import backward as BW
from oracle import rope as orope

pytestmark = pytest.mark.gpu

YARN_SMALL = synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0)


def _run(srt, *, dtype, D, B=1, Hq=4, Hkv=2, Nq=150, Nk=150, q_pos0=0, k_pos0=0, causal=True, window=0, sink=0,
         half=False, rotate=True, seed=51, sm_scale=None):
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, D, dtype, seed)
    do = synth.randn((B, Hq, Nq, D), dtype, seed, synth.DO_ID, "cuda")
    table, _ = device_table(srt, YARN_SMALL, D, max(q_pos0 + Nq, k_pos0 + Nk, 1))
    th, ms, _ = oracle_freq(YARN_SMALL, D)
    pairing = "half" if half else "interleaved"
    if rotate:
        flags = srt.ROTATE_Q | srt.ROTATE_K | (srt.PAIR_HALF if half else 0)
    else:                                   # inputs already rotated, used as given
        q = srt.rope_apply(q, table, pos0=q_pos0, pairing=pairing)
        k = srt.rope_apply(k, table, pos0=k_pos0, pairing=pairing)
        flags = 0
    kw = dict(causal=causal, q_pos0=q_pos0, k_pos0=k_pos0, window=window, sink=sink)
    sm = 1 / math.sqrt(D) if sm_scale is None else sm_scale
    o, l = srt.attn_prefill(q, k, v, table=table, rope_flags=flags, sm_scale=sm, **kw)
    dq, dk, dv = srt.attn_backward(q, k, v, o, do, l, table=table, rope_flags=flags, sm_scale=sm, **kw)
    rq, rk, rv, _ = BW.attention_backward(f64(q), f64(k), f64(v), f64(do), sm_scale=sm,
                                          theta=th if rotate else None, mscale=ms, pairing=pairing, **kw)
    return (f64(dq), f64(dk), f64(dv)), (rq, rk, rv)


def _err(got, ref):
    return max(max_abs(g, r) for g, r in zip(got, ref))


def _rel_err(got, ref):
    """max|err| of each gradient over max(1, its largest reference entry)."""
    return max(max_abs(g, r) / max(1.0, float(np.abs(r).max())) for g, r in zip(got, ref))


def _report(tag, got, ref):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        e = max_abs(g, r)
        print(f"{tag} {name}: max|err| {e:.3g}  max|ref| {np.abs(r).max():.3g}  rms err {np.sqrt(np.mean((g - r) ** 2)):.3g}",
              flush=True)


@pytest.mark.parametrize("kw", [dict(), dict(half=True), dict(window=40, sink=4), dict(q_pos0=300, k_pos0=340),
                                dict(causal=False), dict(rotate=False)],
                         ids=["plain", "half", "window", "offsets", "noncausal", "given"])
def test_backward_fp32(kw):
    srt = need_gpu()
    got, ref = _run(srt, dtype=torch.float32, D=64, **kw)
    assert _err(got, ref) <= 1e-4


@pytest.mark.parametrize("kw", [dict(), dict(half=True), dict(window=100, sink=4), dict(window=70, sink=90),
                                dict(q_pos0=300, k_pos0=340, Nq=130, Nk=257), dict(causal=False),
                                dict(rotate=False), dict(B=2, Nq=64, Nk=64), dict(sm_scale=0.03),
                                dict(sm_scale=0.2, rotate=False, Nq=96, Nk=96),
                                dict(window=64, sink=5, q_pos0=200, k_pos0=0, Nq=170, Nk=370, half=True)],
                         ids=["plain", "half", "window", "wide_sink", "offsets", "noncausal", "given", "batch",
                              "scale_small", "scale_large_given", "window_offsets_half"])
def test_backward_bf16(kw):
    srt = need_gpu()
    base = dict(Nq=300, Nk=300)
    base.update(kw)
    got, ref = _run(srt, dtype=torch.bfloat16, D=128, Hq=8, Hkv=2, **base)
    _report(f"bf16 {kw}", got, ref)
    assert _rel_err(got, ref) <= 2e-2


@pytest.mark.parametrize("G", [1, 2, 8])
def test_backward_bf16_group_sizes(G):
    srt = need_gpu()
    got, ref = _run(srt, dtype=torch.bfloat16, D=128, Hq=G * (2 if G < 8 else 1), Hkv=2 if G < 8 else 1, Nq=200,
                    Nk=200, seed=52)
    _report(f"bf16 G={G}", got, ref)
    assert _rel_err(got, ref) <= 2e-2


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("G,Nq", [(1, 1), (1, 32), (1, 64), (1, 96), (1, 128), (1, 160), (2, 96), (2, 160), (4, 33),
                                  (4, 96), (4, 161), (8, 96)])
def test_backward_bf16_tile_counts(G, Nq, causal):
    """Every residue of the query-tile count a dk/dv workgroup walks (1 to 5
    tiles of one head, several heads), including a single query row."""
    srt = need_gpu()
    got, ref = _run(srt, dtype=torch.bfloat16, D=128, Hq=G, Hkv=1, Nq=Nq, Nk=max(Nq, 96), causal=causal,
                    q_pos0=max(0, 96 - Nq) if causal else 0, seed=55)
    _report(f"bf16 G={G} Nq={Nq} causal={causal}", got, ref)
    assert _rel_err(got, ref) <= 2e-2


def test_backward_bf16_2k():
    """2048 tokens, GQA 8/2: many tiles in both kernels."""
    srt = need_gpu()
    got, ref = _run(srt, dtype=torch.bfloat16, D=128, Hq=8, Hkv=2, Nq=2048, Nk=2048, seed=53)
    _report("bf16 2K", got, ref)
    assert _rel_err(got, ref) <= 2e-2


def test_backward_empty():
    srt = need_gpu()
    D = 128
    q, k, v = qkv(1, 4, 1, 0, 64, D, torch.bfloat16, 54)
    o = torch.empty_like(q)
    l = torch.empty((1, 4, 0), device="cuda")
    dk = torch.full(k.shape, float("nan"), device="cuda")
    dv = torch.full(v.shape, float("nan"), device="cuda")
    _, dk, dv = srt.attn_backward(q, k, v, o, o, l, dk=dk, dv=dv)
    assert (dk == 0).all() and (dv == 0).all()


def test_backward_yarn_32k_full_size_sampled():
    """The benchmark's backward launch at full size (YaRN 32K, GQA 32/8, D=128): dq at sampled query rows
    of every query head of the first and last KV group, dk and dv at the last 48 keys of those KV heads
    (few rows see them, so the oracle forms exactly those rows of P), each against the oracle at those
    entries; and, for each of the two KV heads, the sum of dv over all keys equals the sum of dO over the
    group's rows (every row of P sums to one)."""
    srt = need_gpu()
    w = synth.WORKLOADS["yarn_32k_bf16"]
    D, N, G = w.D, w.N, w.Hq // w.Hkv
    q = synth.randn((w.B, w.Hq, N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    do = synth.randn((w.B, w.Hq, N, D), torch.bfloat16, w.seed, synth.DO_ID, "cuda")
    table, _ = device_table(srt, w.rope, D, N)
    out, lse = srt.attn_prefill(q, k, v, table=table)                     # as the benchmark
    dq, dk, dv = srt.attn_backward(q, k, v, out, do, lse, table=table)
    torch.cuda.synchronize()
    th, ms, _ = oracle_freq(w.rope, D)
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 4095, N // 2, N - 2, N - 1], rng.integers(0, N, 7)]))
    keys = np.arange(N - 48, N)
    worst = 0.0
    for hk in (0, w.Hkv - 1):
        hs = slice(hk * G, (hk + 1) * G)
        rdq, rdk, rdv = BW.attention_backward_sampled(
            f64(q[:, hs]), f64(k[:, hk:hk + 1]), f64(v[:, hk:hk + 1]), f64(do[:, hs]), hk=0, rows=rows, keys=keys,
            sm_scale=1 / math.sqrt(D), theta=th, mscale=ms)
        got_dq = f64(dq[0, hs][:, torch.as_tensor(rows, device="cuda")])
        got_dk = f64(dk[0, hk][torch.as_tensor(keys, device="cuda")])
        got_dv = f64(dv[0, hk][torch.as_tensor(keys, device="cuda")])
        for name, g, r in (("dq", got_dq, rdq), ("dk", got_dk, rdk), ("dv", got_dv, rdv)):
            # dk, dv of the last keys are small (few rows see them): judged against their own scale
            scale = max(1.0, float(np.abs(r).max())) if name == "dq" else float(np.abs(r).max())
            e = max_abs(g, r) / scale
            print(f"32K kv head {hk} {name}: max|err| {max_abs(g, r):.3g} max|ref| {np.abs(r).max():.3g}", flush=True)
            worst = max(worst, e)
        dv_sum = f64(dv[0, hk].sum(dim=0))
        do_sum = f64(do[0, hs].float().sum(dim=(0, 1)))
        rel = max_abs(dv_sum, do_sum) / float(np.abs(do_sum).max())
        print(f"32K kv head {hk}: sum dv vs sum dO rel err {rel:.3g}", flush=True)
        assert rel <= 1e-2
    assert worst <= 2e-2


def test_backward_window_sinks_two_batches_sampled():
    """A window of 512 keys with 4 sinks at GQA 32/8, two batches of 4096 (so both kernels take their items
    through the run-time queues): dq at sampled rows of every query head of the first and last KV group of
    each batch, dk and dv at the keys just past the sinks and at the last keys, against the oracle at those
    entries."""
    srt = need_gpu()
    B, Hq, Hkv, N, D, W, S = 2, 32, 8, 4096, 128, 512, 4
    G = Hq // Hkv
    rope = synth.WORKLOADS["yarn_32k_bf16"].rope
    q, k, v = qkv(B, Hq, Hkv, N, N, D, torch.bfloat16, 57)
    do = synth.randn((B, Hq, N, D), torch.bfloat16, 57, synth.DO_ID, "cuda")
    table, _ = device_table(srt, rope, D, N)
    out, lse = srt.attn_prefill(q, k, v, table=table, window=W, sink=S)
    dq, dk, dv = srt.attn_backward(q, k, v, out, do, lse, table=table, window=W, sink=S)
    torch.cuda.synchronize()
    th, ms, _ = oracle_freq(rope, D)
    rng = np.random.default_rng(57)
    rows = np.unique(np.concatenate([[0, 3, 4, 31, 32, 63, 64, W - 1, W, W + 1, W + 4, 2047, N - 2, N - 1],
                                     rng.integers(0, N, 6)]))
    keys = np.concatenate([np.arange(S, S + 8), np.arange(N - 16, N)])
    worst = 0.0
    for b in range(B):
        for hk in (0, Hkv - 1):
            hs = slice(hk * G, (hk + 1) * G)
            rdq, rdk, rdv = BW.attention_backward_sampled(
                f64(q[:, hs]), f64(k[:, hk:hk + 1]), f64(v[:, hk:hk + 1]), f64(do[:, hs]), hk=0, rows=rows,
                keys=keys, sm_scale=1 / math.sqrt(D), theta=th, mscale=ms, window=W, sink=S, b=b)
            got_dq = f64(dq[b, hs][:, torch.as_tensor(rows, device="cuda")])
            got_dk = f64(dk[b, hk][torch.as_tensor(keys, device="cuda")])
            got_dv = f64(dv[b, hk][torch.as_tensor(keys, device="cuda")])
            for name, g, r in (("dq", got_dq, rdq), ("dk", got_dk, rdk), ("dv", got_dv, rdv)):
                scale = max(1.0, float(np.abs(r).max())) if name == "dq" else float(np.abs(r).max())
                e = max_abs(g, r) / scale
                print(f"window b {b} kv head {hk} {name}: max|err| {max_abs(g, r):.3g} max|ref| {np.abs(r).max():.3g}",
                      flush=True)
                worst = max(worst, e)
    assert worst <= 2e-2


@pytest.mark.parametrize("rotate", [False, True], ids=["given", "rotated"])
def test_backward_recomputes_the_forward_softmax(rotate):
    """With a one-key window every query sees only its own position, so the
    forward's weight is exactly 1: dv of a key is the sum of its group's dO
    and dq = dk = 0.  At sm_scale = 0.5 the scores reach about 30 in log2
    units, where a backward that rounded q * sm_scale log2(e) differently from
    the forward would be off by about 2^-9 of that (4 %).  The backward must
    recompute the forward's own P (given q: kept exact on both sides; rotated
    q: the same one bf16 rounding on both sides)."""
    srt = need_gpu()
    B, Hq, Hkv, N, D = 1, 8, 2, 256, 128
    q, k, v = qkv(B, Hq, Hkv, N, N, D, torch.bfloat16, 61)
    do = synth.randn((B, Hq, N, D), torch.bfloat16, 61, synth.DO_ID, "cuda")
    table, _ = device_table(srt, YARN_SMALL, D, N)
    flags = (srt.ROTATE_Q | srt.ROTATE_K) if rotate else 0
    kw = dict(table=table, rope_flags=flags, sm_scale=0.5, window=1)
    o, l = srt.attn_prefill(q, k, v, **kw)
    dq, dk, dv = srt.attn_backward(q, k, v, o, do, l, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, v.repeat_interleave(Hq // Hkv, dim=1))
    want = do.float().reshape(B, Hkv, Hq // Hkv, N, D).sum(dim=2)
    err = float((dv - want).abs().max())
    print(f"rotate={rotate}: |dv - sum dO| {err:.3g}, |dq| {float(dq.abs().max()):.3g}, |dk| {float(dk.abs().max()):.3g}",
          flush=True)
    assert err <= 1e-4 * float(want.abs().max())
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3
