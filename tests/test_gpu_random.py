"""Seeded randomized parity of every attention entry point vs the fp64 oracle.

Each case draws its parameters from its own seed (printed before the GPU call,
so a failure names it): sizes with ragged tails, GQA groups, position offsets
that leave rows with no visible key, sliding windows with sinks, every RoPE
method or none, both pairings, K rotated on load or beforehand, sm_scale,
output dtype, lse on or off, views sliced along N.  The draws stay inside what
each entry point accepts, and bf16 draws keep sm_scale near the default
1/sqrt(D) (their error grows with the size of the scores); the bars are the
ones of the dedicated tests:
fp32 paths 1e-4, bf16 paths 2e-2 max-abs (a bf16 output of an fp32 path adds
its own rounding, at most 2^-8 |x|), backward bf16 2e-2 of each gradient's
scale."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import device_table, f64, max_abs, need_gpu, oracle_freq, qkv
from oracle import attention as A
from oracle import backward as BW
from oracle import ring as R
from oracle import rope as orope

pytestmark = pytest.mark.gpu

ROPES = [synth.Rope(synth.NONE, 10000.0), synth.Rope(synth.PI, 10000.0, 8.0),
         synth.Rope(synth.NTK, 10000.0, 8.0), synth.Rope(synth.YARN, 10000.0, 16.0, 64.0, 1.0, 32.0),
         synth.Rope(synth.YARN, 500000.0, 32.0, 128.0, 1.0, 32.0)]


def _say(kind, i, case):
    print(f"{kind} case {i}: {case}", flush=True)


def _sliced(t, rng):
    """Same values as t, but a view sliced along N out of a longer tensor."""
    B, H, N, D = t.shape
    a, b = int(rng.integers(0, 17)), int(rng.integers(0, 17))
    big = torch.zeros((B, H, a + N + b, D), dtype=t.dtype, device=t.device)
    big[:, :, a:a + N] = t
    return big[:, :, a:a + N]


def prefill_case(i):
    r = np.random.default_rng(7000 + i)
    bf16 = r.random() < 0.7
    D = 128 if bf16 else int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8, 12])) if bf16 else int(r.choice([1, 2, 3, 4]))
    c = dict(bf16=bf16, D=D, B=int(r.integers(1, 3)), Hkv=int(r.integers(1, 3)), G=G,
             Nq=int(r.integers(1, 330)), Nk=int(r.integers(0, 400)), causal=bool(r.random() < 0.8))
    c["q_pos0"] = int(r.integers(0, 400)) if r.random() < 0.5 else 0
    c["k_pos0"] = int(r.integers(0, 400)) if r.random() < 0.3 else 0
    c["window"] = int(r.integers(1, 260)) if c["causal"] and r.random() < 0.35 else 0
    c["sink"] = int(r.integers(0, 70)) if c["window"] and r.random() < 0.6 else 0
    c["rope"] = int(r.integers(0, len(ROPES) + 1))               # len(ROPES): no table
    c["half"] = bool(c["rope"] < len(ROPES) and r.random() < 0.4)
    c["prerotate_k"] = bool(c["rope"] < len(ROPES) and r.random() < 0.25)
    c["out_f32"] = bool(r.random() < 0.5)
    # The bf16 path's error grows with the size of the scores (its rotated
    # operands are rounded to bf16, which moves a score by about 2^-9 of the
    # product's magnitude): at 2.7x the default scale a row with a few visible
    # keys already reaches 0.03, and a CPU model of those roundings reaches the
    # same.  bf16 draws therefore stay near the default scale 1/sqrt(128); the
    # fp32 path takes larger scales.
    c["sm_scale"] = None if r.random() < 0.5 else float(r.uniform(0.03, 0.1 if bf16 else 0.25))
    c["lse"] = bool(r.random() < 0.85)
    c["sliced"] = bool(r.random() < 0.3)
    c["seed"] = int(r.integers(1, 1 << 20))
    return c


@pytest.mark.parametrize("i", range(48))
def test_prefill_random(i):
    srt = need_gpu()
    c = prefill_case(i)
    _say("prefill", i, c)
    r = np.random.default_rng(c["seed"])
    D, Hq = c["D"], c["G"] * c["Hkv"]
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    q, k, v = qkv(c["B"], Hq, c["Hkv"], c["Nq"], c["Nk"], D, dt, c["seed"])
    pairing = "half" if c["half"] else "interleaved"
    table, th, ms, flags = None, None, 1.0, 0
    if c["rope"] < len(ROPES):
        rp = ROPES[c["rope"]]
        table, _ = device_table(srt, rp, D, max(c["q_pos0"] + c["Nq"], c["k_pos0"] + c["Nk"], 1))
        th, ms, _ = oracle_freq(rp, D)
        flags = srt.ROTATE_Q | srt.ROTATE_K | (srt.PAIR_HALF if c["half"] else 0)
    kin = k
    if c["prerotate_k"]:
        kin = srt.rope_apply(k, table, pos0=c["k_pos0"], pairing=pairing)
        flags &= ~srt.ROTATE_K
    qin, vin = q, v
    if c["sliced"]:
        qin = _sliced(q, r)
        kv = _sliced(torch.stack([kin, v]).flatten(0, 1), r)       # k and v share a head stride
        kin, vin = kv[:c["B"]], kv[c["B"]:]
    out_dt = torch.float32 if c["out_f32"] else dt
    o, l = srt.attn_prefill(qin, kin, vin, sm_scale=c["sm_scale"], causal=c["causal"], q_pos0=c["q_pos0"],
                            k_pos0=c["k_pos0"], table=table, rope_flags=flags, out_dtype=out_dt, lse=c["lse"],
                            window=c["window"], sink=c["sink"])
    sm = 1 / math.sqrt(D) if c["sm_scale"] is None else c["sm_scale"]
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=sm, causal=c["causal"], q_pos0=c["q_pos0"],
                         k_pos0=c["k_pos0"], theta=th, mscale=ms, pairing=pairing, window=c["window"],
                         sink=c["sink"])
    o = f64(o)
    dead = np.isneginf(rl)
    print(f"  max|err| O {max_abs(o, ro):.3g}" + (f" lse {max_abs(f64(l), rl):.3g}" if c["lse"] else ""), flush=True)
    assert (o[dead] == 0).all()
    if c["bf16"]:
        assert max_abs(o, ro) <= 2e-2
    elif c["out_f32"]:
        assert max_abs(o, ro) <= 1e-4
    else:                                   # fp32 path, bf16 output: its rounding on top
        assert (np.abs(o - ro) <= 1e-4 + 2.0 ** -8 * (np.abs(ro) + 1e-4)).all()
    if c["lse"]:
        l = f64(l)
        assert np.array_equal(np.isneginf(l), dead)
        assert max_abs(l, rl) <= (2e-2 if c["bf16"] else 1e-4)
    else:
        assert l is None


def decode_case(i):
    r = np.random.default_rng(8000 + i)
    B = int(r.integers(1, 5))
    Nk = int(r.integers(1, 3000))
    c = dict(B=B, Hkv=int(r.integers(1, 3)), G=int(r.choice([1, 2, 4, 8])), Nk=Nk,
             splits=int(r.choice([1, 2, 7, 16, 64, 130])), rope=int(r.integers(0, len(ROPES) + 1)))
    c["half"] = bool(c["rope"] < len(ROPES) and r.random() < 0.4)
    if r.random() < 0.6:
        lens = r.integers(0, Nk + 1, size=B)
        lens[r.integers(0, B)] = Nk
        c["seq_lens"] = [int(x) for x in lens]
    else:
        c["seq_lens"] = None
    c["window"] = int(r.integers(1, 1500)) if r.random() < 0.35 else 0
    c["sink"] = int(r.integers(0, 40)) if c["window"] and r.random() < 0.6 else 0
    c["sm_scale"] = None if r.random() < 0.6 else float(r.uniform(0.03, 0.1))
    c["noalloc"] = bool(r.random() < 0.3)
    c["lse"] = bool(r.random() < 0.85)
    c["seed"] = int(r.integers(1, 1 << 20))
    return c


@pytest.mark.parametrize("i", range(24))
def test_decode_random(i):
    srt = need_gpu()
    c = decode_case(i)
    _say("decode", i, c)
    D, B, Hq, Hkv, Nk = 128, c["B"], c["G"] * c["Hkv"], c["Hkv"], c["Nk"]
    q = synth.randn((B, Hq, D), torch.bfloat16, c["seed"], synth.Q_ID, "cuda")
    k = synth.randn((B, Hkv, Nk, D), torch.bfloat16, c["seed"], synth.K_ID, "cuda")
    v = synth.randn((B, Hkv, Nk, D), torch.bfloat16, c["seed"], synth.V_ID, "cuda")
    pairing = "half" if c["half"] else "interleaved"
    table, th, ms, kc, kref = None, None, 1.0, k, f64(k)
    if c["rope"] < len(ROPES):
        rp = ROPES[c["rope"]]
        table, _ = device_table(srt, rp, D, Nk)
        th, ms, _ = oracle_freq(rp, D)
        kc = srt.rope_apply(k, table, pairing=pairing)
        rot = orope.rotate_half if c["half"] else orope.rotate
        kref = np.stack([rot(f64(k[b]), np.arange(Nk), th, ms) for b in range(B)])
    sl = None if c["seq_lens"] is None else torch.tensor(c["seq_lens"], dtype=torch.int32, device="cuda")
    call = srt.attn_decode_splitk_noalloc if c["noalloc"] else srt.attn_decode_splitk
    o, l = call(q, kc, v, num_splits=c["splits"], sm_scale=c["sm_scale"], table=table, seq_lens=sl,
                pairing=pairing, window=c["window"], sink=c["sink"], lse=c["lse"])
    sm = 1 / math.sqrt(D) if c["sm_scale"] is None else c["sm_scale"]
    ro, rl = A.decode(f64(q), kref, f64(v), sm_scale=sm, seq_lens=c["seq_lens"], theta=th, mscale=ms,
                      pairing=pairing, window=c["window"], sink=c["sink"])
    o = f64(o)
    print(f"  max|err| O {max_abs(o, ro):.3g}" + (f" lse {max_abs(f64(l), rl):.3g}" if c["lse"] else ""), flush=True)
    assert (o[np.isneginf(rl)] == 0).all()
    assert max_abs(o, ro) <= 2e-2
    if c["lse"]:
        assert max_abs(f64(l), rl) <= 1e-2


def ring_case(i):
    r = np.random.default_rng(9000 + i)
    bf16 = r.random() < 0.75
    mode = str(r.choice(["contiguous", "striped", "zigzag"]))
    P = int(r.choice([1, 2, 3, 4, 5, 8]))
    parts = 2 * P if mode == "zigzag" else P
    N = parts * int(r.integers(max(1, 48 // parts), 640 // parts + 1))
    c = dict(bf16=bf16, D=128 if bf16 else int(r.choice([64, 128])), mode=mode, P=P, N=N,
             B=int(r.integers(1, 3)), Hkv=int(r.integers(1, 3)),
             G=int(r.choice([1, 2, 4, 8])) if bf16 else int(r.choice([1, 2, 3])))
    c["window"] = int(r.integers(1, 300)) if mode != "striped" and r.random() < 0.35 else 0
    c["sink"] = int(r.integers(0, 50)) if c["window"] and r.random() < 0.6 else 0
    c["rope"] = int(r.integers(0, len(ROPES) + 1))
    c["half"] = bool(c["rope"] < len(ROPES) and r.random() < 0.4)
    c["prerotate_k"] = bool(c["rope"] < len(ROPES) and r.random() < 0.3)
    c["sm_scale"] = None if r.random() < 0.6 else float(r.uniform(0.03, 0.1 if bf16 else 0.25))
    c["device"] = -1 if r.random() < 0.7 else int(r.integers(0, P))
    c["seed"] = int(r.integers(1, 1 << 20))
    return c


@pytest.mark.parametrize("i", range(24))
def test_ring_random(i):
    srt = need_gpu()
    c = ring_case(i)
    _say("ring", i, c)
    D, N, P, Hq = c["D"], c["N"], c["P"], c["G"] * c["Hkv"]
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    q, k, v = qkv(c["B"], Hq, c["Hkv"], N, N, D, dt, c["seed"])
    pos = R.partition_positions(N, P, c["mode"])
    ip = torch.from_numpy(pos).cuda()
    pairing = "half" if c["half"] else "interleaved"
    table, th, ms, flags = None, None, 1.0, 0
    if c["rope"] < len(ROPES):
        rp = ROPES[c["rope"]]
        table, _ = device_table(srt, rp, D, N)
        th, ms, _ = oracle_freq(rp, D)
        flags = srt.ROTATE_Q | srt.ROTATE_K | (srt.PAIR_HALF if c["half"] else 0)
    kin = k
    if c["prerotate_k"]:
        kin = srt.rope_apply(k, table, pairing=pairing)
        flags &= ~srt.ROTATE_K
    qs, ks, vs = (t.index_select(2, ip).contiguous() for t in (q, kin, v))
    o = torch.full_like(qs, float("nan"))
    l = torch.full((c["B"], Hq, N), float("nan"), device="cuda")
    srt.attn_ring_prefill(qs, ks, vs, num_devices=P, partition=c["mode"], device=c["device"], window=c["window"],
                          sink=c["sink"], sm_scale=c["sm_scale"], table=table, rope_flags=flags, out=o, lse=l)
    sm = 1 / math.sqrt(D) if c["sm_scale"] is None else c["sm_scale"]
    ro, rl = A.attention(f64(q), f64(k), f64(v), sm_scale=sm, theta=th, mscale=ms, pairing=pairing,
                         window=c["window"], sink=c["sink"])
    ro, rl = ro[:, :, pos], rl[:, :, pos]
    o, l = f64(o), f64(l)
    C = N // P
    if c["device"] >= 0:                    # only that device's rows are written
        rows = slice(c["device"] * C, (c["device"] + 1) * C)
        keep = np.zeros(N, dtype=bool)
        keep[rows] = True
        assert np.isnan(o[:, :, ~keep]).all() and np.isnan(l[:, :, ~keep]).all()
        o, l, ro, rl = o[:, :, rows], l[:, :, rows], ro[:, :, rows], rl[:, :, rows]
    tol = 2e-2 if c["bf16"] else 1e-4
    print(f"  max|err| O {max_abs(o, ro):.3g} lse {max_abs(l, rl):.3g}", flush=True)
    assert max_abs(o, ro) <= tol and max_abs(l, rl) <= tol


def merge_case(i):
    r = np.random.default_rng(9500 + i)
    c = dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 5)), N=int(r.integers(0, 300)),
             D=int(r.choice([8, 16, 32, 64, 128, 256, 512])), in_f32=bool(r.random() < 0.6))
    c["out_f32"] = bool(c["in_f32"] and r.random() < 0.6)
    c["in_place"] = bool(c["in_f32"] == c["out_f32"] and r.random() < 0.4)
    c["dead_a"], c["dead_b"] = int(r.integers(2, 9)), int(r.integers(2, 9))
    c["lse_scale"] = float(r.choice([1.0, 4.0, 30.0]))
    c["seed"] = int(r.integers(1, 1 << 20))
    return c


@pytest.mark.parametrize("i", range(16))
def test_merge_random(i):
    srt = need_gpu()
    c = merge_case(i)
    _say("merge", i, c)
    g = torch.Generator(device="cpu").manual_seed(c["seed"])
    shape = (c["B"], c["H"], c["N"], c["D"])
    in_dt = torch.float32 if c["in_f32"] else torch.bfloat16
    oa = torch.randn(shape, generator=g).to(in_dt).cuda()
    ob = torch.randn(shape, generator=g).to(in_dt).cuda()
    la = (torch.randn(shape[:3], generator=g) * c["lse_scale"]).cuda()
    lb = (torch.randn(shape[:3], generator=g) * c["lse_scale"]).cuda()
    la[..., ::c["dead_a"]] = -float("inf")
    lb[..., ::c["dead_b"]] = -float("inf")
    ro, rl = A.merge(f64(oa), f64(la), f64(ob), f64(lb))
    out_dt = torch.float32 if c["out_f32"] else torch.bfloat16
    if c["in_place"]:
        o, l = srt.attn_merge_states(oa, la, ob, lb, out=oa, lse_out=la)
        assert o.data_ptr() == oa.data_ptr()
    else:
        o, l = srt.attn_merge_states(oa, la, ob, lb, out_dtype=out_dt)
    o, l = f64(o), f64(l)
    print(f"  max|err| O {max_abs(o, ro):.3g} lse {max_abs(l, rl):.3g}", flush=True)
    assert max_abs(o, ro) <= (1e-5 if c["out_f32"] else 2e-2)
    assert max_abs(l, rl) <= 1e-5 * max(1.0, c["lse_scale"])
    assert np.array_equal(np.isneginf(l), np.isneginf(rl))
    assert (o[np.isneginf(rl)] == 0).all()


def backward_case(i):
    r = np.random.default_rng(9800 + i)
    bf16 = r.random() < 0.6
    c = dict(bf16=bf16, D=128 if bf16 else 64, B=int(r.integers(1, 3)), Hkv=int(r.integers(1, 3)),
             G=int(r.choice([1, 2, 4, 8])) if bf16 else int(r.choice([1, 2, 3])),
             Nq=int(r.integers(1, 200)), Nk=int(r.integers(1, 240)), causal=bool(r.random() < 0.8))
    c["q_pos0"] = int(r.integers(0, 200)) if r.random() < 0.4 else 0
    c["k_pos0"] = int(r.integers(0, 200)) if r.random() < 0.3 else 0
    c["window"] = int(r.integers(1, 150)) if c["causal"] and r.random() < 0.35 else 0
    c["sink"] = int(r.integers(0, 40)) if c["window"] and r.random() < 0.6 else 0
    c["rope"] = int(r.integers(0, len(ROPES) + 1))
    c["half"] = bool(c["rope"] < len(ROPES) and r.random() < 0.4)
    c["flags"] = int(r.choice([3, 3, 1, 2])) if c["rope"] < len(ROPES) else 0    # rotate q and/or k
    c["sm_scale"] = None if r.random() < 0.6 else float(r.uniform(0.03, 0.1 if bf16 else 0.25))
    c["seed"] = int(r.integers(1, 1 << 20))
    return c


def _backward_one_side(q, k, v, do, sm, th, ms, pairing, flags, kw):
    """Reference when the kernel rotates only q or only k: the oracle's backward
    on the rotated side's values, its gradient turned back by the transposed
    rotation (d raw = mscale R^T d rotated)."""
    rot = orope.rotate_half if pairing == "half" else orope.rotate
    qpos = kw["q_pos0"] + np.arange(q.shape[2])
    kpos = kw["k_pos0"] + np.arange(k.shape[2])
    qq = rot(f64(q), qpos, th, ms) if flags & 1 else f64(q)
    kk = rot(f64(k), kpos, th, ms) if flags & 2 else f64(k)
    dq, dk, dv, _ = BW.attention_backward(qq, kk, f64(v), f64(do), sm_scale=sm, theta=None, **kw)
    if flags & 1:
        dq = BW.rotate_back(dq, qpos, th, ms, pairing)
    if flags & 2:
        dk = BW.rotate_back(dk, kpos, th, ms, pairing)
    return dq, dk, dv


@pytest.mark.parametrize("i", range(16))
def test_backward_random(i):
    srt = need_gpu()
    c = backward_case(i)
    _say("backward", i, c)
    D, Hq = c["D"], c["G"] * c["Hkv"]
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    q, k, v = qkv(c["B"], Hq, c["Hkv"], c["Nq"], c["Nk"], D, dt, c["seed"])
    do = synth.randn((c["B"], Hq, c["Nq"], D), dt, c["seed"], synth.DO_ID, "cuda")
    pairing = "half" if c["half"] else "interleaved"
    table, th, ms, flags = None, None, 1.0, 0
    if c["rope"] < len(ROPES):
        rp = ROPES[c["rope"]]
        table, _ = device_table(srt, rp, D, max(c["q_pos0"] + c["Nq"], c["k_pos0"] + c["Nk"]))
        th, ms, _ = oracle_freq(rp, D)
        flags = c["flags"] | (srt.PAIR_HALF if c["half"] else 0)
    kw = dict(causal=c["causal"], q_pos0=c["q_pos0"], k_pos0=c["k_pos0"], window=c["window"], sink=c["sink"])
    sm = 1 / math.sqrt(D) if c["sm_scale"] is None else c["sm_scale"]
    o, l = srt.attn_prefill(q, k, v, table=table, rope_flags=flags, sm_scale=sm, **kw)
    dq, dk, dv = srt.attn_backward(q, k, v, o, do, l, table=table, rope_flags=flags, sm_scale=sm, **kw)
    # the oracle rotates both or neither: a side the kernel does not rotate
    # enters the oracle as the same values with a zero-frequency table (identity)
    if (flags & 3) in (0, 3):
        got = BW.attention_backward(f64(q), f64(k), f64(v), f64(do), sm_scale=sm, theta=th if flags else None,
                                    mscale=ms, pairing=pairing, **kw)
    else:
        got = _backward_one_side(q, k, v, do, sm, th, ms, pairing, flags, kw)
    ref = got[:3]
    res = (f64(dq), f64(dk), f64(dv))
    print("  max|err| / scale " + " ".join(
        f"{n_} {max_abs(g_, r_) / max(1.0, float(np.abs(r_).max())):.3g}" for n_, g_, r_ in zip(("dq", "dk", "dv"), res, ref)),
        flush=True)
    for g_, r_ in zip(res, ref):
        scale = max(1.0, float(np.abs(r_).max())) if r_.size else 1.0
        assert max_abs(g_, r_) <= (2e-2 * scale if c["bf16"] else 1e-4 * scale)
