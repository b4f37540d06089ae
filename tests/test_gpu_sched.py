"""GPU tests of the prefill kernel's run-time work assignment (the scheduling
block of srt_attn_prefill).

The assignment only changes which workgroup computes which (head, query tile)
item, never the arithmetic of an item, so the output with a scheduling block
must be bit-identical to the fixed assignment's; the block must be zero-filled
again when the call returns; and calls on two streams with their own blocks
must not disturb each other.  The shapes have more than two workgroups per
compute unit (below that the launcher keeps the fixed assignment): GQA 4, 1
and 8 (workgroup heads 8, 32 and 16), two batches, non-causal, a window with
sinks, and three KV heads (five of the eight XCD queues empty).  Parity of
the same launches with the oracle is covered at full size by the workload
tests, which run with the default block."""
import pytest
import torch

import synth
from gpu_helpers import device_table, need_gpu, qkv

pytestmark = pytest.mark.gpu

YARN = synth.Rope(synth.YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0)
CASES = [
    dict(B=1, Hq=32, Hkv=8, N=8192),
    dict(B=1, Hq=32, Hkv=32, N=8192),
    dict(B=1, Hq=64, Hkv=8, N=4096),
    dict(B=2, Hq=32, Hkv=8, N=4096),
    dict(B=1, Hq=32, Hkv=8, N=8192, causal=False),
    dict(B=1, Hq=32, Hkv=8, N=8192, window=1024, sink=4),
    dict(B=1, Hq=6, Hkv=3, N=32768),
]


def _ids(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


def _inputs(srt, c, seed=11):
    q, k, v = qkv(c["B"], c["Hq"], c["Hkv"], c["N"], c["N"], 128, torch.bfloat16, seed)
    table, _ = device_table(srt, YARN, 128, c["N"])
    kr = srt.rope_apply(k, table)
    kw = dict(causal=c.get("causal", True), window=c.get("window", 0), sink=c.get("sink", 0), table=table,
              rope_flags=srt.ROTATE_Q)
    return q, kr, v, kw


@pytest.mark.parametrize("c", CASES, ids=_ids)
def test_run_time_assignment_is_bit_identical(c):
    srt = need_gpu()
    print("case", c, flush=True)
    q, kr, v, kw = _inputs(srt, c)
    o_fix, l_fix = srt.attn_prefill(q, kr, v, sched=False, **kw)
    blk = torch.zeros(srt.PREFILL_SCHED_BYTES, dtype=torch.uint8, device="cuda")
    for rep in range(2):                     # the block comes back zero-filled and serves the next call
        o, l = srt.attn_prefill(q, kr, v, sched=blk, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, o_fix) and torch.equal(l, l_fix), rep
        assert int(blk.count_nonzero()) == 0, rep


def test_default_block_per_stream_left_zero():
    srt = need_gpu()
    c = CASES[0]
    q, kr, v, kw = _inputs(srt, c)
    o_fix, _ = srt.attn_prefill(q, kr, v, sched=False, **kw)
    o, _ = srt.attn_prefill(q, kr, v, **kw)          # sched=True: the binding's block for this stream
    torch.cuda.synchronize()
    assert torch.equal(o, o_fix)
    blocks = list(srt._sched_blocks.values())
    assert blocks and all(int(b.count_nonzero()) == 0 for b in blocks)


def test_two_streams_with_their_own_blocks():
    """Two launches in flight at once on two streams, one block each."""
    srt = need_gpu()
    c1, c2 = CASES[0], CASES[3]
    a = _inputs(srt, c1, seed=21)
    b = _inputs(srt, c2, seed=22)
    ref_a = srt.attn_prefill(a[0], a[1], a[2], sched=False, **a[3])
    ref_b = srt.attn_prefill(b[0], b[1], b[2], sched=False, **b[3])
    torch.cuda.synchronize()
    blk_a = torch.zeros(srt.PREFILL_SCHED_BYTES, dtype=torch.uint8, device="cuda")
    blk_b = torch.zeros(srt.PREFILL_SCHED_BYTES, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    for rep in range(3):
        with torch.cuda.stream(s1):
            outs["a"] = srt.attn_prefill(a[0], a[1], a[2], sched=blk_a, **a[3])
        with torch.cuda.stream(s2):
            outs["b"] = srt.attn_prefill(b[0], b[1], b[2], sched=blk_b, **b[3])
        torch.cuda.synchronize()
        for name, ref in (("a", ref_a), ("b", ref_b)):
            assert torch.equal(outs[name][0], ref[0]) and torch.equal(outs[name][1], ref[1]), (rep, name)
        assert int(blk_a.count_nonzero()) == 0 and int(blk_b.count_nonzero()) == 0


def test_block_checks():
    srt = need_gpu()
    c = dict(B=1, Hq=8, Hkv=2, N=256)
    q, kr, v, kw = _inputs(srt, c)
    with pytest.raises(ValueError):
        srt.attn_prefill(q, kr, v, sched=torch.zeros(64, dtype=torch.uint8, device="cuda"), **kw)
    with pytest.raises(ValueError):
        srt.attn_prefill(q, kr, v, sched=torch.zeros(256, dtype=torch.uint8), **kw)     # host memory
    # a small launch (at most two workgroups per compute unit) keeps the fixed assignment
    blk = torch.zeros(srt.PREFILL_SCHED_BYTES, dtype=torch.uint8, device="cuda")
    o, l = srt.attn_prefill(q, kr, v, sched=blk, **kw)
    o2, l2 = srt.attn_prefill(q, kr, v, sched=False, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l, l2) and int(blk.count_nonzero()) == 0


def test_grid_split_over_several_launches():
    """More than 2^22 workgroups (2^22 + 4096 one-row sequences): the launcher
    splits the grid into launches of 2^22 items.  With one key per sequence
    the softmax weight is exactly 1, so out = v bit for bit, and the backward
    gives dv = dO and dq = dk = 0 up to the rounding of the row statistics."""
    srt = need_gpu()
    B = (1 << 22) + 4096
    q, k, v = qkv(B, 1, 1, 1, 1, 128, torch.bfloat16, 31)
    print("B", B, flush=True)
    o, l = srt.attn_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, v) and bool(torch.isfinite(l).all())
    do = synth.randn((B, 1, 1, 128), torch.bfloat16, 31, synth.DO_ID, "cuda")
    dq, dk, dv = srt.attn_backward(q, k, v, o, do, l)
    torch.cuda.synchronize()
    assert float((dv - do.float()).abs().max()) <= 1e-5 * max(1.0, float(do.float().abs().max()))
    assert float(dq.abs().max()) <= 1e-4 and float(dk.abs().max()) <= 1e-4
