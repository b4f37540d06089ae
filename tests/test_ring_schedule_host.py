"""The ring launch schedule (csrc/ring.cpp) checked on the CPU.

ring.cpp is compiled together with tests/host/ring_schedule_stub.cpp, whose
launcher stubs print every launch instead of running it.  From the printed
launches the test rebuilds which (query row, key row) pairs the schedule
scores, each under its launch's own mask, and compares them with the oracle's
visible pairs at the partition's true positions: every visible pair exactly
once, nothing else.  It also checks the running-state chain of every query
run (the first launch writes the fp32 state, each later launch folds its
result into that state in its epilogue, in place, and the last one writes the
merged result to the run's output rows) and the RoPE positions each launch is
given."""
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import attention as A
from oracle import ring as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODES = {"contiguous": 0, "striped": 1, "zigzag": 2}


@pytest.fixture(scope="module")
def stub():
    out = os.path.join(ROOT, "_build", "ring_schedule_stub")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    csrc = os.path.join(ROOT, "scaled_rope_tiled_amd", "csrc")
    cmd = ["/opt/rocm/bin/hipcc", "-O1", "-std=c++17", "-I", csrc, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "ring_schedule_stub.cpp"), os.path.join(csrc, "ring.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-3000:])
    return out


def _kv(line):
    return dict(re.findall(r"(\w+)=([^\s]+)", line))


def _loc(s):
    name, off = s.split(":")
    return name, int(off)


def run(stub, B, Hq, Hkv, N, D, P, mode, device, window, sink, flags, bf16):
    r = subprocess.run([stub] + [str(x) for x in (B, Hq, Hkv, N, D, P, MODES[mode], device, window, sink, flags,
                                                 int(bf16))], capture_output=True, text=True, check=True)
    return r.stdout.splitlines()


CASES = [(m, P, N, w, s, dev) for m in MODES for P in (1, 2, 4, 8) for N in (16 * P, 48 * P)
         for (w, s) in ((0, 0), (5, 0), (7, 3), (40, 20)) for dev in (-1, P - 1)
         if not (m == "striped" and w > 0)]


@pytest.mark.parametrize("mode,P,N,window,sink,device", CASES)
def test_schedule_scores_every_visible_pair_once(stub, mode, P, N, window, sink, device):
    D, elt = 128, 2
    lines = run(stub, 1, 4, 2, N, D, P, mode, device, window, sink, 3, True)
    ws_bytes = int(lines[0].split()[1])
    pos = R.partition_positions(N, P, mode)
    C = N // P
    want = A.visible(pos, pos, window=window, sink=sink).astype(int)
    rows = np.zeros(N, dtype=bool)
    for r in (range(P) if device < 0 else [device]):
        rows[r * C:(r + 1) * C] = True
    want[~rows] = 0
    got = np.zeros((N, N), dtype=int)
    chains = {}
    sched = None
    for ln in lines[1:]:
        kv = _kv(ln)
        if ln.startswith("zero"):
            # the prefill launches' scheduling block: zero-filled once, before any launch
            assert sched is None and not chains and kv["n"] == "10"
            sched = kv["at"]
            name, off = _loc(sched)
            assert name == "ws" and off % 8 == 0 and off + 80 <= ws_bytes
            continue
        if ln.startswith("rope"):
            assert "mode=%d" % MODES[mode] in ln and "P=%d" % P in ln and "C=%d" % C in ln
            continue
        if ln.startswith("prefill"):
            qn, qo = _loc(kv["q"])
            kn, ko = _loc(kv["k"])
            assert qn == "q" and kn == "ws" and kv["flags"] == "1"      # K rotated once into the workspace
            q0, k0 = qo // (D * elt), ko // (D * elt)
            Nq, Nk = int(kv["Nq"]), int(kv["Nk"])
            qp, kp, w, s = int(kv["qp"]), int(kv["kp"]), int(kv["window"]), int(kv["sink"])
            vis = A.visible(qp + np.arange(Nq), kp + np.arange(Nk), window=w, sink=s)
            got[q0:q0 + Nq, k0:k0 + Nk] += vis
            # RoPE positions of the launch are the true positions of its rows
            step = int(kv["step"])
            assert int(kv["qr"]) == pos[q0] and int(kv["kr"]) == pos[k0]
            assert all(pos[q0 + t] == pos[q0] + step * t for t in range(Nq))
            assert all(pos[k0 + u] == pos[k0] + step * u for u in range(Nk))
            chains.setdefault(q0, []).append((kv["out"], kv["obf16"], kv["acc"], kv["lse"], kv["acclse"],
                                              int(kv["ohs"]), int(kv["ahs"])))
            assert kv["sched"] == sched                  # every launch shares the one block
            for key in ("out", "lse", "acc", "acclse"):
                name, off = _loc(kv[key])
                if name == "ws":
                    assert 0 <= off < ws_bytes and off + 80 <= _loc(sched)[1]   # state before the block
        assert not ln.startswith("merge")              # no separate merge launches
    np.testing.assert_array_equal(got, want)
    for q0, ch in chains.items():
        out, obf16, acc, lse, acclse, ohs, ahs = zip(*ch)
        # the first launch starts the running state; every later one folds into it
        assert acc[0] == "none:-1" and acclse[0] == "none:-1"
        assert all(_loc(x)[0] == "ws" for x in acc[1:]) and all(_loc(x)[0] == "ws" for x in acclse[1:])
        # all but the last keep the fp32 state in the workspace, in place
        for i in range(len(ch) - 1):
            assert _loc(out[i])[0] == "ws" and obf16[i] == "0" and _loc(lse[i])[0] == "ws"
            if i > 0:
                assert out[i] == acc[i] and lse[i] == acclse[i] and ohs[i] == ahs[i]
        # the last writes the merged result to the run's own output rows
        name, off = _loc(out[-1])
        assert name == "out" and off == q0 * D * elt and obf16[-1] == "1"
        assert _loc(lse[-1]) == ("lse", q0 * 4)


def test_zigzag_and_striped_balance_launch_work(stub):
    """Scored pairs per device from the printed launches: zig-zag equal across
    devices, striped within P diagonals, contiguous growing with the device."""
    N, P, D = 512, 8, 128
    per = {}
    for mode in MODES:
        tot = []
        for dev in range(P):
            n = 0
            for ln in run(stub, 1, 4, 1, N, D, P, mode, dev, 0, 0, 1, True)[1:]:
                if ln.startswith("prefill"):
                    kv = _kv(ln)
                    Nq, Nk, qp, kp = int(kv["Nq"]), int(kv["Nk"]), int(kv["qp"]), int(kv["kp"])
                    n += int(A.visible(qp + np.arange(Nq), kp + np.arange(Nk)).sum())
            tot.append(n)
        per[mode] = tot
    assert len(set(per["zigzag"])) == 1
    assert max(per["striped"]) - min(per["striped"]) <= (P - 1) * (N // P)
    assert per["contiguous"] == sorted(per["contiguous"]) and per["contiguous"][-1] > 1.8 * np.mean(per["contiguous"])
