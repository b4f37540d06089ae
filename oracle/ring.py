"""Oracle, part 3: Ring Attention with contiguous, Striped and Zig-Zag partitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"8.3 长上下文技术" §8.3.5.  P devices form a ring; each holds one query shard
Q_r and one key/value shard (K_r, V_r) of the sequence.  Device r first
attends its own K/V shard, then for P - 1 steps receives the shard of device
(r - 1) mod P (so at step s it holds shard (r - s) mod P), attends it and
folds the result into its running state with the online-softmax rescaling
(here: the log-sum-exp merge of ``attention.merge``).  The result is exact:
it equals attention over the whole sequence.

The shard a device holds depends on the partition (§8.3.5, causal load
balance):
  * contiguous: shard r = positions [r C, (r + 1) C), C = N / P;
  * striped:    shard r = positions {r, r + P, r + 2P, ...} (stride P);
  * zigzag:     the sequence is cut into 2P chunks of h = N / (2P); shard r
                = chunk r followed by chunk 2P - 1 - r.
Shards are stored shard-major: row t of shard r is row r * (N / P) + t of a
[..., N, D] tensor, holding the position ``partition_positions`` gives.
"""
from __future__ import annotations

import numpy as np

from . import attention as _A

PARTITIONS = ("contiguous", "striped", "zigzag")


def partition_positions(N: int, P: int, mode: str) -> np.ndarray:
    """Position of every shard-major row: pos[r * (N/P) + t] for shard r, row t."""
    if P < 1 or N % P:
        raise ValueError("N must be a multiple of P")
    C = N // P
    pos = np.empty(N, dtype=np.int64)
    for r in range(P):
        if mode == "contiguous":
            pos[r * C:(r + 1) * C] = r * C + np.arange(C)
        elif mode == "striped":
            pos[r * C:(r + 1) * C] = r + P * np.arange(C)
        elif mode == "zigzag":
            if N % (2 * P):
                raise ValueError("zigzag needs N a multiple of 2P")
            h = N // (2 * P)
            pos[r * C:r * C + h] = r * h + np.arange(h)
            pos[r * C + h:(r + 1) * C] = (2 * P - 1 - r) * h + np.arange(h)
        else:
            raise ValueError(f"unknown partition {mode}")
    return pos


def ring_order(P: int):
    """(device r, step s, shard j held at that step): j = (r - s) mod P."""
    return [(r, s, (r - s) % P) for r in range(P) for s in range(P)]


def ring_attention(q, k, v, *, P: int, mode: str, sm_scale: float, theta=None, mscale: float = 1.0,
                   window: int = 0, sink: int = 0, pairing: str = "interleaved"):
    """Ring Attention over P simulated devices, inputs and outputs shard-major.

    q: [B, Hq, N, D], k, v: [B, Hkv, N, D], rows in the partition's shard-major
    order.  Each device's partial state over one received shard is plain
    softmax attention of its queries against that shard's keys at their true
    positions (causal mask, optional window and sinks); states are merged in
    ring order.  Returns (O [B, Hq, N, D], lse [B, Hq, N]) shard-major.
    """
    q, k, v = _A._f64(q), _A._f64(k), _A._f64(v)
    B, Hq, N, D = q.shape
    C = N // P
    pos = partition_positions(N, P, mode)
    rot = _A._rotator(pairing)
    # rotate every row at its own position (a device rotates its own shard)
    if theta is not None:
        q = np.stack([rot(q[b], pos, theta, mscale) for b in range(B)])
        k = np.stack([rot(k[b], pos, theta, mscale) for b in range(B)])
    out = np.zeros((B, Hq, N, D))
    lse = np.full((B, Hq, N), -np.inf)
    for r in range(P):
        rows = slice(r * C, (r + 1) * C)
        state = None
        for _, s, j in [x for x in ring_order(P) if x[0] == r]:
            cols = slice(j * C, (j + 1) * C)
            part = _masked_attention(q[:, :, rows], k[:, :, cols], v[:, :, cols], pos[rows], pos[cols],
                                     sm_scale, window, sink)
            state = part if state is None else _A.merge(*state, *part)
        out[:, :, rows], lse[:, :, rows] = state
    return out, lse


def _masked_attention(q, k, v, qpos, kpos, sm_scale, window, sink):
    """Softmax attention with the causal (window, sink) mask on explicit positions."""
    B, Hq, R, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    vis = _A.visible(qpos, kpos, causal=True, window=window, sink=sink)
    o = np.zeros((B, Hq, R, D))
    l = np.full((B, Hq, R), -np.inf)
    for b in range(B):
        for h in range(Hq):
            s = np.where(vis, sm_scale * (q[b, h] @ k[b, h // g].T), -np.inf)
            M = s.max(axis=1, initial=-np.inf)   # no key at all: every row sees none
            ok = np.isfinite(M)
            Ms = np.where(ok, M, 0.0)
            p = np.exp(s - Ms[:, None])
            den = p.sum(axis=1)
            o[b, h, ok] = (p[ok] @ v[b, h // g]) / den[ok, None]
            l[b, h] = np.where(ok, Ms + np.log(np.where(ok, den, 1.0)), -np.inf)
    return o, l


def step_work(N: int, P: int, mode: str, window: int = 0, sink: int = 0) -> np.ndarray:
    """Visible (query, key) pairs of device r at ring step s: array [P, P] (r, s)."""
    pos = partition_positions(N, P, mode)
    C = N // P
    w = np.zeros((P, P), dtype=np.int64)
    for r, s, j in ring_order(P):
        w[r, s] = int(_A.visible(pos[r * C:(r + 1) * C], pos[j * C:(j + 1) * C], window=window,
                                 sink=sink).sum())
    return w
