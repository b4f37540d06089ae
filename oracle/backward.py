"""Oracle, part 4: gradients of RoPE-scaled softmax attention (numpy float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The backward pass of O = softmax(S) V with S = sm_scale * q~ k~^T (masked
entries -inf), q~ = mscale R_p q, k~ = mscale R_p k, written from the chain
rule of that definition ("Long Context: RoPE / YaRN / NTK / MLA" §2.4
rope_attention; "8.3 长上下文技术" §8.3.4 (3): the backward pass recomputes the
attention matrix from Q, K, V and the saved softmax statistics instead of
storing it):

    P  = exp(S - lse)                      (lse saved by the forward pass)
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - delta),  delta_r = sum_d dO_rd O_rd   (= sum_c P_rc dP_rc)
    dq~ = sm_scale dS k~,   dk~ = sm_scale dS^T q~
    dq = mscale R_p^T dq~,  dk = mscale R_p^T dk~

R_p^T is the rotation by -p theta ("长上下文外推" §4 property: the transpose of
a rotation is the rotation by the opposite angle), so the gradient is turned
back with the same table at the negated position.  GQA: a KV head's dk, dv
sum over its query heads.  Rows with no visible key contribute nothing.
"""
from __future__ import annotations

import numpy as np

from . import attention as _A


def rotate_back(g, pos, theta, mscale: float = 1.0, pairing: str = "interleaved") -> np.ndarray:
    """mscale R_p^T g: rotation by the opposite angle."""
    return _A._rotator(pairing)(g, -np.asarray(pos, dtype=np.float64), theta, mscale)


def attention_backward(q, k, v, dout, *, sm_scale: float, causal: bool = True, q_pos0: int = 0, k_pos0: int = 0,
                       theta=None, mscale: float = 1.0, window: int = 0, sink: int = 0,
                       pairing: str = "interleaved"):
    """Returns (dq [B,Hq,Nq,D], dk [B,Hkv,Nk,D], dv [B,Hkv,Nk,D], delta [B,Hq,Nq])."""
    rot = _A._rotator(pairing)
    q, k, v, dout = _A._f64(q), _A._f64(k), _A._f64(v), _A._f64(dout)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    g = Hq // Hkv
    qpos = q_pos0 + np.arange(Nq)
    kpos = k_pos0 + np.arange(Nk)
    vis = _A.visible(qpos, kpos, causal=causal, window=window, sink=sink) if causal else np.ones((Nq, Nk), bool)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((B, Hq, Nq))
    for b in range(B):
        for hk in range(Hkv):
            kt = k[b, hk] if theta is None else rot(k[b, hk], kpos, theta, mscale)
            dkt = np.zeros((Nk, D))
            for h in range(hk * g, (hk + 1) * g):
                qt = q[b, h] if theta is None else rot(q[b, h], qpos, theta, mscale)
                s = np.where(vis, sm_scale * (qt @ kt.T), -np.inf)
                M = s.max(axis=1, initial=-np.inf)   # no key at all: every row sees none
                ok = np.isfinite(M)
                p = np.zeros_like(s)
                p[ok] = np.exp(s[ok] - M[ok, None])
                p[ok] /= p[ok].sum(axis=1, keepdims=True)
                o = p @ v[b, hk]
                do = dout[b, h]
                dv[b, hk] += p.T @ do
                dp = do @ v[b, hk].T
                dl = (do * o).sum(axis=1)
                ds = p * (dp - dl[:, None])
                dqt = sm_scale * ds @ kt
                dkt += sm_scale * ds.T @ qt
                dq[b, h] = dqt if theta is None else rotate_back(dqt, qpos, theta, mscale, pairing)
                delta[b, h] = dl
            dk[b, hk] = dkt if theta is None else rotate_back(dkt, kpos, theta, mscale, pairing)
    return dq, dk, dv, delta


def attention_backward_sampled(q, k, v, dout, *, hk: int, rows, keys, sm_scale: float, causal: bool = True,
                               q_pos0: int = 0, k_pos0: int = 0, theta=None, mscale: float = 1.0, window: int = 0,
                               sink: int = 0, pairing: str = "interleaved", b: int = 0):
    """The same gradients as `attention_backward`, for batch b and KV head hk only, at chosen outputs:
    dq at query rows `rows` of every query head of hk's group ([G][len(rows)][D]) and dk, dv at keys
    `keys` of hk ([len(keys)][D] each).  Every needed row of P is formed whole from its row of S (so its
    own lse and delta are exact); a key's gradients sum over exactly the rows that see it.  The cost is
    one row of S per needed row: cheap for any row, and for keys that few rows see (the end of a
    causal sequence), at any sequence length."""
    rot = _A._rotator(pairing)
    q, k, v, dout = _A._f64(q)[b], _A._f64(k)[b], _A._f64(v)[b], _A._f64(dout)[b]
    Hq, Nq, D = q.shape
    Hkv, Nk, _ = k.shape
    g = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    kpos = k_pos0 + np.arange(Nk)
    kt = k[hk] if theta is None else rot(k[hk], kpos, theta, mscale)
    vv = v[hk]
    # rows that see any sampled key, plus the sampled rows
    see = _A.visible(q_pos0 + np.arange(Nq), kpos[keys], causal=causal, window=window, sink=sink) if causal \
        else np.ones((Nq, len(keys)), bool)
    need = np.union1d(np.nonzero(see.any(axis=1))[0], rows)
    dq = np.zeros((g, len(rows), D))
    dkt = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for gi, h in enumerate(range(hk * g, (hk + 1) * g)):
        for i in need:
            qp = q_pos0 + i
            qt = q[h, i] if theta is None else rot(q[h, i][None, :], np.array([qp]), theta, mscale)[0]
            vis = _A.visible(np.array([qp]), kpos, causal=causal, window=window, sink=sink)[0] if causal \
                else np.ones(Nk, bool)
            if not vis.any():
                continue
            s = np.where(vis, sm_scale * (kt @ qt), -np.inf)
            m = s[vis].max()
            p = np.where(vis, np.exp(s - m), 0.0)
            p /= p.sum()
            o = p @ vv
            do = dout[h, i]
            dl = do @ o
            ds = p * (vv @ do - dl)
            sel = np.nonzero(rows == i)[0]
            if len(sel):
                dqt = sm_scale * (ds @ kt)
                dq[gi, sel[0]] = dqt if theta is None else rotate_back(dqt[None, :], np.array([qp]), theta, mscale,
                                                                       pairing)[0]
            dv += p[keys, None] * do[None, :]
            dkt += sm_scale * ds[keys, None] * qt[None, :]
    dk = dkt if theta is None else rotate_back(dkt, kpos[keys], theta, mscale, pairing)
    return dq, dk, dv
