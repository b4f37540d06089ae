"""Oracle, part 2: RoPE-scaled softmax attention, log-sum-exp merge, decode.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed is the plain definition of "Long Context: RoPE / YaRN / NTK /
MLA" §2.4 (rope_attention: rotate Q and K, scores QK^T / sqrt(d), masked
entries -inf, softmax, times V).  FlashAttention is exact ("8.3 长上下文技术"
§8.3.4: the tiled online softmax equals the exact softmax), so the oracle is
that definition, not the tiled algorithm.  Scores are materialised per block of
query rows only to bound memory; no online softmax is used here.

Conventions (readings of the pages where they are silent):
  * layout [B][H][N][D], D innermost;
  * GQA: query head h reads kv head h // (Hq / Hkv);
  * causal mask on absolute positions: key at k_pos0 + c is visible to the
    query at q_pos0 + r iff k_pos0 + c <= q_pos0 + r;
  * sliding window W (> 0) and S sink tokens on top of the causal mask
    ("Long Context..." §10.1 sliding_window_mask: key j visible to query i iff
    i - W < j <= i; §10.2 StreamingLLM: the first S tokens always stay), see
    ``visible``; W = 0 means no window (full causal attention);
  * lse = M + ln(sum exp(s - M)) of the scaled scores (natural log); a row
    with no visible key has O = 0 and lse = -inf;
  * the temperature factor mscale multiplies both rotated q and rotated k
    ("Long Context..." §6.4, "8.3 长上下文技术" §8.3.3).
"""
from __future__ import annotations

import math

import numpy as np

from . import rope as _rope


def _f64(x) -> np.ndarray:
    """Host float64 copy of a numpy array or a (CPU) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy() if str(x.dtype) == "torch.bfloat16" else x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _rotator(pairing: str):
    if pairing == "interleaved":
        return _rope.rotate
    if pairing == "half":
        return _rope.rotate_half
    raise ValueError(f"unknown pairing {pairing}")


def visible(qpos, kpos, *, causal: bool = True, window: int = 0, sink: int = 0) -> np.ndarray:
    """Boolean mask [len(qpos), len(kpos)] on absolute positions.

    Causal: kpos <= qpos.  Window W > 0 additionally keeps only kpos > qpos - W
    (W keys including the query's own position, "Long Context..." §10.1),
    except that positions kpos < S (the attention sinks of §10.2) stay visible.
    A window needs the causal mask (the pages define it only there).
    """
    qpos = np.asarray(qpos, dtype=np.int64)[:, None]
    kpos = np.asarray(kpos, dtype=np.int64)[None, :]
    if window and not causal:
        raise ValueError("a sliding window is defined on top of the causal mask")
    m = np.ones((qpos.shape[0], kpos.shape[1]), dtype=bool)
    if causal:
        m &= kpos <= qpos
    if window > 0:
        m &= (kpos > qpos - window) | (kpos < sink)
    return m


def visible_pairs(N: int, window: int = 0, sink: int = 0) -> int:
    """Number of visible (query, key) pairs of a causal N x N problem, one row at a time.

    Row i sees min(i + 1, W) window keys plus the sinks that fell out of the
    window, min(S, max(0, i - W + 1)); without a window, i + 1 keys.  This is
    the work count behind "O(W N) instead of O(N^2)" ("Long Context..." §10.1).
    """
    total = 0
    for i in range(N):
        if window > 0:
            total += min(i + 1, window) + min(sink, max(0, i - window + 1))
        else:
            total += i + 1
    return total


def attention(q, k, v, *, sm_scale: float, causal: bool = True, q_pos0: int = 0, k_pos0: int = 0,
              theta=None, mscale: float = 1.0, rows=None, block: int = 256, pairing: str = "interleaved",
              window: int = 0, sink: int = 0):
    """Softmax attention with RoPE applied to q and k.

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D].  theta=None means q and k are
    used as given (already rotated).  ``rows`` (optional int array) restricts
    the computation to those query rows.  ``pairing`` picks interleaved pairs
    (default) or half-split pairs.  ``window`` / ``sink``: see ``visible``.
    Returns (O [B, Hq, R, D], lse [B, Hq, R]).
    """
    rot = _rotator(pairing)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.zeros((B, Hq, R, D))
    lse = np.full((B, Hq, R), -np.inf)
    kpos = k_pos0 + np.arange(Nk)
    for b in range(B):
        for hk in range(Hkv):
            kt = k[b, hk] if theta is None else rot(k[b, hk], kpos, theta, mscale)
            vv = v[b, hk]
            for h in range(hk * g, (hk + 1) * g):
                for r0 in range(0, R, block):
                    rr = rows[r0:r0 + block]
                    qpos = q_pos0 + rr
                    qt = q[b, h, rr] if theta is None else rot(q[b, h, rr], qpos, theta, mscale)
                    s = sm_scale * (qt @ kt.T)                              # [r, Nk]
                    s = np.where(visible(qpos, kpos, causal=causal, window=window, sink=sink), s, -np.inf)
                    M = s.max(axis=1, initial=-np.inf)   # no key at all: every row sees none
                    ok = np.isfinite(M)
                    Ms = np.where(ok, M, 0.0)
                    p = np.exp(s - Ms[:, None])                            # exp(-inf) = 0
                    l = p.sum(axis=1)
                    o = np.zeros((len(rr), D))
                    o[ok] = (p[ok] @ vv) / l[ok, None]
                    out[b, h, r0:r0 + len(rr)] = o
                    lse[b, h, r0:r0 + len(rr)] = np.where(ok, Ms + np.log(np.where(ok, l, 1.0)), -np.inf)
    return out, lse


def brute_force(q, k, v, *, sm_scale: float, causal: bool = True, q_pos0: int = 0, k_pos0: int = 0,
                theta=None, mscale: float = 1.0, window: int = 0, sink: int = 0):
    """Tiny-input check: explicit D x D rotation matrices and the full score matrix.

    Rotates with ``rope.rotation_matrix`` (blkdiag form, "Long Context..."
    §2.2), never with ``rope.rotate``; builds the whole Nq x Nk score matrix and
    an explicit boolean mask; softmax by its definition.  Meant for N <= 64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    g = Hq // Hkv
    out = np.zeros((B, Hq, Nq, D))
    lse = np.zeros((B, Hq, Nq))
    mask = np.ones((Nq, Nk), dtype=bool)
    for r in range(Nq):
        for c in range(Nk):
            i, j = q_pos0 + r, k_pos0 + c
            ok = (j <= i) if causal else True
            if window > 0:
                ok = ok and (i - j < window or j < sink)
            mask[r, c] = ok
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            if theta is None:
                qt, kt = q[b, h], k[b, hk]
            else:
                qt = np.stack([mscale * rope_matrix_apply(q_pos0 + r, theta, q[b, h, r]) for r in range(Nq)])
                kt = np.stack([mscale * rope_matrix_apply(k_pos0 + c, theta, k[b, hk, c]) for c in range(Nk)])
            S = np.full((Nq, Nk), -np.inf)
            for r in range(Nq):
                for c in range(Nk):
                    if mask[r, c]:
                        S[r, c] = sm_scale * float(np.dot(qt[r], kt[c]))
            for r in range(Nq):
                if not mask[r].any():
                    out[b, h, r] = 0.0
                    lse[b, h, r] = -np.inf
                    continue
                e = np.exp(S[r] - S[r].max())
                out[b, h, r] = (e / e.sum()) @ v[b, hk]
                lse[b, h, r] = math.log(np.exp(S[r][mask[r]]).sum())
    return out, lse


def rope_matrix_apply(p: float, theta, x) -> np.ndarray:
    return _rope.rotation_matrix(p, np.asarray(theta, dtype=np.float64)) @ np.asarray(x, dtype=np.float64)


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial softmax states over disjoint key sets.

    lse = log(e^{lse_a} + e^{lse_b});  O = e^{lse_a - lse} O_a + e^{lse_b - lse} O_b.
    This is the rescaling step of the online softmax that Ring Attention
    applies after each K/V block ("8.3 长上下文技术" §8.3.4 (2), §8.3.5 step 3).
    A state with lse = -inf (no visible key) is the identity; two such states
    merge to (O = 0, lse = -inf).
    """
    o_a, o_b = _f64(o_a), _f64(o_b)
    la, lb = _f64(lse_a), _f64(lse_b)
    m = np.maximum(la, lb)
    fin = np.isfinite(m)
    ms = np.where(fin, m, 0.0)
    ea = np.where(np.isfinite(la), np.exp(la - ms), 0.0)
    eb = np.where(np.isfinite(lb), np.exp(lb - ms), 0.0)
    tot = ea + eb
    lse = np.where(fin, ms + np.log(np.where(fin, tot, 1.0)), -np.inf)
    wa = np.where(fin, ea / np.where(fin, tot, 1.0), 0.0)
    wb = np.where(fin, eb / np.where(fin, tot, 1.0), 0.0)
    return wa[..., None] * o_a + wb[..., None] * o_b, lse


def decode(q, k_cache_rotated, v_cache, *, sm_scale: float, seq_lens=None, theta=None, mscale: float = 1.0,
           pairing: str = "interleaved", window: int = 0, sink: int = 0):
    """One new query per sequence against its cache (already rotated keys).

    q: [B, Hq, D] raw, rotated at position seq_len - 1 (the new token's own
    K/V is the last cache row, so every cached key is visible).  The decode
    step reads the whole cache ("Long Context..." §12.3; "长上下文推理" on
    KV-cache reads).  With a window only the last W cached keys and the first
    S (sinks) are visible, the query being at position seq_len - 1.
    Returns (O [B, Hq, D], lse [B, Hq]).
    """
    q, kc, vc = _f64(q), _f64(k_cache_rotated), _f64(v_cache)
    B, Hq, D = q.shape
    _, Hkv, Nk, _ = kc.shape
    lens = [Nk] * B if seq_lens is None else [int(x) for x in seq_lens]
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = lens[b]
        if n <= 0:
            continue
        qb = q[b][:, None, :]                                   # [Hq, 1, D]
        if theta is not None:
            qb = _rotator(pairing)(qb, np.array([n - 1]), theta, mscale)
        o, l = attention(qb[None], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], sm_scale=sm_scale,
                         causal=True, q_pos0=n - 1, theta=None, window=window, sink=sink)
        out[b] = o[0, :, 0]
        lse[b] = l[0, :, 0]
    return out, lse
