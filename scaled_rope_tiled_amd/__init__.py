"""scaled_rope_tiled_amd: RoPE-scaled tiled causal attention for MI355X (gfx950).

Thin Python binding over the C ABI of libsrt.so (include/srt.h).  Functions
carry the same names as the C entry points without the ``srt_`` prefix and do
argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the library's kernels.

    rope_inv_freq(method, base, s, L, alpha, beta, D) -> (theta', mscale, band)
    rope_inv_freq_dynamic_ntk(base, seq_len, L, D)    -> (theta', s)
    rope_inv_freq_factors(base, lambdas, D)           -> theta'
    rope_cos_sin(theta', D, mscale, npos, device)     -> table [npos, D/2, 2] fp32
    rope_apply(x, table, pos0=0, out=None, pairing=) -> rotated x
    attn_prefill(q, k, v, ...)                        -> (out, lse)
    attn_merge_states(o_a, lse_a, o_b, lse_b, ...)    -> (out, lse)
    attn_decode_splitk(q, k_cache, v_cache, ...)      -> (out, lse)
    attn_decode_splitk_noalloc(q, k_cache, v_cache, ...) -> (out, lse), no workspace
    attn_ring_prefill(q, k, v, num_devices=, partition=, ...) -> (out, lse)
    attn_backward(q, k, v, out, dout, lse, ...)      -> (dq, dk, dv) fp32
    attn_backward_workspace_size(dtype, B, Hq, Hkv, Nq, Nk, D, rope_flags) -> bytes
"""
from __future__ import annotations

import ctypes as C
import math

import numpy as np
import torch

from . import _lib

NONE, PI, NTK, YARN = 0, 1, 2, 3
F32, BF16 = 0, 1
ROTATE_Q, ROTATE_K, PAIR_HALF = 1, 2, 4
PAIRING_INTERLEAVED, PAIRING_HALF = 0, 1
PARTITIONS = {"contiguous": 0, "striped": 1, "zigzag": 2}
BAND_LOW, BAND_MID, BAND_HIGH = 0, 1, 2

__all__ = ["rope_inv_freq", "rope_inv_freq_dynamic_ntk", "rope_inv_freq_factors", "rope_cos_sin", "rope_apply", "attn_prefill", "attn_merge_states",
           "attn_decode_splitk", "attn_decode_workspace_size", "attn_decode_splitk_noalloc",
           "attn_decode_noalloc_max_workspace", "attn_ring_prefill", "attn_ring_workspace_size",
           "attn_backward", "attn_backward_workspace_size", "NONE", "PI", "NTK", "YARN",
           "ROTATE_Q", "ROTATE_K", "PAIR_HALF", "PAIRING_INTERLEAVED", "PAIRING_HALF", "PREFILL_SCHED_BYTES", "lib"]


def lib():
    return _lib.load()


# Load at import: the binding has no fallback, a missing library is an error here.
_lib.load()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _tdt(code: int) -> torch.dtype:
    return torch.float32 if code == F32 else torch.bfloat16


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _on_device(dev: torch.device, **tensors) -> None:
    """Every given tensor (None skipped) must live on the GPU `dev`: the kernels
    take raw device pointers, so a host tensor or another device's memory would
    be dereferenced as if it were this device's."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} is on {t.device}; expected {dev}")


def _table(table, D: int, dev: torch.device):
    """(pointer, npos) of a cos/sin table for head size D, or (None, 0).

    The kernels index entry (position, pair) at position * (D/2) + pair, so a
    table built for another D, a strided view or another dtype would be read
    out of bounds or misread."""
    if table is None:
        return None, 0
    _on_device(dev, table=table)
    if table.dtype != torch.float32 or not table.is_contiguous() or table.dim() != 3 \
            or tuple(table.shape[1:]) != (D // 2, 2):
        raise ValueError(f"table must be a contiguous float32 [npos, {D // 2}, 2] tensor for D={D} "
                         f"(got {tuple(table.shape)} {table.dtype})")
    return _ptr(table), int(table.shape[0])


def _head_stride(t: torch.Tensor, name: str) -> int:
    """Head stride of a [B][H][N][D] tensor whose rows are contiguous.

    Allows views sliced along N (for ring chunks); requires D innermost,
    rows D apart and batch stride = H * head stride."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, D]")
    B, H, N, D = t.shape
    sb, sh, sn, sd = t.stride()
    if sd != 1 or (N > 1 and sn != D) or (B > 1 and sb != H * sh) or (H > 1 and sh < N * D):
        raise ValueError(f"{name}: rows must be contiguous [B][H][N][D] (slices along N allowed)")
    return sh if H > 1 else max(sh, N * D)


def rope_inv_freq(method: int, base: float, s: float = 1.0, L: float = 0.0, alpha: float = 1.0,
                  beta: float = 32.0, D: int = 128):
    """Scaled RoPE frequencies (host, fp64).  Returns (theta' [D/2] float64, mscale, band [D/2] int8)."""
    th = (C.c_double * (D // 2))()
    ms = C.c_double()
    band = (C.c_byte * (D // 2))()
    _lib.check(lib().srt_rope_inv_freq(int(method), float(base), float(s), float(L), float(alpha),
                                       float(beta), int(D), th, C.byref(ms), band), "rope_inv_freq")
    return np.frombuffer(th, dtype=np.float64).copy(), ms.value, np.frombuffer(band, dtype=np.int8).copy()


def rope_inv_freq_dynamic_ntk(base: float, seq_len: int, L: float, D: int = 128):
    """NTK-aware frequencies with s = max(1, seq_len / L).  Returns (theta' [D/2] float64, s)."""
    th = (C.c_double * (D // 2))()
    s = C.c_double()
    _lib.check(lib().srt_rope_inv_freq_dynamic_ntk(float(base), int(seq_len), float(L), int(D), th, C.byref(s)),
               "rope_inv_freq_dynamic_ntk")
    return np.frombuffer(th, dtype=np.float64).copy(), s.value


def rope_inv_freq_factors(base: float, lambdas, D: int = 128):
    """theta'_d = base^(-2d/D) / lambda_d.  Returns theta' [D/2] float64."""
    lam = np.ascontiguousarray(np.asarray(lambdas, dtype=np.float64))
    if lam.shape != (D // 2,):
        raise ValueError("one factor per pair (D/2 entries)")
    th = (C.c_double * (D // 2))()
    _lib.check(lib().srt_rope_inv_freq_factors(float(base), lam.ctypes.data_as(C.POINTER(C.c_double)), int(D), th),
               "rope_inv_freq_factors")
    return np.frombuffer(th, dtype=np.float64).copy()


def _pairing(p) -> int:
    if p in (PAIRING_INTERLEAVED, "interleaved"):
        return PAIRING_INTERLEAVED
    if p in (PAIRING_HALF, "half"):
        return PAIRING_HALF
    raise ValueError(f"unknown pairing {p!r}")


def rope_cos_sin(theta, D: int, mscale: float, npos: int, device="cuda") -> torch.Tensor:
    """Device table [npos, D/2, 2] fp32 of mscale*(cos, sin)(p*theta'_i)."""
    th = np.ascontiguousarray(np.asarray(theta, dtype=np.float64))
    if th.shape != (D // 2,):
        raise ValueError("theta must have D/2 entries")
    dev = torch.device(device)
    table = torch.empty((int(npos), D // 2, 2), dtype=torch.float32, device=dev)
    _lib.check(lib().srt_rope_cos_sin(th.ctypes.data_as(C.POINTER(C.c_double)), int(D), float(mscale),
                                      int(npos), _ptr(table), _stream(dev)), "rope_cos_sin")
    return table


def rope_apply(x: torch.Tensor, table: torch.Tensor, pos0: int = 0, out: torch.Tensor | None = None,
               pairing="interleaved"):
    """Rotate every row of x [B, H, N, D] (row r at position pos0 + r).  out may be x.
    pairing: "interleaved" (x_2i, x_2i+1) or "half" (x_i, x_i+D/2)."""
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    out = torch.empty_like(x) if out is None else out
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must match x")
    B, H, N, D = x.shape
    _on_device(x.device, x=x, out=out)
    if table is None:
        raise ValueError("rope_apply needs a table")
    tp, npos = _table(table, D, x.device)
    _lib.check(lib().srt_rope_apply(_ptr(x), _ptr(out), _dt(x), B, H, N, D, int(pos0), tp,
                                    npos, _pairing(pairing), _stream(x.device)), "rope_apply")
    return out


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, sm_scale: float | None = None,
                 causal: bool = True, q_pos0: int = 0, k_pos0: int = 0, table: torch.Tensor | None = None,
                 rope_flags: int | None = None, out: torch.Tensor | None = None,
                 out_dtype: torch.dtype | None = None, lse: torch.Tensor | bool = True,
                 window: int = 0, sink: int = 0, sched=True):
    """Tiled causal attention with rotate-on-load RoPE.

    q [B, Hq, Nq, D], k/v [B, Hkv, Nk, D] (views sliced along N allowed).
    rope_flags defaults to ROTATE_Q|ROTATE_K when a table is given; add
    PAIR_HALF for half-split pairs.  window > 0 (causal only) keeps key j for
    query i iff i - j < window or j < sink (absolute positions).
    sched: the scheduling block of srt_attn_prefill: True (default) uses one
    zero-filled block per (device, stream), kept for reuse (the kernel leaves
    it zero-filled; calls on one stream never overlap); a tensor of at least
    PREFILL_SCHED_BYTES zero-filled bytes on q's device is used as given;
    False or None asks for the fixed assignment.
    Returns (out [B, Hq, Nq, D], lse [B, Hq, Nq] fp32 or None)."""
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, Nk, D] matching q")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    qs, ks, vs = _head_stride(q, "q"), _head_stride(k, "k"), _head_stride(v, "v")
    if ks != vs:
        raise ValueError("k and v must have the same head stride")
    if out is None:
        out = torch.empty((B, Hq, Nq, D), dtype=out_dtype or q.dtype, device=q.device)
    os_ = _head_stride(out, "out")
    if lse is True:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    ls = 0
    if lse is not None:
        if lse.dtype != torch.float32 or lse.stride(-1) != 1 or (Hq > 1 and lse.stride(1) < Nq):
            raise ValueError("lse must be fp32 [B, Hq, Nq] with rows contiguous")
        ls = lse.stride(1) if Hq > 1 else max(lse.stride(1), Nq)
    if rope_flags is None:
        rope_flags = (ROTATE_Q | ROTATE_K) if table is not None else 0
    _on_device(q.device, q=q, k=k, v=v, out=out, lse=lse)
    tp, npos = _table(table, D, q.device)
    sm = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    sp = _sched_block(sched, q.device)
    _lib.check(lib().srt_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _dt(q), B, Hq, Hkv, Nq, Nk, D,
                                      qs, ks, int(q_pos0), int(k_pos0), int(bool(causal)), int(window), int(sink), sm,
                                      tp, npos, int(rope_flags),
                                      _ptr(out), _dt(out), os_, _ptr(lse), ls, sp, _stream(q.device)),
               "attn_prefill")
    return out, lse


PREFILL_SCHED_BYTES = 128     # SRT_PREFILL_SCHED_BYTES
_sched_blocks = {}


def _sched_block(sched, dev: torch.device):
    """Pointer to the scheduling block for this call (see attn_prefill), or None."""
    if sched is None or sched is False:
        return None
    if sched is True:
        key = (dev.index, _stream(dev))
        blk = _sched_blocks.get(key)
        if blk is None:
            blk = _sched_blocks[key] = torch.zeros(PREFILL_SCHED_BYTES, dtype=torch.uint8, device=dev)
        return _ptr(blk)
    _on_device(dev, sched=sched)
    if not sched.is_contiguous() or sched.numel() * sched.element_size() < PREFILL_SCHED_BYTES \
            or sched.data_ptr() % 8:
        raise ValueError(f"sched must be a contiguous, 8-byte aligned block of >= {PREFILL_SCHED_BYTES} bytes")
    return _ptr(sched)


def attn_merge_states(o_a, lse_a, o_b, lse_b, *, out=None, lse_out=None, out_dtype=None):
    """Log-sum-exp merge of two partial states.  out may be o_a (in place)."""
    B, H, N, D = o_a.shape
    if o_b.shape != o_a.shape or o_b.dtype != o_a.dtype:
        raise ValueError("o_a and o_b must match")
    ia, ib = _head_stride(o_a, "o_a"), _head_stride(o_b, "o_b")
    if ia != ib:
        raise ValueError("o_a and o_b must have the same head stride")
    for t in (lse_a, lse_b):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, N):
            raise ValueError("lse_a / lse_b must be contiguous fp32 [B, H, N]")
    if out is None:
        out = torch.empty((B, H, N, D), dtype=out_dtype or o_a.dtype, device=o_a.device)
    os_ = _head_stride(out, "out")
    if lse_out is None:
        lse_out = torch.empty((B, H, N), dtype=torch.float32, device=o_a.device)
    ls = lse_out.stride(1) if H > 1 else max(lse_out.stride(1), N)
    _on_device(o_a.device, o_a=o_a, lse_a=lse_a, o_b=o_b, lse_b=lse_b, out=out, lse_out=lse_out)
    _lib.check(lib().srt_attn_merge_states(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _dt(o_a), ia,
                                           _ptr(out), _dt(out), os_, _ptr(lse_out), ls, B, H, N, D,
                                           _stream(o_a.device)), "attn_merge_states")
    return out, lse_out


def attn_decode_workspace_size(B: int, Hq: int, D: int, num_splits: int) -> int:
    n = C.c_size_t()
    _lib.check(lib().srt_attn_decode_workspace_size(B, Hq, D, num_splits, C.byref(n)),
               "attn_decode_workspace_size")
    return n.value


def attn_decode_splitk(q, k_cache, v_cache, *, num_splits: int, sm_scale: float | None = None,
                       table: torch.Tensor | None = None, seq_lens: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, out=None, lse=True, pairing="interleaved",
                       window: int = 0, sink: int = 0):
    """Split-K decode.  q [B, Hq, D] raw (rotated at seq_len-1 when a table is given);
    k_cache/v_cache [B, Hkv, Nk, D] with rotated keys.  Returns (out [B, Hq, D], lse [B, Hq])."""
    B, Hq, D = q.shape
    _, Hkv, Nk, _ = k_cache.shape
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    need = attn_decode_workspace_size(B, Hq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be contiguous int32 [B]")
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, workspace=workspace, out=out,
               lse=lse)
    tp, npos = _table(table, D, q.device)
    sm = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _lib.check(lib().srt_attn_decode_splitk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dt(q), B, Hq, Hkv, Nk, D,
                                            _ptr(seq_lens), int(num_splits), sm, tp,
                                            npos, _pairing(pairing),
                                            int(window), int(sink),
                                            _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                            _stream(q.device)), "attn_decode_splitk")
    return out, lse


def attn_decode_splitk_noalloc(q, k_cache, v_cache, *, num_splits: int, sm_scale: float | None = None,
                               table: torch.Tensor | None = None, seq_lens: torch.Tensor | None = None,
                               out=None, lse=True, pairing="interleaved", window: int = 0, sink: int = 0):
    """attn_decode_splitk without a workspace: the split partials go to the
    library's static per-GPU scratch (no device allocation in the call, at most
    srt_attn_decode_noalloc_max_workspace() bytes of partials).  Calls that
    overlap on one GPU share that scratch and must be ordered by the caller.
    Pass `out` (and `lse`, or lse=False) to make the whole call allocation-free."""
    B, Hq, D = q.shape
    _, Hkv, Nk, _ = k_cache.shape
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if lse is True:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous()):
        raise ValueError("seq_lens must be contiguous int32 [B]")
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, out=out, lse=lse)
    tp, npos = _table(table, D, q.device)
    sm = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _lib.check(lib().srt_attn_decode_splitk_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _dt(q), B, Hq, Hkv, Nk,
                                                    D, _ptr(seq_lens), int(num_splits), sm, tp, npos,
                                                    _pairing(pairing), int(window), int(sink), _ptr(out), _ptr(lse),
                                                    _stream(q.device)), "attn_decode_splitk_noalloc")
    return out, lse


def attn_decode_noalloc_max_workspace() -> int:
    """Bytes of split partials attn_decode_splitk_noalloc can hold."""
    return int(lib().srt_attn_decode_noalloc_max_workspace())


def _partition(p) -> int:
    if isinstance(p, str):
        if p not in PARTITIONS:
            raise ValueError(f"unknown partition {p!r}")
        return PARTITIONS[p]
    return int(p)


def attn_ring_workspace_size(B: int, Hq: int, Hkv: int, N: int, D: int, dtype: torch.dtype, num_devices: int,
                             partition="contiguous", rope_flags: int = ROTATE_Q | ROTATE_K) -> int:
    n = C.c_size_t()
    _lib.check(lib().srt_attn_ring_workspace_size(B, Hq, Hkv, N, D, F32 if dtype == torch.float32 else BF16,
                                                  int(num_devices), _partition(partition), int(rope_flags),
                                                  C.byref(n)), "attn_ring_workspace_size")
    return n.value


def attn_ring_prefill(q, k, v, *, num_devices: int, partition="contiguous", device: int = -1,
                      window: int = 0, sink: int = 0, sm_scale: float | None = None,
                      table: torch.Tensor | None = None, rope_flags: int | None = None,
                      workspace: torch.Tensor | None = None, out=None, lse=True):
    """Causal Ring Attention over num_devices devices run on this GPU.

    q [B, Hq, N, D], k/v [B, Hkv, N, D] contiguous, rows shard-major for the
    partition ("contiguous", "striped", "zigzag"); device=-1 runs all devices.
    rope_flags defaults to ROTATE_Q|ROTATE_K with a table (K rotated once into
    the workspace).  Returns (out [B, Hq, N, D] shard-major, lse [B, Hq, N])."""
    B, Hq, N, D = q.shape
    _, Hkv, _, _ = k.shape
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("ring tensors must be contiguous")
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k and v must be [B, Hkv, N, D] matching q")
    if rope_flags is None:
        rope_flags = (ROTATE_Q | ROTATE_K) if table is not None else 0
    need = attn_ring_workspace_size(B, Hq, Hkv, N, D, q.dtype, num_devices, partition, rope_flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is True:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N)):
        raise ValueError("lse must be contiguous fp32 [B, Hq, N]")
    _on_device(q.device, q=q, k=k, v=v, workspace=workspace, out=out, lse=lse)
    tp, npos = _table(table, D, q.device)
    sm = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _lib.check(lib().srt_attn_ring_prefill(_ptr(q), _ptr(k), _ptr(v), _dt(q), B, Hq, Hkv, N, D,
                                           int(num_devices), _partition(partition), int(device), int(window),
                                           int(sink), sm, tp, npos,
                                           int(rope_flags), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                                           _stream(q.device)), "attn_ring_prefill")
    return out, lse


def attn_backward_workspace_size(dtype: torch.dtype, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int,
                                 rope_flags: int) -> int:
    """Bytes of workspace attn_backward needs (delta, and rotated q / k copies for bf16)."""
    n = C.c_size_t()
    _lib.check(lib().srt_attn_backward_workspace_size(_dt(torch.empty(0, dtype=dtype)), B, Hq, Hkv, Nq, Nk, D,
                                                      int(rope_flags),
                                                      C.byref(n)), "attn_backward_workspace_size")
    return n.value


def attn_backward(q, k, v, out, dout, lse, *, sm_scale: float | None = None, causal: bool = True,
                  q_pos0: int = 0, k_pos0: int = 0, table: torch.Tensor | None = None,
                  rope_flags: int | None = None, window: int = 0, sink: int = 0,
                  workspace: torch.Tensor | None = None, dq=None, dk=None, dv=None):
    """Gradients of attn_prefill for upstream dout, given its out and lse.

    Same arguments as attn_prefill (rope_flags defaults to ROTATE_Q|ROTATE_K with
    a table; dq, dk are then gradients with respect to the raw q, k).  All
    tensors contiguous.  Returns (dq, dk, dv) in fp32."""
    B, Hq, Nq, D = q.shape
    _, Hkv, Nk, _ = k.shape
    for t in (q, k, v, out, dout, lse):
        if not t.is_contiguous():
            raise ValueError("backward tensors must be contiguous")
    if out.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("out, dout must be [B, Hq, Nq, D] and lse [B, Hq, Nq]")
    if lse.dtype != torch.float32:
        raise ValueError("lse must be fp32")
    if rope_flags is None:
        rope_flags = (ROTATE_Q | ROTATE_K) if table is not None else 0
    need = attn_backward_workspace_size(q.dtype, B, Hq, Hkv, Nq, Nk, D, rope_flags)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("gradient buffers must be contiguous fp32 of the input's shape")
    _on_device(q.device, q=q, k=k, v=v, out=out, dout=dout, lse=lse, workspace=workspace, dq=dq, dk=dk, dv=dv)
    tp, npos = _table(table, D, q.device)
    sm = 1.0 / math.sqrt(D) if sm_scale is None else float(sm_scale)
    _lib.check(lib().srt_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dt(q),
                                       B, Hq, Hkv, Nq, Nk, D, int(q_pos0), int(k_pos0), int(bool(causal)),
                                       int(window), int(sink), sm, tp,
                                       npos, int(rope_flags), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _stream(q.device)), "attn_backward")
    return dq, dk, dv
