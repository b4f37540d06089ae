"""Host-side checks of libsrt.so (no GPU): exported symbols, the fp64
frequency step against the oracle, and argument validation that returns
before anything is enqueued."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import rope as orope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def srt():
    if not os.path.exists(os.path.join(ROOT, "scaled_rope_tiled_amd", "libsrt.so")):
        import __graft_entry__
        __graft_entry__.build()
    import scaled_rope_tiled_amd as m
    return m


def _declared():
    src = open(os.path.join(ROOT, "include", "srt.h"), encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(srt_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(srt):
    names = _declared()
    assert len(names) >= 9
    lib = srt.lib()
    for n in names:
        assert hasattr(lib, n), n
    from scaled_rope_tiled_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_status_strings(srt):
    lib = srt.lib()
    assert lib.srt_abi_version() == 2
    for s in range(5):
        assert lib.srt_status_string(s)
    assert lib.srt_status_string(99) == b"unknown status"


CASES = [
    (orope.NONE, 10000.0, 1.0, 0.0, 1.0, 32.0, 64),
    (orope.NONE, 500000.0, 1.0, 0.0, 1.0, 32.0, 128),
    (orope.PI, 10000.0, 16.0, 0.0, 1.0, 32.0, 128),
    (orope.NTK, 10000.0, 16.0, 0.0, 1.0, 32.0, 128),
    (orope.NTK, 1e6, 4.0, 0.0, 1.0, 32.0, 64),
    (orope.YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0, 128),
    (orope.YARN, 10000.0, 8.0, 4096.0, 1.0, 32.0, 64),
    (orope.YARN, 500000.0, 0.5, 8192.0, 2.0, 16.0, 128),
]


@pytest.mark.parametrize("case", CASES)
def test_inv_freq_matches_oracle(srt, case):
    """Bands exact; theta' within 1e-15 relative; mscale exact to 1e-15."""
    th, ms, band = srt.rope_inv_freq(*case)
    oth, oms, oband = orope.inv_freq(*case)
    np.testing.assert_array_equal(band, oband)
    np.testing.assert_allclose(th, oth, rtol=1e-15, atol=0)
    assert abs(ms - oms) <= 1e-15


def test_yarn_32k_band_classification_exact(srt):
    _, _, band = srt.rope_inv_freq(srt.YARN, 10000.0, 16.0, 2048.0, 1.0, 32.0, 128)
    assert list(np.flatnonzero(band == 2)) == list(range(17))
    assert list(np.flatnonzero(band == 1)) == list(range(17, 41))
    assert list(np.flatnonzero(band == 0)) == list(range(41, 64))


@pytest.mark.parametrize("args,frag", [
    ((3, 1e4, 16.0, 2048.0, 32.0, 1.0, 128), "beta > alpha"),
    ((0, 1e4, 1.0, 0.0, 1.0, 32.0, 63), "even"),
    ((0, -1.0, 1.0, 0.0, 1.0, 32.0, 64), "base"),
    ((9, 1e4, 1.0, 0.0, 1.0, 32.0, 64), "unknown method"),
    ((1, 1e4, 0.0, 0.0, 1.0, 32.0, 64), "scale"),
    ((3, 1e4, 16.0, 0.0, 1.0, 32.0, 64), "L > 0"),
])
def test_inv_freq_validation(srt, args, frag):
    from scaled_rope_tiled_amd._lib import SrtError
    with pytest.raises(SrtError, match=frag) as e:
        srt.rope_inv_freq(*args)
    assert e.value.status == 1


def test_abi_rejects_before_launch(srt):
    """Argument errors return SRT_ERR_INVALID / UNSUPPORTED with no GPU call."""
    lib = srt.lib()
    fake = C.c_void_p(0x100000)      # never dereferenced: every call below fails validation first
    st = lib.srt_attn_prefill(None, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, 0, 0, 0.1,
                              None, 0, 0, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"NULL" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 3, 8, 8, 128, 1024, 1024, 0, 0, 1, 0, 0, 0.1,
                              None, 0, 0, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"multiple" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 96, 768, 768, 0, 0, 1, 0, 0, 0.1,
                              None, 0, 0, fake, 1, 768, None, 0, None, None)
    assert st == 2
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, 0, 0, 0.1,
                              None, 0, 3, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"table" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, 0, 0, 0.1,
                              fake, 4, 3, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"outside table" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 0, 16, 0, 0.1,
                              None, 0, 0, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"causal" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, -1, 0, 0.1,
                              None, 0, 0, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"window" in lib.srt_last_error()
    st = lib.srt_attn_prefill(fake, fake, fake, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, 16, -4, 0.1,
                              None, 0, 0, fake, 1, 1024, None, 0, None, None)
    assert st == 1 and b"sink" in lib.srt_last_error()
    st = lib.srt_rope_apply(fake, fake, 1, 1, 1, 8, 128, 5, fake, 10, 0, None)
    assert st == 1 and b"outside table" in lib.srt_last_error()
    st = lib.srt_rope_apply(fake, fake, 7, 1, 1, 8, 128, 0, fake, 10, 0, None)
    assert st == 1
    st = lib.srt_rope_apply(fake, fake, 1, 1, 1, 8, 128, 0, fake, 10, 2, None)
    assert st == 1 and b"pairing" in lib.srt_last_error()
    st = lib.srt_rope_apply(fake, fake, 1, 1, 1, 8, 40, 0, fake, 10, 1, None)
    assert st in (1, 2)
    n = C.c_size_t()
    assert lib.srt_attn_decode_workspace_size(16, 32, 128, 64, C.byref(n)) == 0
    assert n.value == 16 * 32 * 64 * 129 * 4
    st = lib.srt_attn_decode_splitk(fake, fake, fake, 1, 16, 32, 8, 1024, 128, None, 64, 0.1, None, 0, 0, 0, 0,
                                    fake, n.value - 1, fake, None, None)
    assert st == 4
    st = lib.srt_attn_decode_splitk(fake, fake, fake, 1, 16, 24, 8, 1024, 128, None, 64, 0.1, None, 0, 0, 0, 0,
                                    fake, n.value, fake, None, None)
    assert st == 2
    st = lib.srt_attn_decode_splitk(fake, fake, fake, 1, 16, 32, 8, 1024, 128, None, 0, 0.1, None, 0, 0, 0, 0,
                                    fake, n.value, fake, None, None)
    assert st == 1
    st = lib.srt_attn_decode_splitk(fake, fake, fake, 1, 16, 32, 8, 1024, 128, None, 64, 0.1, None, 0, 0, -1, 0,
                                    fake, n.value, fake, None, None)
    assert st == 1 and b"window" in lib.srt_last_error()
    st = lib.srt_attn_merge_states(fake, fake, fake, fake, 0, 64, fake, 1, 128, None, 0, 1, 1, 1, 128, None)
    assert st == 1 and b"stride" in lib.srt_last_error()
    st = lib.srt_attn_merge_states(fake, fake, fake, fake, 0, 96, fake, 0, 96, None, 0, 1, 1, 1, 96, None)
    assert st == 2
    # backward: workspace size, bad D, window without causal, missing workspace
    # delta (fp32 [B][Hq][Nq]), then for bf16 the rotated q and k copies and two 128-byte scheduling
    # blocks, each region 256-byte aligned
    ws = lambda *args: (lib.srt_attn_backward_workspace_size(*args, C.byref(n)), n.value)
    assert ws(0, 2, 8, 2, 100, 50, 64, 3) == (0, 6400)
    qcopy = 2 * 8 * 100 * 128 * 2               # bf16 always keeps a scaled copy of q
    sched = 256
    assert ws(1, 2, 8, 2, 100, 50, 128, 0) == (0, 6400 + qcopy + sched)
    assert ws(1, 2, 8, 2, 100, 50, 128, 1) == (0, 6400 + qcopy + sched)
    assert ws(1, 2, 8, 2, 100, 50, 128, 2) == (0, 6400 + qcopy + 2 * 2 * 50 * 128 * 2 + sched)
    assert ws(1, 2, 8, 2, 0, 50, 128, 3) == (0, 2 * 2 * 50 * 128 * 2)
    assert ws(1, 1, 1, 1, 3, 5, 128, 7) == (0, 256 + 768 + 1280 + sched)
    assert ws(1, 2, 8, 2, 100, 50, 128, 8)[0] == 1 and b"rope_flags" in lib.srt_last_error()
    assert ws(2, 2, 8, 2, 100, 50, 128, 0)[0] == 1
    bw = lambda dt, D, causal, window, ws, wsb: lib.srt_attn_backward(
        fake, fake, fake, fake, fake, fake, dt, 1, 8, 2, 64, 64, D, 0, 0, causal, window, 0, 0.1, None, 0, 0,
        ws, wsb, fake, fake, fake, None)
    assert bw(1, 64, 1, 0, fake, 1 << 20) == 2
    assert bw(0, 128, 1, 0, fake, 1 << 20) == 2
    assert bw(1, 128, 0, 16, fake, 1 << 20) == 1 and b"causal" in lib.srt_last_error()
    assert bw(1, 128, 1, 0, None, 0) == 4
    th = (C.c_double * 4)(1.0, 0.1, 0.01, float("inf"))
    st = lib.srt_rope_cos_sin(th, 8, 1.0, 16, fake, None)
    assert st == 1 and b"finite" in lib.srt_last_error()


@pytest.mark.parametrize("base,seq_len,L,D", [
    (10000.0, 1000, 2048.0, 128),      # shorter than L: original frequencies
    (10000.0, 2048, 2048.0, 128),      # exactly L
    (10000.0, 32768, 2048.0, 128),     # s = 16
    (500000.0, 12345, 4096.0, 64),     # non-integer s
])
def test_dynamic_ntk_matches_oracle(srt, base, seq_len, L, D):
    th, s = srt.rope_inv_freq_dynamic_ntk(base, seq_len, L, D)
    assert s == pytest.approx(orope.dynamic_ntk_scale(seq_len, L), rel=1e-15)
    np.testing.assert_allclose(th, orope.inv_freq_dynamic_ntk(base, seq_len, L, D), rtol=1e-15, atol=0)


def test_factors_match_oracle(srt):
    lam = 1.0 + np.random.default_rng(3).random(64) * 15.0
    np.testing.assert_allclose(srt.rope_inv_freq_factors(1e4, lam, 128), orope.inv_freq_factors(1e4, lam, 128),
                               rtol=1e-15, atol=0)
    from scaled_rope_tiled_amd._lib import SrtError
    bad = lam.copy()
    bad[5] = 0.0
    with pytest.raises(SrtError):
        srt.rope_inv_freq_factors(1e4, bad, 128)
    bad[5] = float("nan")
    with pytest.raises(SrtError):
        srt.rope_inv_freq_factors(1e4, bad, 128)


def test_empty_problems_return_ok_without_pointers(srt):
    """An empty problem (no row, no sequence) is a successful no-op: every entry
    point returns SRT_OK before it looks at a pointer or touches the device, so
    NULL pointers and a null stream are accepted (this runs with no GPU)."""
    lib = srt.lib()
    assert lib.srt_rope_apply(None, None, 1, 1, 4, 0, 128, 0, None, 0, 0, None) == 0
    assert lib.srt_rope_apply(None, None, 0, 0, 4, 16, 128, 0, None, 0, 0, None) == 0
    # prefill: no query row (Nq = 0), then no batch
    assert lib.srt_attn_prefill(None, None, None, 1, 1, 4, 2, 0, 64, 128, 0, 0, 0, 0, 1, 0, 0, 0.1,
                                None, 0, 0, None, 1, 0, None, 0, None, None) == 0
    assert lib.srt_attn_prefill(None, None, None, 1, 0, 4, 2, 64, 64, 128, 0, 0, 0, 0, 1, 0, 0, 0.1,
                                None, 0, 0, None, 1, 0, None, 0, None, None) == 0
    assert lib.srt_attn_merge_states(None, None, None, None, 0, 0, None, 1, 0, None, 0, 1, 4, 0, 128, None) == 0
    assert lib.srt_attn_decode_splitk(None, None, None, 1, 0, 32, 8, 1024, 128, None, 64, 0.1, None, 0, 0, 0, 0,
                                      None, 0, None, None, None) == 0
    assert lib.srt_attn_ring_prefill(None, None, None, 1, 1, 32, 8, 0, 128, 8, 0, -1, 0, 0, 0.1, None, 0, 0,
                                     None, 0, None, None, None) == 0
    assert lib.srt_attn_backward(None, None, None, None, None, None, 1, 0, 8, 2, 64, 64, 128, 0, 0, 1, 0, 0, 0.1,
                                 None, 0, 0, None, 0, None, None, None, None) == 0
    # sizes are still validated first: a negative size is an error even when the problem is empty
    assert lib.srt_attn_prefill(None, None, None, 1, 1, 4, 2, -1, 64, 128, 0, 0, 0, 0, 1, 0, 0, 0.1,
                                None, 0, 0, None, 1, 0, None, 0, None, None) == 1
    assert lib.srt_attn_merge_states(None, None, None, None, 0, 0, None, 1, 0, None, 0, 1, -4, 0, 128, None) == 1


def test_prefill_rejects_misaligned_pointers_and_strides(srt):
    """The kernels move q/k/v/out rows and table entries in 16-byte vectors:
    a base pointer off a 16-byte boundary or a head stride that is not a
    multiple of 8 elements is SRT_ERR_INVALID before anything is enqueued."""
    lib = srt.lib()
    good = C.c_void_p(0x100000)
    odd = C.c_void_p(0x100008)         # 8-byte aligned only
    call = lambda q, k, v, out, tab, flags, qs, ks, os_: lib.srt_attn_prefill(
        q, k, v, 1, 1, 4, 2, 8, 8, 128, qs, ks, 0, 0, 1, 0, 0, 0.1, tab, 64 if tab else 0, flags, out, 1, os_,
        None, 0, None, None)
    for args in ((odd, good, good, good, None, 0), (good, odd, good, good, None, 0),
                 (good, good, odd, good, None, 0), (good, good, good, odd, None, 0),
                 (good, good, good, good, odd, 1)):
        assert call(*args, 1024, 1024, 1024) == 1 and b"aligned" in lib.srt_last_error(), args
    for qs, ks, os_ in ((1028, 1024, 1024), (1024, 1028, 1024), (1024, 1024, 1028)):
        assert call(good, good, good, good, None, 0, qs, ks, os_) == 1
        assert b"multiples of 8" in lib.srt_last_error()
    # the scheduling block: 8-byte alignment
    assert lib.srt_attn_prefill(good, good, good, 1, 1, 4, 2, 8, 8, 128, 1024, 1024, 0, 0, 1, 0, 0, 0.1, None, 0, 0,
                                good, 1, 1024, None, 0, C.c_void_p(0x100004), None) == 1
    assert b"sched" in lib.srt_last_error()


def test_binding_rejects_host_tensors_and_wrong_tables(srt):
    """The binding hands raw pointers to the library: every tensor must be on
    q's GPU and the table must be a contiguous fp32 [npos, D/2, 2] for this D.
    Host (CPU) tensors fail before any call, with no GPU in this process."""
    import torch
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="cpu"):
        srt.attn_prefill(q, k, k)
    with pytest.raises(ValueError, match="cpu"):
        srt.rope_apply(k, torch.zeros(8, 64, 2))
    with pytest.raises(ValueError, match="cpu"):
        srt.attn_decode_splitk(q[:, :, 0].contiguous(), k, k, num_splits=2)

    class FakeCuda:
        """Stands in for a device tensor so the table-shape checks run without a GPU."""
        def __init__(self, shape, dtype=torch.float32, contiguous=True):
            self.shape, self.dtype, self._c = torch.Size(shape), dtype, contiguous
            self.is_cuda, self.device = True, torch.device("cuda:0")

        def is_contiguous(self):
            return self._c

        def dim(self):
            return len(self.shape)

        def data_ptr(self):
            return 0x100000

    dev = torch.device("cuda:0")
    assert srt._table(FakeCuda((64, 64, 2)), 128, dev)[1] == 64
    for bad in (FakeCuda((64, 32, 2)), FakeCuda((64, 64, 2), torch.float16), FakeCuda((64, 64, 2), contiguous=False),
                FakeCuda((64, 128))):
        with pytest.raises(ValueError, match="table"):
            srt._table(bad, 128, dev)
    with pytest.raises(ValueError, match="cuda:1"):
        other = FakeCuda((64, 64, 2))
        other.device = torch.device("cuda:1")
        srt._table(other, 128, dev)


def test_noalloc_decode_rejects_oversize_before_any_gpu_call(srt):
    """The allocation-free decode holds at most its static scratch of split
    partials: a larger problem is SRT_ERR_WORKSPACE before anything runs (this
    process has no GPU); an empty problem is a no-op."""
    lib = srt.lib()
    cap = lib.srt_attn_decode_noalloc_max_workspace()
    assert cap == 32 << 20
    fake = C.c_void_p(0x100000)
    # 16 x 32 x 64 splits x 129 x 4 = 16.9 MB fits; 64 x 32 x 64 x 129 x 4 = 67.6 MB does not
    st = lib.srt_attn_decode_splitk_noalloc(fake, fake, fake, 1, 64, 32, 8, 1024, 128, None, 64, 0.1, None, 0,
                                            0, 0, 0, fake, None, None)
    assert st == 4 and b"static scratch" in lib.srt_last_error()
    st = lib.srt_attn_decode_splitk_noalloc(None, None, None, 1, 0, 32, 8, 1024, 128, None, 64, 0.1, None, 0,
                                            0, 0, 0, None, None, None)
    assert st == 0
    st = lib.srt_attn_decode_splitk_noalloc(fake, fake, fake, 1, 16, 24, 8, 1024, 128, None, 64, 0.1, None, 0,
                                            0, 0, 0, fake, None, None)
    assert st == 2
