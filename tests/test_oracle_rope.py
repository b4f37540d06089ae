"""Pins of the oracle's frequency step and rotation (CPU only).

Each test checks ``oracle.rope`` against something other than itself: values
printed on the pages (tests/golden), closed forms stated on the pages,
invariants of rotations, or an independent formulation (complex numbers,
the piecewise gamma(d) of a second page).
"""
import math

import numpy as np
import pytest

from conftest import half_ulp, read_golden
from oracle import rope

RNG = np.random.default_rng(20240601)


def _golden_kv(name):
    return {r[0]: r[1] for r in read_golden(name)}


# --------------------------------------------------------------------------- frequencies

def test_printed_frequency_table_d64():
    """"长上下文外推" §5.2 printed frequencies, degrees per step and period."""
    g = _golden_kv("rope_freq_d64_base1e4.txt")
    th = rope.base_inv_freq(64, 10000.0)
    assert len(th) == int(g["pairs"])
    for i in (0, 16, 31):
        assert abs(th[i] - float(g[f"theta_{i}"])) <= half_ulp(g[f"theta_{i}"])
        deg = math.degrees(th[i])
        assert abs(deg - float(g[f"deg_per_step_{i}"])) <= half_ulp(g[f"deg_per_step_{i}"])
    assert abs(2 * math.pi / th[31] - float(g["period_31"])) <= 0.5


def test_printed_slow_pair_angles():
    """"长上下文外推" §6.3: pair 31 reaches 31.3 deg at 4095 and 62.6 deg at 8191."""
    g = _golden_kv("slow_pair_angles.txt")
    th = rope.base_inv_freq(64, 10000.0)
    a_tr = math.degrees(4095 * th[31])
    a_ex = math.degrees(8191 * th[31])
    assert abs(a_tr - float(g["train_deg_4095"])) <= half_ulp(g["train_deg_4095"])
    assert abs(a_ex - float(g["extrap_deg_8191"])) <= half_ulp(g["extrap_deg_8191"])
    assert abs((a_ex - a_tr) - float(g["excess_deg"])) <= half_ulp(g["excess_deg"])
    turns = 4096 * th[0] / (2 * math.pi)
    assert round(turns) == int(g["turns_pair0_4096"])


def test_printed_ntk_rope_theta_table():
    """"长上下文外推" §15.1: NTK table from rope_theta = 1e6, head_dim 64, 32768 positions.

    The printed integers come from b * s^(64/62); the oracle's NTK frequencies
    must correspond to exactly that base (theta'_1 = b'^(-2/D))."""
    for tgt, scale, printed in read_golden("ntk_rope_theta_table.txt"):
        s = int(tgt) / 32768
        assert s == float(scale)
        th, msc, _ = rope.inv_freq(rope.NTK, 1e6, s, D=64)
        b_eff = th[1] ** (-64 / 2)                    # recover the base from theta'_1
        assert round(b_eff) == int(printed), (tgt, b_eff)
        assert msc == 1.0


def test_ntk_base_examples():
    """Order-of-magnitude and 1 % examples of the NTK base printed on two pages."""
    for row in read_golden("ntk_base_examples.txt"):
        key = row[0]
        if key == "hw1":
            base, D, s, exp_p, exp_tol, rel = float(row[1]), int(row[2]), float(row[3]), float(row[4]), float(row[5]), float(row[6])
            bp = rope.ntk_base(base, s, D)
            exponent = math.log(bp / base) / math.log(s)
            assert abs(exponent - exp_p) < exp_tol
            hint = base * s ** exp_p                  # the hint's own arithmetic with the printed 1.016
            assert abs(bp - hint) / hint < rel
            continue
        base, D, s, printed, rel = float(row[1]), int(row[2]), float(row[3]), float(row[4]), float(row[5])
        bp = rope.ntk_base(base, s, D)
        assert abs(bp - printed) / printed < rel, (key, bp)


def test_ntk_endpoints():
    """"Long Context..." §5.2: theta'_0 = theta_0 and theta'_{D/2-1} = theta_{D/2-1} / s."""
    for D in (8, 64, 128, 256):
        for s in (2.0, 4.0, 16.0, 40.0):
            th = rope.base_inv_freq(D, 10000.0)
            tp, _, _ = rope.inv_freq(rope.NTK, 10000.0, s, D=D)
            assert tp[0] == pytest.approx(th[0], rel=1e-14)
            assert tp[-1] == pytest.approx(th[-1] / s, rel=1e-12)
            # "8.3 长上下文技术" §8.3.2: theta' = theta * s^(-2d/(D-2)) pair by pair
            d = np.arange(D // 2)
            np.testing.assert_allclose(tp, th * s ** (-2.0 * d / (D - 2)), rtol=1e-12)


def test_pi_equals_position_division():
    """"Long Context..." §4.2: dividing theta by s equals rotating at position m/s."""
    D, s = 64, 16.0
    th = rope.base_inv_freq(D, 10000.0)
    tp, msc, band = rope.inv_freq(rope.PI, 10000.0, s, D=D)
    x = RNG.standard_normal((50, D))
    pos = RNG.integers(0, 200000, 50)
    np.testing.assert_allclose(rope.rotate(x, pos, tp), rope.rotate(x, pos / s, th), atol=1e-12)
    assert msc == 1.0 and (band == rope.BAND_LOW).all()


def _gamma_p5(r, alpha, beta, s):
    """The piecewise gamma(d) of "8.3 长上下文技术" §8.3.3, written independently."""
    out = np.empty_like(r)
    for j, rj in enumerate(r):
        if rj > beta:
            out[j] = 1.0
        elif rj < alpha:
            out[j] = 1.0 / s
        else:
            out[j] = (rj - alpha) / (beta - alpha) * (1.0 - 1.0 / s) + 1.0 / s
    return out


@pytest.mark.parametrize("D,base,L,s,alpha,beta", [
    (128, 10000.0, 2048.0, 16.0, 1.0, 32.0),
    (64, 10000.0, 4096.0, 8.0, 1.0, 32.0),
    (128, 500000.0, 8192.0, 4.0, 2.0, 16.0),
])
def test_yarn_two_pages_agree(D, base, L, s, alpha, beta):
    """Ramp form ("Long Context..." §6.2) == piecewise gamma(d) form ("8.3..." §8.3.3)."""
    th = rope.base_inv_freq(D, base)
    tp, msc, band = rope.inv_freq(rope.YARN, base, s, L, alpha, beta, D)
    r = L / (2 * math.pi * np.power(base, 2.0 * np.arange(D // 2) / D))   # r(d) = L / lambda_d
    np.testing.assert_allclose(tp, _gamma_p5(r, alpha, beta, s) * th, rtol=1e-14)
    assert msc == pytest.approx(0.1 * math.log(s) + 1.0, rel=1e-15)


def test_yarn_bands_32k_workload_exact():
    """Band of every pair at D=128, b=1e4, L=2048, alpha=1, beta=32 (exact).

    Inverting r(d) = L / (2 pi b^(2d/D)) against the thresholds gives the band
    edges in closed form: r > beta  <=>  d < D/2 log_b(L / (2 pi beta)),
    r < alpha <=>  d > D/2 log_b(L / (2 pi alpha)).  That is high 0..16,
    mid 17..40, low 41..63."""
    D, b, L, a, be = 128, 10000.0, 2048.0, 1.0, 32.0
    hi_edge = D / 2 * math.log(L / (2 * math.pi * be)) / math.log(b)     # 16.13
    lo_edge = D / 2 * math.log(L / (2 * math.pi * a)) / math.log(b)      # 40.21
    expect = np.array([2 if d < hi_edge else (0 if d > lo_edge else 1) for d in range(D // 2)], np.int8)
    _, _, band = rope.inv_freq(rope.YARN, b, 16.0, L, a, be, D)
    np.testing.assert_array_equal(band, expect)
    assert list(np.flatnonzero(band == 2)) == list(range(0, 17))
    assert list(np.flatnonzero(band == 1)) == list(range(17, 41))
    assert list(np.flatnonzero(band == 0)) == list(range(41, 64))


def test_yarn_limits():
    """"Long Context..." §6.2: r >= beta keeps theta; r <= alpha divides by s."""
    D, b, L, s = 128, 10000.0, 2048.0, 16.0
    th = rope.base_inv_freq(D, b)
    tp, _, band = rope.inv_freq(rope.YARN, b, s, L, 1.0, 32.0, D)
    np.testing.assert_allclose(tp[band == 2], th[band == 2], rtol=1e-15)
    np.testing.assert_allclose(tp[band == 0], th[band == 0] / s, rtol=1e-15)
    mid = band == 1
    assert ((tp[mid] < th[mid]) & (tp[mid] > th[mid] / s)).all()


def test_yarn_temperature_printed():
    """"Long Context..." §6.3: s = 8 gives sqrt(1/t) ≈ 1.21 and t ≈ 0.68; s <= 1 gives 1 (§6.6)."""
    for key, s, printed, tol in read_golden("yarn_temperature.txt"):
        m = rope.yarn_mscale(float(s))
        val = m if key.startswith("mscale") else 1.0 / m ** 2
        assert abs(val - float(printed)) <= float(tol), (key, val)
    assert rope.yarn_mscale(1.0) == 1.0 and rope.yarn_mscale(0.5) == 1.0
    _, msc, _ = rope.inv_freq(rope.YARN, 1e4, 16.0, 2048.0, 1.0, 32.0, 128)
    assert abs(msc - (0.1 * math.log(16) + 1)) < 1e-15 and 1.27 < msc < 1.28


def test_over_extrapolated_range_printed_and_brute_force():
    """"8.3 长上下文技术" §8.3.2 example (D=128, L=4096, s=40): printed [45, 63).

    The pairs are found again by brute force from the two conditions the page
    states (no full period in training; largest NTK-aware angle beyond the
    largest trained one)."""
    (_, D, L, s, base, plo, phi), = read_golden("over_extrapolated_range.txt")
    D, L, s, base = int(D), float(L), float(s), float(base)
    lo, hi = rope.over_extrapolated_range(D, L, s, base)
    assert math.floor(lo) == int(plo) and math.floor(hi) == int(phi)
    th = rope.base_inv_freq(D, base)
    Lp = s * L
    over = []
    for d in range(D // 2):
        no_period = 2 * math.pi / th[d] >= L
        gamma = s ** (-2.0 * d / (D - 2))
        beyond = (Lp - 1) * gamma * th[d] > (L - 1) * th[d]
        if no_period and beyond:
            over.append(d)
    assert over == [d for d in range(D // 2) if lo <= d < hi]
    assert over[0] == 46 and over[-1] == 63


def test_methods_validate():
    with pytest.raises(ValueError):
        rope.base_inv_freq(63, 1e4)
    with pytest.raises(ValueError):
        rope.inv_freq(rope.YARN, 1e4, 16.0, 2048.0, 32.0, 1.0, 128)
    with pytest.raises(ValueError):
        rope.inv_freq(7, 1e4, 16.0, D=128)


# --------------------------------------------------------------------------- rotation

def test_rotation_matches_complex_multiplication():
    """"Long Context..." §2.1: f(x, m) = x ⊙ e^{i m theta} with pairs packed as x_{2i} + i x_{2i+1}."""
    D = 16
    th = rope.base_inv_freq(D, 10000.0)
    x = RNG.standard_normal((7, D))
    pos = np.array([0, 1, 2, 5, 100, 4095, 131071])
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * th[None, :])
    y = rope.rotate(x, pos, th)
    np.testing.assert_allclose(y[:, 0::2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], z.imag, atol=1e-12)


def test_rotation_direction_and_pairing():
    """"长上下文外推" §4.2: counter-clockwise: e_{2i} turned by 90 deg is e_{2i+1}.

    Only pair i moves, by p * theta_i (adjacent dims form a pair, §5.1)."""
    D = 8
    th = np.array([math.pi / 2, 0.3, 0.01, 1e-4])
    for i in range(D // 2):
        x = np.zeros((1, D))
        x[0, 2 * i] = 1.0
        p = (math.pi / 2) / th[i]
        y = rope.rotate(x, [p], th)[0]
        expect = np.zeros(D)
        expect[2 * i + 1] = 1.0
        np.testing.assert_allclose(y, expect, atol=1e-9)


def test_rotation_preserves_norm_and_scales_by_mscale():
    """"长上下文外推" §4.2: ||R v|| = ||v||; YaRN multiplies by sqrt(1/t)."""
    D = 128
    th, msc, _ = rope.inv_freq(rope.YARN, 1e4, 16.0, 2048.0, 1.0, 32.0, D)
    x = RNG.standard_normal((64, D))
    pos = RNG.integers(0, 1 << 17, 64)
    n0 = np.linalg.norm(x, axis=1)
    np.testing.assert_allclose(np.linalg.norm(rope.rotate(x, pos, th), axis=1), n0, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(rope.rotate(x, pos, th, msc), axis=1), msc * n0, rtol=1e-13)


def test_relative_position_property():
    """"Long Context..." §2.2: <R_m q, R_n k> depends only on n - m."""
    D = 64
    th = rope.base_inv_freq(D, 10000.0)
    for _ in range(20):
        q, k = RNG.standard_normal(D), RNG.standard_normal(D)
        m, n, delta = (int(v) for v in RNG.integers(0, 100000, 3))
        a = rope.rotate(q[None], [m], th)[0] @ rope.rotate(k[None], [n], th)[0]
        b = rope.rotate(q[None], [m + delta], th)[0] @ rope.rotate(k[None], [n + delta], th)[0]
        assert abs(a - b) <= 1e-10 * (abs(a) + np.linalg.norm(q) * np.linalg.norm(k))


def test_worked_2d_example():
    """"长上下文外推" §4.2: q = k = (1,1), theta = 15 deg.

    (m,n) = (2,5), (10,13), (0,3) all give 2 cos 45 deg = sqrt 2; (2,6) gives
    2 cos 60 deg = 1; unrotated q.k = 2."""
    th = np.array([math.pi / 12])
    q = np.array([[1.0, 1.0]])
    dot = lambda m, n: float(rope.rotate(q, [m], th)[0] @ rope.rotate(q, [n], th)[0])
    for m, n in ((2, 5), (10, 13), (0, 3)):
        assert dot(m, n) == pytest.approx(math.sqrt(2), abs=1e-12)
    assert dot(2, 6) == pytest.approx(1.0, abs=1e-12)
    assert dot(0, 0) == pytest.approx(2.0, abs=1e-12)


def test_rotation_matrix_form_equals_pairwise_form():
    """Block-diagonal matrix form (§2.2) and the pairwise formula agree; R_m^T R_n = R_{n-m}."""
    D = 16
    th = rope.base_inv_freq(D, 500000.0)
    x = RNG.standard_normal(D)
    for p in (0, 3, 1000, 131071):
        np.testing.assert_allclose(rope.rotation_matrix(p, th) @ x, rope.rotate(x[None], [p], th)[0], atol=1e-11)
    Rm, Rn, Rd = (rope.rotation_matrix(p, th) for p in (17, 40, 23))
    np.testing.assert_allclose(Rm.T @ Rn, Rd, atol=1e-12)


def test_homework_angle():
    """"长上下文外推" homework 2: base 1e4, d = 4, pair 0 at m = 100 turns 100 rad."""
    th = rope.base_inv_freq(4, 10000.0)
    assert 100 * th[0] == 100.0
    assert 0 * th[0] == 0.0


# --------------------------------------------------------------------------- frequency-step variants

def test_rotate_half_matches_complex_form_and_permutation():
    """"Long Context..." §2.4: half-split pairs (x_i, x_{i+D/2}) are the interleaved rule on permuted dims."""
    D = 16
    th = rope.base_inv_freq(D, 10000.0)
    x = RNG.standard_normal((9, D))
    pos = np.array([0, 1, 2, 7, 100, 4095, 8191, 65536, 131071])
    y = rope.rotate_half(x, pos, th, 1.3)
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * th[None, :]) * 1.3
    np.testing.assert_allclose(y[:, :D // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, D // 2:], z.imag, atol=1e-12)
    perm = np.empty(D, dtype=int)             # interleaved slot 2i <- half slot i, 2i+1 <- i + D/2
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    np.testing.assert_allclose(rope.rotate(x[:, perm], pos, th, 1.3), y[:, perm], atol=1e-12)
    # on random data the two pairings give different vectors: the table must match the pairing
    assert np.abs(rope.rotate(x, pos, th) - rope.rotate_half(x, pos, th)).max() > 0.1


def test_dynamic_ntk_follows_length():
    """Short sequences keep the original base; at N = s L it is the NTK-aware base for s."""
    D, b, L = 128, 10000.0, 8192.0
    np.testing.assert_array_equal(rope.inv_freq_dynamic_ntk(b, 100, L, D), rope.base_inv_freq(D, b))
    np.testing.assert_array_equal(rope.inv_freq_dynamic_ntk(b, L, L, D), rope.base_inv_freq(D, b))
    th16, _, _ = rope.inv_freq(rope.NTK, b, 16.0, D=D)
    np.testing.assert_allclose(rope.inv_freq_dynamic_ntk(b, 16 * L, L, D), th16, rtol=1e-14)
    # the printed example of the NTK base for 8K -> 128K holds for the dynamic rule at N = 128K
    b_eff = rope.inv_freq_dynamic_ntk(b, 131072, L, D)[1] ** (-D / 2)
    assert 1.6e5 < b_eff < 1.8e5


def test_factor_table_reduces_to_pi_ntk_none():
    """theta / lambda: lambda = s gives PI, lambda_i = s^(2i/(D-2)) gives NTK-aware, lambda = 1 gives RoPE."""
    D, b, s = 64, 10000.0, 8.0
    d = np.arange(D // 2)
    th_pi, _, _ = rope.inv_freq(rope.PI, b, s, D=D)
    th_ntk, _, _ = rope.inv_freq(rope.NTK, b, s, D=D)
    np.testing.assert_allclose(rope.inv_freq_factors(b, np.full(D // 2, s), D), th_pi, rtol=1e-15)
    np.testing.assert_allclose(rope.inv_freq_factors(b, s ** (2.0 * d / (D - 2)), D), th_ntk, rtol=1e-13)
    np.testing.assert_array_equal(rope.inv_freq_factors(b, np.ones(D // 2), D), rope.base_inv_freq(D, b))
    with pytest.raises(ValueError):
        rope.inv_freq_factors(b, np.zeros(D // 2), D)
