"""Oracle, part 1: the RoPE frequency step and the rotation (numpy float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows "8.3 长上下文技术" §8.3.1: D is the head dimension, d (or i)
the pair index 0 .. D/2-1, b the base, s = L'/L the extension factor, L the
training length.
"""
from __future__ import annotations

import math

import numpy as np

NONE, PI, NTK, YARN = 0, 1, 2, 3

# band labels of the NTK-by-parts rule ("8.3 长上下文技术" §8.3.3)
BAND_LOW, BAND_MID, BAND_HIGH = 0, 1, 2


def base_inv_freq(D: int, base: float) -> np.ndarray:
    """theta_d = b^(-2d/D), d = 0 .. D/2-1.

    "Long Context: RoPE / YaRN / NTK / MLA" §2.1 (theta_i = b^{-2i/d}) and
    "8.3 长上下文技术" §8.3.1 (angular frequency of pair d).
    """
    if D % 2:
        raise ValueError("RoPE rotates pairs: D must be even")
    d = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * d / D)


def ntk_base(base: float, s: float, D: int) -> float:
    """NTK-aware base change b' = b * s^(D/(D-2)).

    "Long Context: RoPE / YaRN / NTK / MLA" §5.2: the lowest frequency is
    divided by s while theta_0 stays 1.
    """
    return float(base) * float(s) ** (D / (D - 2.0))


def yarn_ramp(r: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """Ramp clip((r - alpha) / (beta - alpha), 0, 1) of NTK-by-parts.

    "Long Context: RoPE / YaRN / NTK / MLA" §6.2 (called gamma there; it is
    the interpolation weight, 1 = keep theta, 0 = divide by s).
    """
    return np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)


def yarn_mscale(s: float) -> float:
    """sqrt(1/t) = 0.1 ln s + 1 for s > 1, else 1.

    "Long Context: RoPE / YaRN / NTK / MLA" §6.3 (fit), §6.6 (s <= 1 gives 1);
    "8.3 长上下文技术" §8.3.3 (temperature).
    """
    return 0.1 * math.log(s) + 1.0 if s > 1.0 else 1.0


def inv_freq(method: int, base: float, s: float = 1.0, L: float = 0.0,
             alpha: float = 1.0, beta: float = 32.0, D: int = 128):
    """Scaled frequencies theta'_d, the temperature factor and the band of each pair.

    Returns ``(theta_prime[D/2] float64, mscale float, band[D/2] int8)``.

    * NONE: theta' = theta.
    * PI:   theta' = theta / s        ("Long Context..." §4.2: m -> m/s is the
                                       same as theta -> theta/s).
    * NTK:  theta' = (b')^(-2d/D) with b' = b s^(D/(D-2))  (§5.2, §5.4).
    * YARN: the number of turns pair d makes within the training length,
            r_d = L theta_d / (2 pi) (§6.2; the ORIGINAL base, as §6.2 and
            "8.3 长上下文技术" §8.3.3 both state), sets the interpolation
            weight gamma_d = ramp(r_d) and theta'_d = gamma_d theta_d +
            (1 - gamma_d) theta_d / s (§6.2); mscale = 0.1 ln s + 1 (§6.3,
            folded into cos/sin by §6.4).
    band: YARN labels each pair by "8.3 长上下文技术" §8.3.3: high if
    r > beta (gamma = 1), low if r < alpha (gamma = 1/s), mid otherwise.
    The other methods have no bands; they are labelled by what their rule
    does to every pair: NONE all high (kept), PI all low (divided by s),
    NTK all mid (a blend between the two).
    """
    theta = base_inv_freq(D, base)
    h = D // 2
    if method == NONE:
        return theta.copy(), 1.0, np.full(h, BAND_HIGH, np.int8)
    if method == PI:
        return theta / s, 1.0, np.full(h, BAND_LOW, np.int8)
    if method == NTK:
        if D <= 2:
            raise ValueError("NTK-aware needs D > 2")
        return base_inv_freq(D, ntk_base(base, s, D)), 1.0, np.full(h, BAND_MID, np.int8)
    if method == YARN:
        if not beta > alpha:
            raise ValueError("YaRN needs beta > alpha")
        turns = L * theta / (2.0 * math.pi)          # r_d: turns of pair d over the training length
        gamma = yarn_ramp(turns, alpha, beta)        # 1: keep theta_d (many turns); 0: theta_d / s (few)
        theta_p = gamma * theta + (1.0 - gamma) * (theta / s)
        band = np.where(turns > beta, BAND_HIGH, np.where(turns < alpha, BAND_LOW, BAND_MID)).astype(np.int8)
        return theta_p, yarn_mscale(s), band
    raise ValueError(f"unknown rope method {method}")


def rotate(x: np.ndarray, pos, theta: np.ndarray, mscale: float = 1.0) -> np.ndarray:
    """Interleaved-pair RoPE: pair (x_{2i}, x_{2i+1}) at position p turns by p*theta_i.

    y_{2i}   = mscale (x_{2i} cos a - x_{2i+1} sin a)
    y_{2i+1} = mscale (x_{2i} sin a + x_{2i+1} cos a),   a = p theta_i.

    "Long Context: RoPE / YaRN / NTK / MLA" §2.2 (2-D rotation matrix per
    pair); "长上下文外推" §4.2 (counter-clockwise rotation formula) and §5.1
    (adjacent dims form a pair).  The angle is formed in fp64.

    x: [..., N, D]; pos: [N] integer positions (one per row).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    a = pos[:, None] * np.asarray(theta, dtype=np.float64)[None, :]      # [N, D/2]
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return mscale * y


def rotation_matrix(p: float, theta: np.ndarray) -> np.ndarray:
    """R_p = blkdiag(R_{theta_0, p}, ..., R_{theta_{D/2-1}, p}) as a dense D x D matrix.

    "Long Context: RoPE / YaRN / NTK / MLA" §2.2 (real matrix form).  Used by
    the brute-force attention, which never calls ``rotate``.
    """
    h = len(theta)
    R = np.zeros((2 * h, 2 * h))
    for i in range(h):
        a = p * float(theta[i])
        R[2 * i, 2 * i], R[2 * i, 2 * i + 1] = math.cos(a), -math.sin(a)
        R[2 * i + 1, 2 * i], R[2 * i + 1, 2 * i + 1] = math.sin(a), math.cos(a)
    return R


def over_extrapolated_range(D: int, L: float, s: float, base: float = 10000.0):
    """Real bounds of the pairs that NTK-aware scaling over-extrapolates.

    "8.3 长上下文技术" §8.3.2.  A pair d is over-extrapolated when
    (1) its wavelength 2 pi b^(2d/D) reaches L (no full period in training),
        i.e. d >= D/2 log_b(L / 2 pi), and
    (2) under gamma(d) = s^(-2d/(D-2)) the largest inference angle
        (L'-1) gamma(d) theta_d still exceeds the largest trained angle
        (L-1) theta_d, i.e. d < (D-2)/2 log_s((L'-1)/(L-1)), with L' = s L.
    The page prints the two bounds in the opposite order; as an interval the
    lower end is (1) and the upper end is (2).  Returns (lower, upper).
    """
    Lp = s * L
    lower = D / 2.0 * math.log(L / (2.0 * math.pi)) / math.log(base)
    upper = (D - 2) / 2.0 * math.log((Lp - 1.0) / (L - 1.0)) / math.log(s)
    return lower, upper


# --------------------------------------------------------------------------- frequency-step variants

def rotate_half(x: np.ndarray, pos, theta: np.ndarray, mscale: float = 1.0) -> np.ndarray:
    """Half-split pairing: pair i is (x_i, x_{i+D/2}), turned by p * theta_i.

    "Long Context: RoPE / YaRN / NTK / MLA" §2.4 (apply_rope: the first and the
    second half of the row form the real and imaginary parts; the page notes it
    is the interleaved rule up to a permutation of the dimensions).
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    pos = np.asarray(pos, dtype=np.float64)
    a = pos[:, None] * np.asarray(theta, dtype=np.float64)[None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :h], x[..., h:]
    return mscale * np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def dynamic_ntk_scale(seq_len: float, L: float) -> float:
    """Dynamic NTK: the scale follows the actual sequence length at inference.

    "AI Day 9: 长上下文技术" (Dynamic NTK: the base is adjusted from the actual
    length; short sequences lose nothing).  Reading: s = max(1, N / L) fed to
    the NTK-aware base change, so N <= L keeps the original base.
    """
    return max(1.0, float(seq_len) / float(L))


def inv_freq_dynamic_ntk(base: float, seq_len: float, L: float, D: int) -> np.ndarray:
    s = dynamic_ntk_scale(seq_len, L)
    return base_inv_freq(D, ntk_base(base, s, D))


def inv_freq_factors(base: float, lambdas, D: int) -> np.ndarray:
    """Per-dimension factors: theta'_i = theta_i / lambda_i.

    "Long Context: RoPE / YaRN / NTK / MLA" §7.3 (LongRoPE's search space; the
    search itself needs a trained model and is not part of this oracle).
    """
    lam = np.asarray(lambdas, dtype=np.float64)
    if lam.shape != (D // 2,):
        raise ValueError("one factor per pair")
    if not (lam > 0).all():
        raise ValueError("factors must be positive")
    return base_inv_freq(D, base) / lam
