"""CPU models of arithmetic shortcuts the HIP kernels take, checked against the oracle.

These tests need no GPU: each one restates, in float32 numpy, a rule a kernel
uses in place of the plain definition, and compares its decisions with the
oracle's (which the pin tests tie to exact rational brute force).

Midpoint candidate search (activation encoder).  "RaZeR summary" (gist.science
technical summary of "RaZeR: Pushing the Limits of NVFP4 Quantization with
Redundant Zero Remapping"), §2.2: an activation block picks one of the two
special values +M, -M by the lower block squared error.  When M lies halfway
between its FP4 neighbours (M = 2.5, 3.5, 5 with half-gap h = 0.5, 0.5, 1), an
element y moves to sign(y) * M iff |u| < h / 2 with u = |y| - M, and the move
changes the error by -h * (h - 2|u|) whichever neighbour y rounds to.  The
kernel therefore sums sign(y) * max(h - 2|u|, 0) over the block in fp32
(exact: every term is a multiple of 2^-21 of magnitude at most 1) and picks -M
iff the sum is negative.
"""
import numpy as np
import pytest

import oracle

MIDPOINTS = [(5.0, 1.0), (3.5, 0.5), (2.5, 0.5)]


def _kernel_midpoint_rule(y, m, h):
    """The kernel's fp32 steps for one block: (candidate index, window mask)."""
    y = np.asarray(y, dtype=np.float32)
    m32, h32, two = np.float32(m), np.float32(h), np.float32(2.0)
    dsum = np.float32(0.0)
    window = []
    for v in y[::-1]:  # the kernel's order (any order gives the same exact sum)
        u = np.float32(abs(v)) - m32
        e = h32 - two * np.float32(abs(u))  # the kernel's fma; exact where it matters
        t = max(e, np.float32(0.0))
        dsum = np.float32(dsum + (-t if np.signbit(v) else t))
        window.append(bool(e > 0))
    return (1 if dsum < 0 else 0), window[::-1]


def _blocks(m, h, n, seed):
    """Blocks of 16 scaled values, many placed on the window edges, on M and
    within two ulps of them."""
    rng = np.random.default_rng(seed)
    edges = [m - h / 2, m + h / 2, m, m - h / 4, m + h / 4]
    for _ in range(n):
        y = (rng.normal(0.0, 1.5, 16) * (m / 3)).astype(np.float32)
        for i in rng.choice(16, int(rng.integers(1, 9)), replace=False):
            if rng.integers(4) == 0:
                v = np.float32(m - h / 2 + rng.random() * h)
            else:
                v = np.float32(edges[rng.integers(len(edges))])
                k = int(rng.integers(-2, 3))
                for _ in range(abs(k)):
                    v = np.nextafter(v, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            y[i] = -v if rng.integers(2) else v
        yield y


@pytest.mark.parametrize("m,h", MIDPOINTS)
def test_midpoint_search_matches_oracle_selection(m, h):
    n_neg = 0
    for y in _blocks(m, h, 400, seed=int(m * 10)):
        codes, sel = oracle.encode_block_scaled(y, [m, -m])
        ksel, window = _kernel_midpoint_rule(y, m, h)
        assert ksel == sel, (y.tolist(), m)
        # the remap step: window elements whose sign matches the chosen
        # candidate become code 0b1000
        moved = [w and (bool(np.signbit(v)) == (sel == 1)) for v, w in zip(y, window)]
        assert [c == 8 for c in codes.tolist()] == moved, (y.tolist(), m)
        n_neg += sel
    assert 0 < n_neg < 400  # both candidates are exercised


def test_midpoint_rule_applies_only_to_midpoint_candidates():
    # the candidates the encoder sends down this path: M halfway between its
    # FP4 neighbours; every other offset in [-7, 7] keeps the integer search
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    found = []
    for off in range(-7, 8):
        m = 6.0 + off / 2.0
        below = max(g for g in grid if g < m) if m > 0 else None
        above = [g for g in grid if g > m]
        if m in grid or not above:
            continue
        if m - below == above[0] - m:
            found.append((m, above[0] - m))
    assert found == [(2.5, 0.5), (3.5, 0.5), (5.0, 1.0)]


# ---- block-scale quotient (activation encoder, 16-bit inputs) ----------------
# "RaZeR summary" §2.1: the block scale code is the nearest-even E4M3 value of
# S_MAX * amax_b / amax, the quotient an IEEE fp32 division.  For bf16 and fp16
# inputs the kernel forms it from rinv = RN(1 / amax) by Markstein's correction:
# q0 = RN(amax_b * rinv), e = amax_b - q0 * amax (one fma, exact), q =
# RN(q0 + e * rinv) (one fma).  Both operands are 16-bit values, so every case
# is a pair of 8-bit (bf16) or 11-bit (fp16) significands and an exponent
# difference: scaling both operands by a power of two scales every step exactly
# while they stay normal (the kernel takes this path only for amax in
# [2^-60, 2^60]; below a quotient of 2^-19 the scale code is 0 whatever the
# last bit).  The test runs the kernel's steps on all such pairs and compares
# them with the correctly rounded quotient, both decided with exact arithmetic
# where a float64 intermediate lands on a float32 rounding midpoint.

def _rn32_from(g, sign_of_excess):
    """RN to float32 of a true value whose float64 rounding is g; where g is
    exactly a float32 midpoint, sign_of_excess() gives the sign of
    (true value - g) and decides the direction (0: ties to even)."""
    r = g.astype(np.float32)
    rb = r.astype(np.float64)
    toward = np.where(g > rb, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    other = np.nextafter(r, toward).astype(np.float64)
    mid = (g != rb) & (g == (rb + other) / 2)
    if mid.any():
        s = sign_of_excess()
        up = np.maximum(rb, other).astype(np.float32)
        dn = np.minimum(rb, other).astype(np.float32)
        r = np.where(mid & (s > 0), up, np.where(mid & (s < 0), dn, r))
    return r


def _rn32_div(num, den):
    g = num / den
    return _rn32_from(g, lambda: np.sign(num - den * g))  # den * g is exact (<= 53 bits)


def _markstein_mismatches(sig_bits, exps=range(0, -27, -1)):
    n = 1 << (sig_bits - 1)
    mant = np.arange(n, 2 * n, dtype=np.float64) / n  # every significand, in [1, 2)
    bad = total = 0
    for d in exps:
        a, b = np.meshgrid(mant * 2.0 ** d, mant, indexing="ij")
        a, b = a.ravel(), b.ravel()
        keep = a <= b  # amax_b never exceeds amax
        a, b = a[keep], b[keep]
        want = _rn32_div(a, b)
        rinv = _rn32_div(np.ones_like(b), b)
        q0 = a.astype(np.float32) * rinv  # float32 product, correctly rounded
        e64 = a - q0.astype(np.float64) * b  # exact: 24 + 11 bits of product
        e = e64.astype(np.float32)
        assert np.array_equal(e.astype(np.float64), e64), "the fma residual must be exact"
        p = e.astype(np.float64) * rinv.astype(np.float64)  # exact (48 bits)
        hi = q0.astype(np.float64) + p  # two-sum: hi + lo == q0 + p exactly
        bb = hi - q0.astype(np.float64)
        lo = (q0.astype(np.float64) - (hi - bb)) + (p - bb)
        got = _rn32_from(hi, lambda: np.sign(lo))
        bad += int(np.count_nonzero(got != want))
        total += a.size
    return bad, total


@pytest.mark.parametrize("sig_bits", [8, 11], ids=["bf16", "fp16"])
def test_markstein_quotient_is_the_ieee_quotient(sig_bits):
    bad, total = _markstein_mismatches(sig_bits)
    assert total > 0 and bad == 0, f"{bad} of {total} quotients differ"


def test_markstein_model_sees_a_missing_correction():
    """The model is not vacuous: the uncorrected product q0 misses the IEEE
    quotient on many of the same pairs."""
    n = 1 << 7
    mant = np.arange(n, 2 * n, dtype=np.float64) / n
    a, b = np.meshgrid(mant * 0.5, mant, indexing="ij")
    a, b = a.ravel(), b.ravel()
    q0 = a.astype(np.float32) * _rn32_div(np.ones_like(b), b)
    assert np.count_nonzero(q0 != _rn32_div(a, b)) > 100
