"""Premises of the bf16 router's error bound, checked on the CPU.

For more than 16 experts with bf16 activations, moe_route computes each
logit from the fp32 gate weight split into three bf16 parts and keeps a
token's choice only when the bound C1 ||x|| ||w|| (plus the fp32 roundings)
proves it. This file checks what that argument rests on, with plain NumPy:

  * the split is exact: hi + mid + lo == w for every fp32 w of magnitude
    2^-100 .. 2^100, with |hi| <= (1 + 2^-8) |w| and |mid| + |lo| <= 2^-7 |w|;
  * C1 = gamma_65 (1 + 2^-8) + gamma_129 2^-7 + 1.02 2^-23 + 2^-40 (with a
    2^-10 margin) is below the 8.1e-6 that moe.h states;
  * an fp32 accumulation in the kernel's windows (hi: 64 products, mid and
    lo: 128, each window summed in fp32 in the worst order for rounding, the
    windows added in fp64) stays within that bound of the exact sum.
"""
import numpy as np
import pytest


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def split3(w: np.ndarray):
    w = np.asarray(w, np.float32)
    hi = bf16_rne(w)
    r1 = (w - hi).astype(np.float32)
    mid = bf16_rne(r1)
    r2 = (r1 - mid).astype(np.float32)
    lo = bf16_rne(r2)
    return hi, mid, lo


def gamma(n):
    u = 2.0 ** -23
    return n * u / (1 - n * u)


C1 = (gamma(65) * (1 + 2 ** -8) + gamma(129) * 2 ** -7 + 1.02 * 2 ** -23 + 2 ** -40) * (
    1 + 2 ** -10)


def test_split_is_exact_and_bounded():
    g = np.random.default_rng(0)
    n = 400_000
    mant = g.uniform(1.0, 2.0, n)
    expo = g.integers(-100, 101, n)
    sign = np.where(g.random(n) < 0.5, -1.0, 1.0)
    w = (sign * np.ldexp(mant, expo)).astype(np.float32)
    w = np.concatenate([w, np.float32([0.0, -0.0, 1.0, -3.0, 2 ** -100, 1.99999988])])
    hi, mid, lo = split3(w)
    w64 = w.astype(np.float64)
    total = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert np.array_equal(total, w64), "hi + mid + lo differs from w"
    aw = np.abs(w64)
    assert np.all(np.abs(hi.astype(np.float64)) <= (1 + 2 ** -8) * aw)
    assert np.all(np.abs(mid.astype(np.float64)) + np.abs(lo.astype(np.float64))
                  <= 2 ** -7 * aw)
    # every part is a bf16 value (low 16 bits zero)
    for p in (hi, mid, lo):
        assert np.all((p.view(np.uint32) & 0xFFFF) == 0)


def test_c1_value():
    assert 7.9e-6 < C1 < 8.1e-6


def _worst_order_fp32_sum(p: np.ndarray) -> float:
    """fp32 sum of the products of one window, largest magnitudes last (the
    order that loses most to rounding among simple orders)."""
    s = np.float32(0.0)
    for v in p[np.argsort(np.abs(p))]:
        s = np.float32(s + np.float32(v))
    return float(s)


@pytest.mark.parametrize("D", [1024, 4096])
def test_windowed_fp32_accumulation_within_bound(D):
    g = np.random.default_rng(D)
    worst = 0.0
    for _ in range(6):
        x = bf16_rne(g.standard_normal(D).astype(np.float32)).astype(np.float64)
        w = (0.02 * g.standard_normal(D)).astype(np.float32)
        hi, mid, lo = (p.astype(np.float64) for p in split3(w))
        exact = float(np.dot(x, w.astype(np.float64)))
        approx = 0.0
        for k0 in range(0, D, 64):  # one flush window of 64 hidden elements
            sl = slice(k0, k0 + 64)
            h = _worst_order_fp32_sum(x[sl] * hi[sl])
            m = _worst_order_fp32_sum(np.concatenate([x[sl] * mid[sl], x[sl] * lo[sl]]))
            approx += h + m
        bound = C1 * np.linalg.norm(x) * np.linalg.norm(w.astype(np.float64))
        err = abs(approx - exact)
        assert err <= bound, (err, bound)
        worst = max(worst, err / bound)
    assert worst < 0.1  # typical errors are far inside the worst-case bound
