"""Why the chunked prefill splits P into a bf16 head and tail for bf16 caches.

The P.V product of the prefill runs on bf16 matrix cores, so P has to be
rounded to bf16. The parity bound for bf16 caches is a max abs error of 2e-3.
A row whose weight sits on a few keys shows that a single rounding of P can
break that bound whatever the row's key count: with two dominant keys the
error is (rounding error of p2) * |v2 - O| / (p1 + p2), up to about
2^-9 * 8 / 1.5 for standard-normal values. Splitting P into head = bf16(p)
and tail = bf16(p - head) leaves an error of order 2^-17 * p, far below the
bound. Everything here is numpy in float64 apart from the roundings.
"""
import numpy as np

TOL_BF16 = 2e-3


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even)."""
    b = np.asarray(x, dtype=np.float32).reshape(-1).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def attend(p: np.ndarray, v: np.ndarray, denom: float) -> np.ndarray:
    return (p[:, None] * v).sum(0) / denom


def test_bf16_round_worked_values():
    # 0.7f = 0x3F333333: the low half is below 0x8000, so it rounds down
    assert bf16_round(0.7)[0] == 0.69921875
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even one
    assert bf16_round(1.0 + 2.0 ** -8)[0] == 1.0
    assert bf16_round(1.0 + 3 * 2.0 ** -8)[0] == 1.0 + 2.0 ** -6
    # representable values stay as they are
    for x in (0.5, -3.0, 2.0 ** -20, 1.5):
        assert bf16_round(x)[0] == x


def test_two_dominant_keys_break_the_bound_with_one_rounding():
    # weights relative to the row maximum: the first key at 1, the second
    # just above 0.5, where bf16's spacing (2^-8) gives an error near 2^-9
    p = np.array([1.0, 0.5 + 0.999 * 2.0 ** -9], dtype=np.float32).astype(np.float64)
    v = np.array([[4.0], [-4.0]])  # values four standard deviations out
    exact = attend(p, v, p.sum())
    ph = bf16_round(p)
    # the kernel's sum of P is taken in fp32 from the unrounded weights ...
    err_kernel_sum = np.abs(attend(ph, v, p.sum()) - exact).max()
    # ... and with the rounded weights in the sum the output is a convex
    # combination again, but still off by the same order
    err_rounded_sum = np.abs(attend(ph, v, ph.sum()) - exact).max()
    assert err_kernel_sum > TOL_BF16
    assert err_rounded_sum > TOL_BF16
    # the error follows the closed form of the two-key case
    d = p[1] - ph[1]
    assert abs(err_rounded_sum - abs(ph[0] * d * (v[0, 0] - v[1, 0])) / (ph.sum() * p.sum())) < 1e-12


def test_many_small_keys_do_not_rescue_a_dominant_pair():
    # 8192 further keys with weights of 2^-30 (a long history far below the
    # maximum) leave the two-key error where it was: the key count does not
    # bound it
    rng = np.random.default_rng(5)
    p = np.concatenate([[1.0, 0.5 + 0.999 * 2.0 ** -9], np.full(8192, 2.0 ** -30)]).astype(np.float32)
    p = p.astype(np.float64)
    v = np.concatenate([[[4.0], [-4.0]], rng.standard_normal((8192, 1))])
    exact = attend(p, v, p.sum())
    ph = bf16_round(p)
    assert np.abs(attend(ph, v, p.sum()) - exact).max() > TOL_BF16


def test_head_and_tail_stay_far_inside_the_bound():
    rng = np.random.default_rng(7)
    worst = 0.0
    for _ in range(200):
        n = int(rng.integers(2, 64))
        s = rng.standard_normal(n) * 3.0
        p = np.exp2(s - s.max()).astype(np.float32).astype(np.float64)
        v = np.clip(rng.standard_normal((n, 8)), -5, 5)
        v = bf16_round(v).reshape(n, 8)
        head = bf16_round(p)
        tail = bf16_round(p - head)
        got = attend(head, v, p.sum()) + attend(tail, v, p.sum())
        worst = max(worst, np.abs(got - attend(p, v, p.sum())).max())
    assert worst < 1e-4
    # the two-key row of the test above is fine with the split
    p = np.array([1.0, 0.5 + 0.999 * 2.0 ** -9], dtype=np.float32).astype(np.float64)
    v = np.array([[4.0], [-4.0]])
    head = bf16_round(p)
    tail = bf16_round(p - head)
    assert np.abs(attend(head + tail, v, p.sum()) - attend(p, v, p.sum())).max() < 1e-5
