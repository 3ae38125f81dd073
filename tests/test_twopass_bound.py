"""The two-pass decode route's rounding bound, on the CPU. Scores s~ from bf16
copies C~ of fp32 chunk summaries C must stay within
    e = 0.0045 * sum|q||C~| + 1e-30 * (1 + sum|q|)
of the fp32 scores s, whatever order either fp32 dot product of 128 terms is
summed in: that is what lets the route re-score only the chunks within 2e of
the k-th largest s~ and still select exactly the fp32 top k. Checked here
for sequential, pairwise and 8-lane-then-tree orders, over random, cancelling,
huge and subnormal data; also that the bound is not vacuous."""
import numpy as np
import torch

D = 128
BOUND_REL, BOUND_ABS = 0.0045, 1e-30


def to_bf16(x):
    """fp32 -> bf16 (as fp32 values), round to nearest even, from the bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def dot_seq(q, c):
    s = np.float32(0)
    for a, b in zip(q, c):
        s = np.float32(s + np.float32(a * b))
    return s


def dot_pairwise(q, c):
    v = (q * c).astype(np.float32)
    while v.size > 1:
        v = (v[0::2] + v[1::2]).astype(np.float32)
    return v[0]


def dot_lanes(q, c):
    # 8 lanes, each a sequential sum of 16 products, then a 3-level tree
    p = (q * c).astype(np.float32).reshape(16, 8)
    acc = np.zeros(8, np.float32)
    for row in p:
        acc = (acc + row).astype(np.float32)
    while acc.size > 1:
        acc = (acc[0::2] + acc[1::2]).astype(np.float32)
    return acc[0]


ORDERS = (dot_seq, dot_pairwise, dot_lanes)


def _check(q, C):
    q = q.astype(np.float32)
    C = C.astype(np.float32)
    Cl = to_bf16(C)
    q1 = np.float32(np.abs(q).sum(dtype=np.float64))
    worst = 0.0
    for m in range(C.shape[0]):
        a = np.float32(np.abs(q).astype(np.float64) @ np.abs(Cl[m]).astype(np.float64))
        e = BOUND_REL * float(a) + BOUND_ABS * (1.0 + float(q1))
        for f in ORDERS:
            for g in ORDERS:
                gap = abs(float(f(q, C[m])) - float(g(q, Cl[m])))
                assert gap <= e, (m, f.__name__, g.__name__, gap, e)
                if a > 0:
                    worst = max(worst, gap / float(a))
    return worst


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4096), rng.standard_normal(512) * 1e-39,
                        rng.standard_normal(512) * 1e36, [0.0, -0.0, 3.3895e38, 3.4e38]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(to_bf16(x), want)


def test_bound_holds_on_random_and_structured_summaries():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(D) / np.sqrt(D)
    C = rng.standard_normal((64, D)) * 0.1 + rng.standard_normal(D) * 0.5   # shared offset
    worst = _check(q, C)
    assert worst < 2 ** -8            # the bf16 term dominates and stays below its unit roundoff


def test_bound_holds_under_cancellation():
    # q . C near zero with large terms: the bound is relative to sum|q||C~|, not |s|
    rng = np.random.default_rng(3)
    q = rng.standard_normal(D)
    C = np.tile(q[::-1], (32, 1)) + rng.standard_normal((32, D)) * 1e-3
    C[:, : D // 2] *= -1
    _check(q, C)


def test_bound_holds_at_extreme_scales():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(D)
    for scale in (1e-39, 1e-30, 1e20, 1e35):
        _check(q, rng.standard_normal((16, D)) * scale)
    _check(q * 1e-20, rng.standard_normal((16, D)) * 1e-20)   # products underflow


def test_bound_is_not_vacuous():
    # the kernel's constant is within 15% of the worst case 2^-8/(1-2^-8) + 2*128*2^-24
    worst_case = 2.0 ** -8 / (1 - 2.0 ** -8) + 2 * 128 * 2.0 ** -24
    assert worst_case < BOUND_REL < 1.15 * worst_case
