"""The quotient rule of the normalized query means (CPU, numpy).

The query-side statistics round each normalized value v / n to f32 once, from
the correctly rounded f64 quotient (section 3.1 of the AdaCluster page:
queries put on the unit sphere before clustering). The kernel forms
p = v * RN64(1 / n) instead and keeps RN32(p) only when p lies more than 16
f64 units in the last place from every f32 rounding midpoint and inside the
normal f32 range; otherwise it divides. These tests check that rule on the
bit patterns, the same way the kernel tests them: wherever it accepts p,
RN32(p) equals RN32(RN64(v / n)), on ordinary rows and on quotients built to
sit next to a midpoint or below the normal range.
"""
import numpy as np


def settled(p):
    b = np.asarray(p, np.float64).view(np.uint64)
    low = (b & np.uint64(0x1FFFFFFF)).astype(np.uint32)
    hi = ((b >> np.uint64(32)) & np.uint64(0x7FFFFFFF)).astype(np.uint32)
    lo32 = (b & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    normal = (hi >= np.uint32(898 << 20)) | ((hi | lo32) == 0)
    return normal & ((low - np.uint32(0x10000000 - 16)) > np.uint32(32))


def bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32)


def seq_norm(rows):
    s = np.zeros(rows.shape[0])
    for j in range(rows.shape[1]):           # index order, as the definition
        s = s + rows[:, j].astype(np.float64) * rows[:, j].astype(np.float64)
    n = np.sqrt(s)
    return np.maximum(n, 1e-12)


def check(v, n):
    v = np.asarray(v, np.float64)
    t = v / n                                 # RN64(v / n)
    p = v * (1.0 / n)                         # RN64(v * RN64(1 / n))
    ok = settled(p)
    assert np.array_equal(t[ok].astype(np.float32).view(np.uint32),
                          p[ok].astype(np.float32).view(np.uint32))
    return ok, t, p


def test_rule_on_query_rows():
    rng = np.random.default_rng(0)
    rows = bf16(rng.standard_normal((4000, 64)).astype(np.float32) * rng.uniform(0.01, 30, (4000, 1)))
    n = seq_norm(rows)
    ok, _, _ = check(rows, n[:, None])
    assert ok.mean() > 0.9999                 # the division is the rare path


def test_rule_next_to_midpoints():
    # quotients placed within a few f64 units of an f32 rounding midpoint
    rng = np.random.default_rng(1)
    x = rng.uniform(2.0 ** -20, 1.0, 200000).astype(np.float32)
    up = np.nextafter(x, np.float32(2.0))
    mid = (x.astype(np.float64) + up.astype(np.float64)) / 2       # exact in f64
    v = bf16(rng.uniform(0.05, 8.0, x.size).astype(np.float32)).astype(np.float64)
    n = v / mid
    ok, t, p = check(v, n)
    assert (~ok).mean() > 0.99                # the rule declines next to a midpoint
    # and there the product alone would round differently in some cases
    diff = t.astype(np.float32) != p.astype(np.float32)
    assert diff.any()
    assert not (diff & ok).any()


def test_rule_declines_below_the_normal_range():
    v = np.array([2.0 ** -130, 2.0 ** -127, 3.0 * 2.0 ** -128, -2.0 ** -126])
    n = np.ones(4)
    assert not settled(v * (1.0 / n)).any()
    assert settled(np.array([0.0, -0.0, 2.0 ** -125, 0.5])).all()
