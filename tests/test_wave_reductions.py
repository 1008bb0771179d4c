"""The composite backward's wave reductions, modelled lane by lane on the CPU.

The kernels sum 16, 14 or 10 per-lane values over a 64-lane wave with a halving
reduction: a cross-half swap (lanes 32-63 with 0-31), a swap of odd 16-lane rows
with even ones, a rotation of each 16-lane row by 8, a mirror within each 8-lane
half row and two quad permutations.  This test models those moves as permutations
of 64-element fp32 arrays, follows the three reductions step by step as the kernels
write them (wave_sum16, wave_sum14, wave_sum10 with their lane maps), and checks
that every reported lane holds the total of the value its map names, that each
value is reported exactly once, and that the 14- and 10-value forms give totals
bit-identical to the 16-value form (same pairing order).  The GPU parity tests check
the kernels themselves; this pins the lane bookkeeping the flush depends on.
"""
import numpy as np

L = np.arange(64)
F32 = np.float32


def swap32(x, y):
    """Cross-half swap: lanes 32-63 of x trade places with lanes 0-31 of y."""
    r0, r1 = x.copy(), y.copy()
    r0[32:], r1[:32] = y[:32], x[32:]
    return r0, r1


def swap16(x, y):
    """Row swap: the odd 16-lane rows of x trade places with the even rows of y."""
    r0, r1 = x.copy(), y.copy()
    for row in (1, 3):
        r0[row * 16:(row + 1) * 16] = y[(row - 1) * 16:row * 16]
        r1[(row - 1) * 16:row * 16] = x[row * 16:(row + 1) * 16]
    return r0, r1


def perm(x, src):
    return x[src]


ROR8 = (L & ~15) | ((L + 8) & 15)
MIRROR8 = (L & ~7) | (7 - (L & 7))
QUAD_2301 = (L & ~3) | np.array([2, 3, 0, 1])[L & 3]
QUAD_1032 = (L & ~3) | np.array([1, 0, 3, 2])[L & 3]
H3 = (L & 8) != 0
H2 = (L & 4) != 0


def add(a, b):
    return (a + b).astype(F32)


def tail(b):
    """The steps after the row swap, from four row partial sums b[0..3]."""
    c = [add(np.where(H3, b[2 + i], b[i]), perm(np.where(H3, b[i], b[2 + i]), ROR8)) for i in range(2)]
    d = add(np.where(H2, c[1], c[0]), perm(np.where(H2, c[0], c[1]), MIRROR8))
    d = add(d, perm(d, QUAD_2301))
    return add(d, perm(d, QUAD_1032))


def sum16(v):
    a = [add(*swap32(v[i], v[8 + i])) for i in range(8)]
    b = [add(*swap16(a[i], a[4 + i])) for i in range(4)]
    return tail(b)


def sum14(v):
    a = [add(*swap32(v[i], v[7 + i])) for i in range(7)]
    b = [add(*swap16(a[i], a[4 + i] if i < 3 else a[3])) for i in range(4)]
    return tail(b)


def sum10(v):
    a = [add(*swap32(v[i], v[5 + i])) for i in range(5)]
    b = [add(*swap16(a[i], a[3 + i] if i < 2 else a[2])) for i in range(3)]
    c0 = add(np.where(H3, b[2], b[0]), perm(np.where(H3, b[0], b[2]), ROR8))
    c1 = add(b[1], perm(b[1], ROR8))
    d = add(np.where(H2, c1, c0), perm(np.where(H2, c0, c1), MIRROR8))
    d = add(d, perm(d, QUAD_2301))
    return add(d, perm(d, QUAD_1032))


def basis16(lane):
    return lane >> 2


def basis14(lane):
    H, R = lane & 32, lane & 16
    j = (2 if lane & 8 else 0) + (1 if lane & 4 else 0)
    ai = (-1 if R else 3) if j == 3 else ((4 + j) if R else j)
    return -1 if ai < 0 else ai + (7 if H else 0)


def basis10(lane):
    H, R, h3, h2 = lane & 32, lane & 16, lane & 8, lane & 4
    ai = (-1 if (h2 or R) else 2) if h3 else ((3 if R else 0) + (1 if h2 else 0))
    return -1 if ai < 0 else ai + (5 if H else 0)


def _reported(d, basis, n):
    out = {}
    for lane in range(0, 64, 4):
        c = basis(lane)
        if c >= 0:
            assert c not in out, "value reported twice"
            out[c] = d[lane]
    assert sorted(out) == list(range(n)), "a value is not reported"
    return out


def test_reductions_sum_every_value_once_and_agree_bitwise():
    rng = np.random.default_rng(7)
    for _ in range(100):
        v = [(rng.standard_normal(64) * 10.0 ** rng.uniform(-3, 3, 64)).astype(F32) for _ in range(16)]
        r16 = _reported(sum16(v), basis16, 16)
        for k in range(16):
            exact = v[k].astype(np.float64).sum()
            assert abs(r16[k] - exact) <= 1e-5 * np.abs(v[k]).astype(np.float64).sum() + 1e-30
        v14 = [x if i < 14 else np.zeros(64, F32) for i, x in enumerate(v)]
        r16z = _reported(sum16(v14), basis16, 16)
        r14 = _reported(sum14(v14[:14]), basis14, 14)
        assert all(r14[k] == r16z[k] for k in range(14))
        v10 = [x if i < 10 else np.zeros(64, F32) for i, x in enumerate(v)]
        r16z = _reported(sum16(v10), basis16, 16)
        r10 = _reported(sum10(v10[:10]), basis10, 10)
        assert all(r10[k] == r16z[k] for k in range(10))


def test_a_wrong_lane_map_is_caught():
    """A map that swaps two values' lanes must fail the comparison above."""
    rng = np.random.default_rng(8)
    v = [rng.standard_normal(64).astype(F32) for _ in range(14)]
    d = sum14(v)

    def bad(lane):
        c = basis14(lane)
        return {3: 10, 10: 3}.get(c, c)
    r = _reported(d, bad, 14)
    assert any(abs(r[k] - v[k].astype(np.float64).sum()) > 1e-3 for k in (3, 10))
