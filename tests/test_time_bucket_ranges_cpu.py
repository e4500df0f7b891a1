"""The block-level time-bucket rules the attention kernels use, checked on the
CPU against the definition of the time bucket (floor(log2(1 + |t_i - t_j|)),
"HSTU tensor by tensor: SiLU aggregation, temporal bias and gating", the
temporal bias): for a block of rows with times in [wmin, wmax] and keys with
times in [kmin, kmax] (32-bit relative times), every pair's gap lies between
the two ranges' smallest and largest distance, so its bucket lies between
those distances' buckets; when they are adjacent, one compare of 1 + gap with
2^(upper bucket) tells the two apart."""
import numpy as np

M32 = (1 << 32) - 1


def bucket(dt):
    return int(dt + 1).bit_length() - 1   # floor(log2(1 + dt))


def clz32(x):
    return 32 - int(x).bit_length()


def range_distances(wmin, wmax, kmin, kmax):
    """Smallest and largest |a - b| over a in [wmin, wmax], b in [kmin, kmax]
    (reals in the ranges; the smallest is 0 when they overlap), written the
    way the kernels do (unsigned max - b forms)."""
    dmin = (max(wmin, kmax) - kmax) + (max(kmin, wmax) - wmax)
    dmax = max(max(wmax, kmin) - kmin, max(kmax, wmin) - wmin)
    return dmin, dmax


def test_pair_buckets_lie_between_the_range_buckets():
    rng = np.random.default_rng(7)
    two = 0
    for _ in range(3000):
        scale = int(rng.choice([10, 1000, 3600 * 50, 1 << 28]))
        base = int(rng.integers(1, 1 << 30))
        rows = base + np.sort(rng.integers(0, scale, size=16))
        keys = base + int(rng.integers(-4 * scale, 4 * scale)) + np.sort(rng.integers(0, scale, size=32))
        keys = np.clip(keys, 1, M32)
        wmin, wmax, kmin, kmax = int(rows.min()), int(rows.max()), int(keys.min()), int(keys.max())
        dmin, dmax = range_distances(wmin, wmax, kmin, kmax)
        gaps = np.abs(rows[:, None].astype(np.int64) - keys[None, :].astype(np.int64))
        assert dmin <= int(gaps.min()) and dmax == int(gaps.max())   # dmin: a bound (0 when the ranges overlap)
        z0, z1 = clz32(dmin + 1), clz32(dmax + 1)
        lo, hi = 31 - z0, 31 - z1
        b = np.array([[bucket(g) for g in row] for row in gaps])
        assert b.min() >= lo and b.max() <= hi
        if z0 == z1:
            assert (b == lo).all()
        elif z0 == z1 + 1:
            two += 1
            thr = 1 << (31 - z1)
            sel = np.where(gaps + 1 >= thr, hi, lo)
            assert (sel == b).all()
    assert two > 100   # the two-bucket case was exercised


def test_two_bucket_boundary_values():
    # gaps straddling a power of two exactly: 1 + gap = 2^k - 1, 2^k, 2^k + 1
    for k in range(1, 31):
        for g in ((1 << k) - 2, (1 << k) - 1, 1 << k):
            z0, z1 = clz32((1 << k) - 2 + 1), clz32((1 << k) + 1)
            if z0 == z1 + 1:
                assert (31 - z1 if g + 1 >= (1 << (31 - z1)) else 31 - z0) == bucket(g)
