"""Integer arithmetic the kernels rely on, checked exhaustively on the host.

The gathered GEMM operands divide row-map entries n (0 <= n < 2^31) by the
row divisor d with a multiply-high by m = ceil(2^32 / d) mod 2^32 and one
correction each way (d = 1 passed through, powers of two shifted).  Here the
same steps run in exact Python integers with 32-bit wrap-around and must give
n // d for every divisor up to 64 (MOE_MAX_TOPK is 32) over the numerators
where an error would show: around every multiple of d near 0, near 2^31, and
a random sample in between.
"""
import numpy as np

M32 = (1 << 32) - 1


def div_rows(n, d, m):
    q = (n * m) >> 32
    q -= 1 if (q * d) & M32 > n else 0
    q += 1 if ((q + 1) * d) & M32 <= n else 0
    return n if d == 1 else q


def magic(d):
    return ((1 << 32) + d - 1) // d & M32


def test_row_division_exhaustive_edges():
    rng = np.random.default_rng(0)
    sample = [int(v) for v in rng.integers(0, 1 << 31, 20000)]
    top = (1 << 31) - 1
    for d in range(1, 65):
        m = magic(d)
        ns = set(sample)
        for base in list(range(0, 64 * d, d)) + list(range(top - 64 * d, top, d)):
            ns.update(b for b in (base - 1, base, base + 1) if 0 <= b <= top)
        ns.add(top)
        for n in ns:
            assert div_rows(n, d, m) == n // d, (n, d)
