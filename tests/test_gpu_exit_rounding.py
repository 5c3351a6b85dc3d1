"""The pair-packed products' exit rounding on the GPU, entry by entry, against
the oracle (GPU tests).

The exit turns an entry's exact total -- its group sums, group g counting
units 2^(sc - 13(g+3)) -- into the nearest double-double ("Multiple Double
Arithmetic on NVIDIA Tensor Cores", §2 overview, fifth step, with the parts
added exactly and rounded once).  Products of random operands almost never
put that total exactly on a tie, or at the ends of the exponent range, so the
exit is driven here directly through the diagnostic entry point
ddgemm_probe_pair_round: seeded totals of every magnitude, sparse and tiny
ones, carry chains between groups, and totals built bit by bit with a tie, or
one unit off it, at random positions (the leading word's and the trailing
word's), under scales from the subnormal range to overflow.  The expected
words come from oracle.exact.nearest_dd, the exact rational total rounded to
the nearest double-double.
"""
import numpy as np
import pytest

from oracle import exact

pytestmark = pytest.mark.gpu

DIGIT = 13


def _signed_bits(rng, maxbits, size):
    b = rng.integers(0, maxbits + 1, size)
    mag = np.array([int(rng.integers(0, 1 << int(x))) if x > 0 else 0 for x in b.ravel()], dtype=object)
    sign = rng.integers(0, 2, size).ravel()
    return [int(v) if s else -int(v) for v, s in zip(mag, sign)]


def _cases(ns, count, seed):
    """(units (count, ns-1) as Python ints, scales (count,))."""
    rng = np.random.default_rng(seed)
    L = DIGIT * (ns - 2)
    units, scales = [], []
    for _ in range(count):
        mode = int(rng.integers(0, 10))
        if mode >= 6:
            # T = M 2^L + R, R a bit pattern with a tie, or one unit off it, at position p - 1
            R = 0
            top = int(rng.integers(0, L + 1))
            for t in range(top):
                if rng.integers(0, 2):
                    R |= 1 << (L - 1 - t)
            p = int(rng.integers(0, L + 1))
            if p > 0:
                R &= ~((1 << p) - 1)
                R |= 1 << (p - 1)
                if mode == 9:
                    R += 1          # just above the tie
                elif mode == 8:
                    R -= 1          # just below it
            R &= (1 << L) - 1
            M = _signed_bits(rng, 53 if rng.integers(0, 4) else 24, 1)[0]
            N = [M] + [(R >> (DIGIT * (ns - 2 - g))) & 8191 for g in range(1, ns - 1)]
            if rng.integers(0, 2):  # negative digits with compensating carries: the same total
                for g in range(ns - 2, 0, -1):
                    if rng.integers(0, 2):
                        N[g] -= 8192
                        N[g - 1] += 1
        elif mode == 0:
            N = _signed_bits(rng, 60, ns - 1)
        elif mode == 1:
            N = _signed_bits(rng, 53, ns - 1)
        elif mode == 2:
            N = [v if rng.integers(0, 3) == 0 else 0 for v in _signed_bits(rng, 53, ns - 1)]
        elif mode == 3:
            N = [int(x) for x in rng.integers(-2, 3, ns - 1)]
        elif mode == 4:
            N = [int(rng.choice([8191, -1, 8192])) for _ in range(ns - 1)]
        else:
            N = [v << int(rng.integers(0, 40)) for v in _signed_bits(rng, 20, ns - 1)]
        which = int(rng.integers(0, 10))
        if which < 7:
            sc = int(rng.integers(-40, 41))
        elif which == 7:
            sc = int(rng.integers(-1000, -900))   # words reaching the subnormal range
        elif which == 8:
            sc = int(rng.integers(-1120, -1040))  # totals around and below the smallest subnormal
        else:
            sc = int(rng.integers(940, 1080))     # totals around and beyond the largest double
        units.append(N)
        scales.append(sc)
    return units, scales


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float64).view(np.int64)


@pytest.mark.parametrize("ns", [4, 5, 6, 7, 8, 12, 16])
def test_exit_rounding_equals_the_nearest_double_double(gpu, ns):
    import torch
    count = 3000 if ns <= 8 else 1000
    units, scales = _cases(ns, count, 4400 + ns)
    U = np.array(units, dtype=np.int64)
    S = np.zeros((ns, count, 1), dtype=np.int64)
    S[1:, :, 0] = U.T  # group g counts the units of level g + 1
    hi, lo = exact.nearest_dd(S, np.array(scales, dtype=np.int64), [0])
    out = gpu.probe_pair_round(torch.from_numpy(U).cuda(), torch.tensor(scales, dtype=torch.int32).cuda(),
                               nslices=ns)
    got = out.cpu().numpy()
    bad = np.nonzero((_bits(got[:, 0]) != _bits(hi[:, 0])) | (_bits(got[:, 1]) != _bits(lo[:, 0])))[0]
    assert bad.size == 0, [(units[i], scales[i], got[i].tolist(), (hi[i, 0], lo[i, 0])) for i in bad[:3]]
