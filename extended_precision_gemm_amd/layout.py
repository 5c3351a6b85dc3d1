"""Host-side description of the packed slice layout (pure index bookkeeping).

For one operand with ``outer`` rows (A) or columns (B), inner dimension k and n
slices per entry (8 for the double-double product), slice s of entry (o, p)
lives at

    ((((o // 16) * KB + p // 4) * n + s) * 64) + (p % 4) * 16 + (o % 16)

with Op = roundup(outer, 128), Kp = roundup(k, 16), KB = Kp // 4: fragments of
64 doubles in the lane order of the FP64 16x16x4 matrix instruction.  These
helpers turn a packed buffer into plain (8, outer, k) planes and back; they do
no arithmetic on the values.
"""
from __future__ import annotations

PACK_OUTER = 64
PACK_K = 16


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def padded(outer: int, k: int) -> tuple[int, int]:
    return _round_up(outer, PACK_OUTER), _round_up(k, PACK_K)


def unpack(packed, outer: int, k: int, nslices: int = 8):
    """(Op*Kp*n,) packed tensor/array -> (n, outer, k) view-copy (torch or numpy)."""
    Op, Kp = padded(outer, k)
    x = packed.reshape(Op // 16, Kp // 4, nslices, 4, 16)  # [ob, kb, s, kk, oi]
    if hasattr(x, "permute"):
        x = x.permute(2, 0, 4, 1, 3)
    else:
        x = x.transpose(2, 0, 4, 1, 3)                       # [s, ob, oi, kb, kk]
    x = x.reshape(nslices, Op, Kp)
    return x[:, :outer, :k]


def pack(planes, outer: int, k: int):
    """(n, outer, k) planes -> packed (Op*Kp*n,) layout, zero padded (numpy)."""
    import numpy as np
    n = planes.shape[0]
    Op, Kp = padded(outer, k)
    full = np.zeros((n, Op, Kp), dtype=np.float64)
    full[:, :outer, :k] = planes
    x = full.reshape(n, Op // 16, 16, Kp // 4, 4).transpose(1, 3, 0, 4, 2)
    return np.ascontiguousarray(x).reshape(-1)
