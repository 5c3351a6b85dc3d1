"""ORACLE -- test infrastructure only.

A plain, slow, obviously correct CPU implementation of the double-double matrix
product and of every intermediate of the sliced method, used to check the HIP
path.  Only tests/, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import anything here; the product path never does, and the two share no
code.

* ``native``  -- classical double-double GEMM (C, OpenMP), one inner product per
                 entry in ascending k (pages: "Multiple Double Arithmetic on
                 NVIDIA Tensor Cores", §4.2).
* ``exact``   -- big-integer slicing, level sums, the renormalisation cascade and
                 exact rational inner products (same page, §2 and §3).
* ``compare`` -- the componentwise acceptance test |C - R| <= 1e-28 (|A||B|)_ij.
"""
from . import compare, exact, native  # noqa: F401
