"""Double-double and quad-double matrix products C = A·B on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libddgemm.so`` (C ABI in ``include/ddgemm.h`` and
``include/qdgemm.h``).  It
only marshals arguments: every step of the product runs in the library's HIP
kernels; PyTorch supplies device memory and the current stream.  Importing
this module fails loudly when the library has not been built.

The method ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §2-§3): each
double-double entry is cut into eight 13-bit slices below a per-row (A) or
per-column (B) balancing exponent, the 36 slice pairs inside the double-double
window are multiplied exactly on FP64 matrix cores and summed per level, and
the eight level sums of every output entry are renormalised into (hi, lo) once.
The quad-double product (``qd_*``) takes sixteen slices, 136 pairs and sixteen
levels, whose exact total is rounded to the nearest four-double result.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import layout  # noqa: F401  (host-side description of the packed slice layout)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddgemm.so")

NUM_SLICES = 8          # the double-double product
MIN_SLICES = 4          # the pages' four quarters of a leading double
MAX_SLICES = 16         # double-double inputs with windows 13 * (n - 8) bits deeper
NUM_LEVELS = 8
SLICE_BITS = 13
K_MAX = 8388608
QD_NUM_SLICES = 16      # the quad-double product
QD_K_MAX = 4194304
QD_K_MAX_BLOCKED = 4294967296   # longer qd products run in k-blocks sharing their exponents
NOALLOC_SCRATCH_BYTES = 256 << 20  # the device array dd_gemm_noalloc works in, per GPU

SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_WORKSPACE = 2
ERROR_LAUNCH = 3
ERROR_DEVICE = 4


class DDGemmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_st = ctypes.c_int
_pp = ctypes.POINTER(ctypes.c_void_p)   # a host array of four device pointers (qd planes)

# name -> (restype, argtypes); mirrors include/ddgemm.h
_SIGNATURES = {
    "dd_split_slices_bytes": (_sz, [_i64, _i64]),
    "dd_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "dd_split_balanced": (_st, [_i64, _i64, _vp, _vp, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "dd_sliced_gemm": (_st, [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "dd_renorm_levels": (_st, [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
    "dd_sliced_gemm_renorm": (_st, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "dd_gemm": (_st, [_i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp]),
    "dd_gemm_ws": (_st, [_i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _sz, _vp]),
    "dd_split_slices_bytes_ns": (_sz, [_i64, _i64, ctypes.c_int]),
    "dd_gemm_workspace_size_ns": (_sz, [_i64, _i64, _i64, ctypes.c_int]),
    "dd_split_balanced_ns": (_st, [_i64, _i64, _vp, _vp, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "dd_sliced_gemm_renorm_ns": (_st, [_i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "dd_gemm_ws_ns": (_st, [_i64, _i64, _i64, ctypes.c_int, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                            _vp, _sz, _vp]),
    "qd_split_slices_bytes": (_sz, [_i64, _i64]),
    "qd_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "qd_split_balanced": (_st, [_i64, _i64, _pp, _i64, ctypes.c_int, _vp, _vp, _vp]),
    "qd_sliced_gemm_renorm": (_st, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _pp, _i64, _vp]),
    "qd_gemm": (_st, [_i64, _i64, _i64, _pp, _i64, _pp, _i64, _pp, _i64, _vp]),
    "qd_gemm_ws": (_st, [_i64, _i64, _i64, _pp, _i64, _pp, _i64, _pp, _i64, _vp, _sz, _vp]),
    "qd_gemm_workspace_size_kb": (_sz, [_i64, _i64, _i64, _i64]),
    "qd_gemm_ws_kb": (_st, [_i64, _i64, _i64, _i64, _pp, _i64, _pp, _i64, _pp, _i64, _vp, _sz, _vp]),
    "qd_gemm_ws_timed": (_st, [_i64, _i64, _i64, _pp, _i64, _pp, _i64, _pp, _i64, _vp, _sz, _vp, _vp]),
    "dd_gemm_workspace_size_kb": (_sz, [_i64, _i64, _i64, ctypes.c_int, _i64]),
    "dd_gemm_ws_kb": (_st, [_i64, _i64, _i64, ctypes.c_int, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                            _vp, _sz, _vp]),
    "ddgemm_split_parts": (_i64, [_i64, _i64, _i64, ctypes.c_int]),
    "ddgemm_small_product": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int]),
    "ddgemm_split_first_row": (_i64, [_i64, _i64, _i64, ctypes.c_int]),
    "ddgemm_split_first_tile": (_i64, [_i64, _i64, _i64, ctypes.c_int]),
    "dd_gemm_noalloc": (_st, [_i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp]),
    "dd_sliced_gemm_pairs": (_st, [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "dd_sliced_gemm_pairs_ns": (_st, [_i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _i64, _vp]),
    "dd_gemm_ws_timed": (_st, [_i64, _i64, _i64, ctypes.c_int, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                               _vp, _sz, _vp, _vp]),
    "dd_gemm_kblock_max": (_i64, [ctypes.c_int]),
    "ddgemm_status_string": (ctypes.c_char_p, [_st]),
    "ddgemm_probe_mfma_f64": (_st, [_vp, _vp]),
    "ddgemm_probe_pair_round": (_st, [_i64, ctypes.c_int, _vp, _vp, _vp, _vp]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.ddgemm_status_string(status).decode()


def _check(status: int) -> None:
    if status != SUCCESS:
        raise DDGemmError(status, status_string(status))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _matrix(t, name, shape=None):
    """Validate a float64 row-major device matrix; return its leading dimension."""
    if t.dtype != torch.float64:
        raise TypeError(f"{name} must be float64, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0), cols, 1) if rows > 1 else max(cols, 1)


def _device(*tensors):
    """The one device of the given tensors (None entries skipped).  The library
    runs on the current device, so each product is called under this one."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"operands and results must be on one device, got {sorted(map(str, devs))}")
    return devs.pop()


def _workspace(workspace, need, dev, stream=None):
    """A caller's workspace (uint8, contiguous, on the operands' device), or a
    new one of `need` bytes from PyTorch's allocator.  A new workspace is taken
    on the current stream; when the library runs on another one, the tensor is
    recorded on that stream, so that the allocator does not hand its memory to
    a later allocation while the kernels may still use it."""
    if workspace is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        if stream is not None and ws.is_cuda and stream != torch.cuda.current_stream(dev):
            ws.record_stream(stream)
        return ws
    if workspace.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8, got {workspace.dtype}")
    if workspace.device != dev:
        raise ValueError(f"workspace must be a device tensor on {dev}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace


def _buffer(t, name, dtype, numel, dev):
    """Validate a flat device buffer a stage call reads or writes: the given
    dtype, contiguous, on device `dev`, at least `numel` elements."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")
    return t


def _operand_buffers(m, n, k, A_slices, E, B_slices, F, nslices):
    """The packed slices and exponents of both operands of an m×k by k×n stage
    call, checked against the sizes the library will touch; returns their device."""
    dev = A_slices.device
    _buffer(A_slices, "A_slices", torch.float64, slices_bytes(m, k, nslices) // 8, dev)
    _buffer(B_slices, "B_slices", torch.float64, slices_bytes(n, k, nslices) // 8, dev)
    if E is not None:
        _buffer(E, "E", torch.int32, m, dev)
    if F is not None:
        _buffer(F, "F", torch.int32, n, dev)
    return dev


def _check_lo(lo, hi, name):
    if lo is None:
        return
    _matrix(lo, name, hi.shape)
    if lo.stride() != hi.stride():
        raise ValueError(f"{name} must have the same strides as its hi plane")


def pair_products(nslices: int = NUM_SLICES) -> int:
    """FP64 matrix products per k-block of the pair-packed schedule (20 for 8
    slices): slices 2u, 2u+1 of A packed into one operand, every product
    covering two window pairs but where only one lies in the window."""
    return sum(1 for u in range((nslices + 1) // 2) for t in range(nslices)
               if (2 * u + 1 < nslices and 2 * u + 1 + t <= nslices - 1) or 2 * u + t == nslices - 1)


def k_max(nslices: int = NUM_SLICES) -> int:
    """Largest k for n slices (§2 eq. (5): at most 67,108,865 exact terms per level sum)."""
    return K_MAX if nslices <= NUM_SLICES else 67108865 // nslices


def split_parts(m: int, n: int, k: int, nslices: int = NUM_SLICES) -> int:
    """k-parts the product entry points use for an m×n×k product (1 = not split)."""
    return lib.ddgemm_split_parts(m, n, k, nslices)


def small_product(m: int, n: int, k: int, nslices: int = NUM_SLICES) -> bool:
    """Whether the product entry points run the small-output kernel for m×n×k."""
    return bool(lib.ddgemm_small_product(m, n, k, nslices))


def split_first_row(m: int, n: int, k: int, nslices: int = NUM_SLICES) -> int:
    """First row of the tile row holding the first split tile (m when not split)."""
    return lib.ddgemm_split_first_row(m, n, k, nslices)


def split_first_tile(m: int, n: int, k: int, nslices: int = NUM_SLICES) -> int:
    """First output tile (row-major) split over k; the tiles before it run unsplit."""
    return lib.ddgemm_split_first_tile(m, n, k, nslices)


def slices_bytes(outer: int, k: int, nslices: int = NUM_SLICES) -> int:
    if nslices == NUM_SLICES:
        return lib.dd_split_slices_bytes(outer, k)
    return lib.dd_split_slices_bytes_ns(outer, k, nslices)


def workspace_size(m: int, n: int, k: int, nslices: int = NUM_SLICES, kblock: int | None = None) -> int:
    if kblock is not None:
        return lib.dd_gemm_workspace_size_kb(m, n, k, nslices, kblock)
    if nslices == NUM_SLICES:
        return lib.dd_gemm_workspace_size(m, n, k)
    return lib.dd_gemm_workspace_size_ns(m, n, k, nslices)


def split_balanced(X_hi, X_lo, axis: int, exps=None, slices=None, stream=None, nslices: int = NUM_SLICES):
    """Balancing exponents and packed slices of one operand (axis 0: A, axis 1: B),
    with ``nslices`` 13-bit slices per entry (8: double-double)."""
    ldx = _matrix(X_hi, "X_hi")
    _check_lo(X_lo, X_hi, "X_lo")
    rows, cols = X_hi.shape
    outer = rows if axis == 0 else cols
    k = cols if axis == 0 else rows
    dev = _device(X_hi, X_lo)
    if exps is None:
        exps = torch.empty(outer, dtype=torch.int32, device=dev)
    if slices is None:
        slices = torch.empty(slices_bytes(outer, k, nslices) // 8, dtype=torch.float64, device=dev)
    _buffer(exps, "exps", torch.int32, outer, dev)
    _buffer(slices, "slices", torch.float64, slices_bytes(outer, k, nslices) // 8, dev)
    if nslices == NUM_SLICES:
        _check(lib.dd_split_balanced(rows, cols, _ptr(X_hi), _ptr(X_lo), ldx, axis, _ptr(exps), _ptr(slices),
                                     _stream(stream)))
    else:
        _check(lib.dd_split_balanced_ns(rows, cols, _ptr(X_hi), _ptr(X_lo), ldx, axis, nslices, _ptr(exps),
                                        _ptr(slices), _stream(stream)))
    return exps, slices


def sliced_gemm(m: int, n: int, k: int, A_slices, B_slices, levels=None, stream=None):
    """The eight exact level sums, returned as a (8, m, n) float64 tensor."""
    dev = _operand_buffers(m, n, k, A_slices, None, B_slices, None, NUM_SLICES)
    if levels is None:
        levels = torch.empty((NUM_LEVELS, m, n), dtype=torch.float64, device=dev)
    ldl = max(n, 1)
    if tuple(levels.shape) != (NUM_LEVELS, m, n):
        raise ValueError(f"levels must be a ({NUM_LEVELS}, m, n) tensor, got {tuple(levels.shape)}")
    _buffer(levels, "levels", torch.float64, NUM_LEVELS * m * n, dev)
    _check(lib.dd_sliced_gemm(m, n, k, _ptr(A_slices), _ptr(B_slices), _ptr(levels), ldl, _stream(stream)))
    return levels


def renorm_levels(levels, E, F, C_hi=None, C_lo=None, stream=None):
    if levels.dim() != 3 or levels.shape[0] != NUM_LEVELS:
        raise ValueError(f"levels must be a ({NUM_LEVELS}, m, n) tensor, got {tuple(levels.shape)}")
    _, m, n = levels.shape
    dev = levels.device
    _buffer(levels, "levels", torch.float64, NUM_LEVELS * m * n, dev)
    _buffer(E, "E", torch.int32, m, dev)
    _buffer(F, "F", torch.int32, n, dev)
    C_hi = torch.empty((m, n), dtype=torch.float64, device=levels.device) if C_hi is None else C_hi
    C_lo = torch.empty((m, n), dtype=torch.float64, device=levels.device) if C_lo is None else C_lo
    ldc = _matrix(C_hi, "C_hi", (m, n))
    _check_lo(C_lo, C_hi, "C_lo")
    _device(levels, C_hi, C_lo)
    _check(lib.dd_renorm_levels(m, n, _ptr(levels), max(n, 1), _ptr(E), _ptr(F), _ptr(C_hi), _ptr(C_lo), ldc,
                                _stream(stream)))
    return C_hi, C_lo


def sliced_gemm_renorm(m, n, k, A_slices, E, B_slices, F, C_hi=None, C_lo=None, stream=None,
                       nslices: int = NUM_SLICES):
    dev = _operand_buffers(m, n, k, A_slices, E, B_slices, F, nslices)
    _buffer(E, "E", torch.int32, m, dev)
    _buffer(F, "F", torch.int32, n, dev)
    C_hi = torch.empty((m, n), dtype=torch.float64, device=dev) if C_hi is None else C_hi
    C_lo = torch.empty((m, n), dtype=torch.float64, device=dev) if C_lo is None else C_lo
    ldc = _matrix(C_hi, "C_hi", (m, n))
    _check_lo(C_lo, C_hi, "C_lo")
    _device(A_slices, C_hi, C_lo)
    if nslices == NUM_SLICES:
        _check(lib.dd_sliced_gemm_renorm(m, n, k, _ptr(A_slices), _ptr(E), _ptr(B_slices), _ptr(F),
                                         _ptr(C_hi), _ptr(C_lo), ldc, _stream(stream)))
    else:
        _check(lib.dd_sliced_gemm_renorm_ns(m, n, k, nslices, _ptr(A_slices), _ptr(E), _ptr(B_slices), _ptr(F),
                                            _ptr(C_hi), _ptr(C_lo), ldc, _stream(stream)))
    return C_hi, C_lo


def sliced_gemm_pairs(m: int, n: int, k: int, A_slices, B_slices, units=None, stream=None,
                      nslices: int = NUM_SLICES):
    """The exact group sums of the pair-packed schedule the product entry points
    run: an int64 (nslices - 1, m, n) tensor, group g in units 2^(-13(g+3))."""
    dev = _operand_buffers(m, n, k, A_slices, None, B_slices, None, nslices)
    if units is None:
        units = torch.empty((nslices - 1, m, n), dtype=torch.int64, device=dev)
    if tuple(units.shape) != (nslices - 1, m, n):
        raise ValueError(f"units must be a ({nslices - 1}, m, n) tensor, got {tuple(units.shape)}")
    _buffer(units, "units", torch.int64, (nslices - 1) * m * n, dev)
    _check(lib.dd_sliced_gemm_pairs_ns(m, n, k, nslices, _ptr(A_slices), _ptr(B_slices), _ptr(units), max(n, 1),
                                       _stream(stream)))
    return units


def kblock_max(nslices: int = NUM_SLICES) -> int:
    """Largest k-block of the product entry points (longer k runs in blocks)."""
    return lib.dd_gemm_kblock_max(nslices)


def _gemm_args(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo):
    lda = _matrix(A_hi, "A_hi")
    _check_lo(A_lo, A_hi, "A_lo")
    ldb = _matrix(B_hi, "B_hi")
    _check_lo(B_lo, B_hi, "B_lo")
    m, k = A_hi.shape
    k2, n = B_hi.shape
    if k != k2:
        raise ValueError(f"inner dimensions differ: {k} vs {k2}")
    dev = _device(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo)
    C_hi = torch.empty((m, n), dtype=torch.float64, device=dev) if C_hi is None else C_hi
    C_lo = torch.empty((m, n), dtype=torch.float64, device=dev) if C_lo is None else C_lo
    ldc = _matrix(C_hi, "C_hi", (m, n))
    _check_lo(C_lo, C_hi, "C_lo")
    return m, n, k, lda, ldb, ldc, C_hi, C_lo, dev


def dd_gemm(A_hi, A_lo, B_hi, B_lo, C_hi=None, C_lo=None, workspace=None, stream=None,
            nslices: int = NUM_SLICES, kblock: int | None = None):
    """C = A·B; returns (C_hi, C_lo).  ``nslices`` = 8 is the double-double
    product; 4..7 keep fewer slices (n(n+1)/2 pairs) for less accuracy and time,
    9..16 more, for entries far below their row's (column's) largest.  ``kblock``
    cuts k into blocks summed in double-double arithmetic (k beyond k_max(n) is
    blocked automatically).
    The workspace comes from PyTorch's allocator unless a uint8 device tensor of
    at least workspace_size(m, n, k, nslices) bytes is given."""
    m, n, k, lda, ldb, ldc, C_hi, C_lo, dev = _gemm_args(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo)
    with torch.cuda.device(dev):
        workspace = _workspace(workspace, workspace_size(m, n, k, nslices, kblock), dev, stream)
        _dd_gemm_call(m, n, k, nslices, kblock, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, workspace, stream)
    return C_hi, C_lo


def _dd_gemm_call(m, n, k, nslices, kblock, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, workspace, stream):
    if kblock is not None:
        _check(lib.dd_gemm_ws_kb(m, n, k, nslices, kblock, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo),
                                 ldb, _ptr(C_hi), _ptr(C_lo), ldc, _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    elif nslices == NUM_SLICES:
        _check(lib.dd_gemm_ws(m, n, k, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo), ldb,
                              _ptr(C_hi), _ptr(C_lo), ldc, _ptr(workspace), workspace.numel(), _stream(stream)))
    else:
        _check(lib.dd_gemm_ws_ns(m, n, k, nslices, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo), ldb,
                                 _ptr(C_hi), _ptr(C_lo), ldc, _ptr(workspace), workspace.numel(), _stream(stream)))


def dd_gemm_timed(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo, workspace, after_split, stream=None,
                  nslices: int = NUM_SLICES):
    """dd_gemm on the caller's workspace, recording the hipEvent_t handle
    `after_split` (an int, or None) on the stream once the operands are sliced."""
    m, n, k, lda, ldb, ldc, C_hi, C_lo, dev = _gemm_args(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo)
    workspace = _workspace(workspace, workspace_size(m, n, k, nslices), dev, stream)
    with torch.cuda.device(dev):
        _check(lib.dd_gemm_ws_timed(m, n, k, nslices, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo), ldb,
                                    _ptr(C_hi), _ptr(C_lo), ldc, _ptr(workspace), workspace.numel(), after_split,
                                    _stream(stream)))
    return C_hi, C_lo


def dd_gemm_alloc(A_hi, A_lo, B_hi, B_lo, C_hi=None, C_lo=None, stream=None):
    """C = A·B through the entry point that allocates its own (stream-ordered) workspace."""
    m, n, k, lda, ldb, ldc, C_hi, C_lo, dev = _gemm_args(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo)
    with torch.cuda.device(dev):
        _check(lib.dd_gemm(m, n, k, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo), ldb,
                           _ptr(C_hi), _ptr(C_lo), ldc, _stream(stream)))
    return C_hi, C_lo


def dd_gemm_noalloc(A_hi, A_lo, B_hi, B_lo, C_hi=None, C_lo=None, stream=None):
    """C = A·B through the entry point that allocates nothing: its workspace is
    the library's own device array of NOALLOC_SCRATCH_BYTES per GPU (products
    needing more are rejected).  Calls that overlap on one GPU race on it."""
    m, n, k, lda, ldb, ldc, C_hi, C_lo, dev = _gemm_args(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo)
    with torch.cuda.device(dev):
        _check(lib.dd_gemm_noalloc(m, n, k, _ptr(A_hi), _ptr(A_lo), lda, _ptr(B_hi), _ptr(B_lo), ldb,
                                   _ptr(C_hi), _ptr(C_lo), ldc, _stream(stream)))
    return C_hi, C_lo


# ---------------------------------------------------------------------------
# quad-double product
# ---------------------------------------------------------------------------
def _qd_planes(X, name, shape=None):
    """Components of a quad-double matrix: a (4, rows, cols) tensor or a sequence
    of up to four (rows, cols) tensors (None after the first = zero plane).
    Returns (components, leading dimension, ctypes array of four pointers)."""
    comps = [X[c] for c in range(X.shape[0])] if isinstance(X, torch.Tensor) else list(X)
    if not 1 <= len(comps) <= 4 or comps[0] is None:
        raise ValueError(f"{name} needs one to four component planes, the first present")
    ld = _matrix(comps[0], f"{name}[0]", shape)
    for c, t in enumerate(comps[1:], 1):
        if t is not None:
            _matrix(t, f"{name}[{c}]", comps[0].shape)
            if t.stride() != comps[0].stride():
                raise ValueError(f"{name}[{c}] must have the strides of {name}[0]")
    comps = comps + [None] * (4 - len(comps))
    return comps, ld, (ctypes.c_void_p * 4)(*[_ptr(t) for t in comps])


def _qd_out(C, m, n, device):
    if C is None:
        C = torch.empty((4, m, n), dtype=torch.float64, device=device)
    comps = [C[c] for c in range(4)] if isinstance(C, torch.Tensor) else list(C)
    if len(comps) != 4 or any(t is None for t in comps):
        raise ValueError("C needs four component planes")
    ldc = _matrix(comps[0], "C[0]", (m, n))
    for c in range(1, 4):
        _matrix(comps[c], f"C[{c}]", (m, n))
        if comps[c].stride() != comps[0].stride():
            raise ValueError(f"C[{c}] must have the strides of C[0]")
    return C, ldc, (ctypes.c_void_p * 4)(*[_ptr(t) for t in comps])


def qd_slices_bytes(outer: int, k: int) -> int:
    return lib.qd_split_slices_bytes(outer, k)


def qd_workspace_size(m: int, n: int, k: int, kblock: int | None = None) -> int:
    if kblock is not None:
        return lib.qd_gemm_workspace_size_kb(m, n, k, kblock)
    return lib.qd_gemm_workspace_size(m, n, k)


def qd_split_balanced(X, axis: int, exps=None, slices=None, stream=None):
    """Balancing exponents and the sixteen packed slices of one quad-double operand."""
    comps, ldx, arr = _qd_planes(X, "X")
    rows, cols = comps[0].shape
    outer = rows if axis == 0 else cols
    k = cols if axis == 0 else rows
    dev = _device(*comps)
    if exps is None:
        exps = torch.empty(outer, dtype=torch.int32, device=dev)
    if slices is None:
        slices = torch.empty(qd_slices_bytes(outer, k) // 8, dtype=torch.float64, device=dev)
    _buffer(exps, "exps", torch.int32, outer, dev)
    _buffer(slices, "slices", torch.float64, qd_slices_bytes(outer, k) // 8, dev)
    _check(lib.qd_split_balanced(rows, cols, arr, ldx, axis, _ptr(exps), _ptr(slices), _stream(stream)))
    return exps, slices


def qd_sliced_gemm_renorm(m, n, k, A_slices, E, B_slices, F, C=None, stream=None):
    """Level sums of the 136 slice pairs and the exact four-double epilogue; returns C."""
    dev = A_slices.device
    _buffer(A_slices, "A_slices", torch.float64, qd_slices_bytes(m, k) // 8, dev)
    _buffer(B_slices, "B_slices", torch.float64, qd_slices_bytes(n, k) // 8, dev)
    _buffer(E, "E", torch.int32, m, dev)
    _buffer(F, "F", torch.int32, n, dev)
    C, ldc, arr = _qd_out(C, m, n, dev)
    _device(A_slices, *[C[q] for q in range(4)])
    _check(lib.qd_sliced_gemm_renorm(m, n, k, _ptr(A_slices), _ptr(E), _ptr(B_slices), _ptr(F), arr, ldc,
                                     _stream(stream)))
    return C


def _qd_gemm_args(A, B, C):
    a, lda, pa = _qd_planes(A, "A")
    b, ldb, pb = _qd_planes(B, "B")
    m, k = a[0].shape
    k2, n = b[0].shape
    if k != k2:
        raise ValueError(f"inner dimensions differ: {k} vs {k2}")
    dev = _device(*a, *b, *(C if C is not None else []))
    C, ldc, pc = _qd_out(C, m, n, dev)
    return m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev


def qd_gemm(A, B, C=None, workspace=None, stream=None, kblock: int | None = None):
    """C = A·B for quad-double A (m×k) and B (k×n); returns C as a (4, m, n) tensor
    (or the given planes).  The workspace comes from PyTorch's allocator unless a
    uint8 device tensor of at least qd_workspace_size(m, n, k, kblock) bytes is
    given.  ``kblock`` runs the product in k-blocks of that many terms (the
    result does not depend on it); by default k is split only beyond QD_K_MAX."""
    m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev = _qd_gemm_args(A, B, C)
    with torch.cuda.device(dev):
        workspace = _workspace(workspace, qd_workspace_size(m, n, k, kblock), dev, stream)
        if kblock is None:
            _check(lib.qd_gemm_ws(m, n, k, pa, lda, pb, ldb, pc, ldc, _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
        else:
            _check(lib.qd_gemm_ws_kb(m, n, k, kblock, pa, lda, pb, ldb, pc, ldc, _ptr(workspace),
                                     workspace.numel(), _stream(stream)))
    return C


def qd_gemm_timed(A, B, C, workspace, after_split, stream=None):
    """qd_gemm on the caller's workspace, recording the hipEvent_t handle
    `after_split` (an int, or None) on the stream once the operands are sliced."""
    m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev = _qd_gemm_args(A, B, C)
    with torch.cuda.device(dev):
        workspace = _workspace(workspace, qd_workspace_size(m, n, k), dev, stream)
        _check(lib.qd_gemm_ws_timed(m, n, k, pa, lda, pb, ldb, pc, ldc, _ptr(workspace), workspace.numel(),
                                    after_split, _stream(stream)))
    return C


def qd_gemm_alloc(A, B, C=None, stream=None):
    """C = A·B through the entry point that allocates its own (stream-ordered) workspace."""
    m, n, k, pa, lda, pb, ldb, C, pc, ldc, dev = _qd_gemm_args(A, B, C)
    with torch.cuda.device(dev):
        _check(lib.qd_gemm(m, n, k, pa, lda, pb, ldb, pc, ldc, _stream(stream)))
    return C


def probe_mfma_f64(device="cuda", stream=None):
    out = torch.empty((64, 4), dtype=torch.float64, device=device)
    _check(lib.ddgemm_probe_mfma_f64(_ptr(out), _stream(stream)))
    return out


def probe_pair_round(units, scale, out=None, stream=None, nslices: int = NUM_SLICES):
    """The products' exit rounding on given group sums (diagnostics):
    ``units`` int64 (count, nslices - 1) on a device, ``scale`` int32 (count,);
    returns float64 (count, 2): the nearest double-double of each entry's exact
    total sum_g units[i, g] 2^(scale[i] - 13(g + 3))."""
    if units.dim() != 2 or units.shape[1] != nslices - 1:
        raise ValueError(f"units must have shape (count, {nslices - 1}), got {tuple(units.shape)}")
    dev = units.device
    count = units.shape[0]
    _buffer(units, "units", torch.int64, count * (nslices - 1), dev)
    _buffer(scale, "scale", torch.int32, count, dev)
    if out is None:
        out = torch.empty((count, 2), dtype=torch.float64, device=dev)
    _buffer(out, "out", torch.float64, 2 * count, dev)
    with torch.cuda.device(dev):
        _check(lib.ddgemm_probe_pair_round(count, nslices, _ptr(units), _ptr(scale), _ptr(out), _stream(stream)))
    return out