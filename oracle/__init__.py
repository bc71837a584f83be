"""CPU oracle of the Q8_0 weight product -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does; the two share no code.  The arithmetic lives in ``q8_oracle.c`` (plain C,
fp64 / int64), built by ``oracle/build.py``; this module marshals numpy arrays
to it.

Every array here is in the canonical layout of the pages
(logicaffeine_compile/spatial/passes/from_q8.rs, module doc): values ``q`` are
``K x N`` int8 (k outer), scales ``s`` are ``K/32 x N`` fp32, the activation
``x`` is ``m x K`` bf16 given as its raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK = 32

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _configure(lib):
    """Declare the C signatures on a loaded oracle library."""
    lib.q8o_set_threads.argtypes = [ctypes.c_int]
    lib.q8o_threads.restype = ctypes.c_int
    lib.q8o_quantize_exact.argtypes = [_p, _i64, _i64, _p, _p]
    lib.q8o_quantize_exact.restype = ctypes.c_int
    lib.q8o_dequant.argtypes = [_p, _p, _i64, _i64, _p]
    lib.q8o_quantize_act.argtypes = [_p, _i64, _i64, _p, _p]
    lib.q8o_quantize_rows_f32.argtypes = [_p, _i64, _i64, _p, _p]
    lib.q8o_gemv_bf16.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.q8o_gemv_bf16.restype = ctypes.c_int
    lib.q8o_block_dots.argtypes = [_p, _p, _i64, _i64, _i64, _p, _i64, _p]
    lib.q8o_block_dots.restype = ctypes.c_int
    lib.q8o_gemv_q8.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.q8o_gemv_q8.restype = ctypes.c_int
    lib.q8o_quantize_act_two_words.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.q8o_gemv_q8_two_words.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i64,
                                          _p, _p]
    lib.q8o_gemv_q8_two_words.restype = ctypes.c_int
    lib.q8o_swiglu.argtypes = [_p, _p, _p, _p, _i64, _i64, _p]
    lib.q8o_epilogue.argtypes = [_p, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p]
    lib.q8o_view_rows.argtypes = [_i64, _i64]
    lib.q8o_view_rows.restype = _i64
    lib.q8o_fold_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64,
                                   ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # compiles the C oracle with gcc
        _build.build()
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def swap_library(path: Optional[str]):
    """Use the oracle library at `path` (None: the built one) for the calls
    below; returns the previous handle.  For the mutation tests, which plant
    a mistake in a copy of q8_oracle.c and check that the pins catch it."""
    global _lib
    prev = _lib
    _lib = None if path is None else _configure(ctypes.CDLL(path))
    return prev


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use (0: the OpenMP default)."""
    _load().q8o_set_threads(int(n))


def threads() -> int:
    return int(_load().q8o_threads())


def _cols(cols: Optional[Sequence[int]], N: int):
    if cols is None:
        return None, N
    c = _c(cols, np.int64)
    if c.ndim != 1 or (c.size and (c.min() < 0 or c.max() >= N)):
        raise ValueError("column list out of range")
    return c, int(c.size)


def quantize_exact(w: np.ndarray) -> Optional[Tuple[np.ndarray, np.ndarray]]:
    """The pages' exact Q8_0 encoder (from_q8.rs, fn quantize): ``(q, s)``, or
    ``None`` when some block is not an int8 multiple of its fp32 ``amax/127``."""
    w = _c(w, np.float64)
    K, N = w.shape
    q = np.zeros((K, N), np.int8)
    s = np.zeros((K // BLOCK, N), np.float32)
    rc = _load().q8o_quantize_exact(_ptr(w), K, N, _ptr(q), _ptr(s))
    if rc < 0:
        raise ValueError(f"bad shape {w.shape}: K must be a positive multiple of {BLOCK}")
    return (q, s) if rc == 1 else None


def dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """``w = q * d`` per element, fp64."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    K, N = q.shape
    w = np.empty((K, N), np.float64)
    _load().q8o_dequant(_ptr(q), _ptr(s), K, N, _ptr(w))
    return w


def quantize_act(x_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-32-block int8 activation and its fp32 scales (reading in q8_oracle.c)."""
    x = _c(x_bf16, np.uint16)
    m, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    xq = np.empty((m, K), np.int8)
    dx = np.empty((m, K // BLOCK), np.float32)
    _load().q8o_quantize_act(_ptr(x), m, K, _ptr(xq), _ptr(dx))
    return xq, dx


def quantize_rows_f32(z: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The quantized form of an fp32 ``m x K`` array (a product's output as the
    next projection reads it): int8 values and one fp32 scale per 32."""
    z = _c(z, np.float32)
    m, K = z.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    zq = np.empty((m, K), np.int8)
    dz = np.empty((m, K // BLOCK), np.float32)
    _load().q8o_quantize_rows_f32(_ptr(z), m, K, _ptr(zq), _ptr(dz))
    return zq, dz


def gemv_bf16(x_bf16: np.ndarray, q: np.ndarray, s: np.ndarray,
              cols: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``(y, bound)``, both fp64 ``m x len(cols)``: ``y = x . W`` and
    ``bound = sum_k |x_k w_kn|`` for bf16 activations."""
    x = _c(x_bf16, np.uint16)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    m, K = x.shape
    K2, N = q.shape
    if K2 != K or s.shape != (K // BLOCK, N):
        raise ValueError("shape mismatch")
    c, nc = _cols(cols, N)
    y = np.empty((m, nc), np.float64)
    b = np.empty((m, nc), np.float64)
    rc = _load().q8o_gemv_bf16(_ptr(x), _ptr(q), _ptr(s), m, K, N,
                               None if c is None else _ptr(c), nc, _ptr(y), _ptr(b))
    if rc:
        raise ValueError("bad shape")
    return y, b


def block_dots(xq: np.ndarray, q: np.ndarray,
               cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """int64 ``D[r, b, j] = sum_i xq[r, 32b+i] * q[32b+i, cols[j]]``."""
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    m, K = xq.shape
    K2, N = q.shape
    if K2 != K:
        raise ValueError("shape mismatch")
    c, nc = _cols(cols, N)
    D = np.empty((m, K // BLOCK, nc), np.int64)
    rc = _load().q8o_block_dots(_ptr(xq), _ptr(q), m, K, N,
                                None if c is None else _ptr(c), nc, _ptr(D))
    if rc:
        raise ValueError("bad shape")
    return D


def gemv_q8(xq: np.ndarray, dx: np.ndarray, q: np.ndarray, s: np.ndarray,
            cols: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``(y, bound)`` for int8 activations ``x_k = dx[r, k/32] * xq[r, k]``."""
    xq = _c(xq, np.int8)
    dx = _c(dx, np.float32)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    m, K = xq.shape
    K2, N = q.shape
    if K2 != K or dx.shape != (m, K // BLOCK) or s.shape != (K // BLOCK, N):
        raise ValueError("shape mismatch")
    c, nc = _cols(cols, N)
    y = np.empty((m, nc), np.float64)
    b = np.empty((m, nc), np.float64)
    rc = _load().q8o_gemv_q8(_ptr(xq), _ptr(dx), _ptr(q), _ptr(s), m, K, N,
                             None if c is None else _ptr(c), nc, _ptr(y), _ptr(b))
    if rc:
        raise ValueError("bad shape")
    return y, b


def quantize_act_two_words(x_bf16: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The two-word form of a bf16 activation: ``(hi, lo, dx)``, two ``m x K``
    int8 words and one fp32 scale per 32, standing for
    ``dx * (hi + lo / 128)`` (reading in q8_oracle.c)."""
    x = _c(x_bf16, np.uint16)
    m, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    hi = np.empty((m, K), np.int8)
    lo = np.empty((m, K), np.int8)
    dx = np.empty((m, K // BLOCK), np.float32)
    _load().q8o_quantize_act_two_words(_ptr(x), m, K, _ptr(hi), _ptr(lo), _ptr(dx))
    return hi, lo, dx


def gemv_q8_two_words(hi: np.ndarray, lo: np.ndarray, dx: np.ndarray, q: np.ndarray,
                      s: np.ndarray, cols: Optional[Sequence[int]] = None
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """``(y, bound)`` for two-word int8 activations
    ``x_k = dx[r, k/32] * (hi[r, k] + lo[r, k] / 128)``."""
    hi = _c(hi, np.int8)
    lo = _c(lo, np.int8)
    dx = _c(dx, np.float32)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    m, K = hi.shape
    K2, N = q.shape
    if (lo.shape != hi.shape or K2 != K or dx.shape != (m, K // BLOCK)
            or s.shape != (K // BLOCK, N)):
        raise ValueError("shape mismatch")
    c, nc = _cols(cols, N)
    y = np.empty((m, nc), np.float64)
    b = np.empty((m, nc), np.float64)
    rc = _load().q8o_gemv_q8_two_words(_ptr(hi), _ptr(lo), _ptr(dx), _ptr(q), _ptr(s), m, K,
                                       N, None if c is None else _ptr(c), nc, _ptr(y), _ptr(b))
    if rc:
        raise ValueError("bad shape")
    return y, b


def swiglu(g: np.ndarray, u: np.ndarray, bg: Optional[np.ndarray] = None,
           bu: Optional[np.ndarray] = None) -> np.ndarray:
    """``silu(g + bg) * (u + bu)`` elementwise, fp64 (plan.rs, Launch::GemvGlu)."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    if g.shape != u.shape or g.ndim != 2:
        raise ValueError("g and u must be equal m x n arrays")
    m, n = g.shape
    b1 = None if bg is None else _c(bg, np.float32)
    b2 = None if bu is None else _c(bu, np.float32)
    for b in (b1, b2):
        if b is not None and b.shape != (n,):
            raise ValueError("bias must have n values")
    out = np.empty((m, n), np.float64)
    _load().q8o_swiglu(_ptr(g), _ptr(u), None if b1 is None else _ptr(b1),
                       None if b2 is None else _ptr(b2), m, n, _ptr(out))
    return out


def gemv_glu_bf16(x_bf16, qg, sg, qu, su, bg=None, bu=None, cols=None):
    """The gated pair on bf16 activations: ``(out, g, u, bound_g, bound_u)``,
    fp64 over the listed columns (biases indexed by column)."""
    g, bnd_g = gemv_bf16(x_bf16, qg, sg, cols)
    u, bnd_u = gemv_bf16(x_bf16, qu, su, cols)
    c = slice(None) if cols is None else np.asarray(cols)
    out = swiglu(g, u, None if bg is None else np.asarray(bg)[c],
                 None if bu is None else np.asarray(bu)[c])
    return out, g, u, bnd_g, bnd_u


def gemv_glu_q8(xq, dx, qg, sg, qu, su, bg=None, bu=None, cols=None):
    """The gated pair on int8 activations, as gemv_glu_bf16."""
    g, bnd_g = gemv_q8(xq, dx, qg, sg, cols)
    u, bnd_u = gemv_q8(xq, dx, qu, su, cols)
    c = slice(None) if cols is None else np.asarray(cols)
    out = swiglu(g, u, None if bg is None else np.asarray(bg)[c],
                 None if bu is None else np.asarray(bu)[c])
    return out, g, u, bnd_g, bnd_u


def epilogue(y: np.ndarray, bound: np.ndarray, bias: Optional[np.ndarray] = None,
             residual: Optional[np.ndarray] = None,
             cols: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``(z, bound)`` of a fused projection: ``z = y + bias + residual`` over
    the listed columns, in fp64 (plan.rs, enum Launch, variant Gemv, field
    ``bias``; the residual add of its gemv_norm_epilogue note).  ``y, bound``
    are a product's ``m x len(cols)`` output from gemv_bf16 / gemv_q8; ``bias``
    holds one fp32 value per column of the whole output, ``residual`` is an
    fp32 ``m x W`` array (W >= the largest listed column + 1)."""
    y = _c(y, np.float64)
    bound = _c(bound, np.float64)
    m, nc = y.shape
    if bound.shape != y.shape:
        raise ValueError("y and bound must have one shape")
    ncols_all = None
    b = None if bias is None else _c(bias, np.float32)
    r = None if residual is None else _c(residual, np.float32)
    if b is not None:
        ncols_all = b.shape[0]
    if r is not None:
        if r.ndim != 2 or r.shape[0] != m:
            raise ValueError("residual must be m x W")
        ncols_all = r.shape[1] if ncols_all is None else min(ncols_all, r.shape[1])
    c = None
    if cols is not None:
        c = _c(cols, np.int64)
        if c.shape != (nc,):
            raise ValueError("one column per output column")
        if ncols_all is not None and c.size and (c.min() < 0 or c.max() >= ncols_all):
            raise ValueError("column list out of range")
    elif ncols_all is not None and nc > ncols_all:
        raise ValueError("bias or residual narrower than y")
    z = np.empty((m, nc), np.float64)
    zb = np.empty((m, nc), np.float64)
    _load().q8o_epilogue(_ptr(y), _ptr(bound), m, nc, None if c is None else _ptr(c),
                         None if b is None else _ptr(b), None if r is None else _ptr(r),
                         0 if r is None else r.shape[1], _ptr(z), _ptr(zb))
    return z, zb


# ---------------------------------------------------------------------------
# The library's packed weight layout, written out from its definition (layout
# version 2).  The pages fix only the canonical tensors (from_q8.rs, enum
# Q8Part: the host repacks the checkpoint's blocks into a values tensor and a
# scales tensor); the device layout is this library's own choice, and these
# two functions state it independently of the HIP code, as a plain numpy
# permutation of the canonical arrays:
#   * N is padded to N_pad = 64 * ceil(N / 64) with zero values and scales;
#     T = N_pad / 64 column tiles, NB = K / 32 blocks;
#   * values: tile t, block b is a 2048-byte chunk at (t * NB + b) * 2048, in
#     two 1024-byte halves h (rows 0-15 and 16-31 of the block); inside half
#     h, column c (0..63 within the tile) holds its 16 values, k ascending,
#     at bytes c * 16 .. c * 16 + 15;
#   * scales: tile t, block b is a 64-float row at (t * NB + b) * 64; the
#     scale of column c = 16 g + i (i < 16, g < 4) sits at position 4 i + g.
# ---------------------------------------------------------------------------

def _padded(N: int) -> int:
    return (N + 63) // 64 * 64


def repack_ref(q: np.ndarray, s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Packed ``(values, scales)`` of the canonical ``q`` (K x N int8) and
    ``s`` (K/32 x N fp32): ``values`` is ``K * N_pad`` int8, ``scales`` is
    ``K/32 * N_pad`` fp32, both flat."""
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    K, N = q.shape
    if K % BLOCK or s.shape != (K // BLOCK, N):
        raise ValueError("shape mismatch")
    NB, Np = K // BLOCK, _padded(N)
    T = Np // 64
    qp = np.zeros((K, Np), np.int8)
    qp[:, :N] = q
    sp = np.zeros((NB, Np), np.float32)
    sp[:, :N] = s
    # q index (k, n) = (32 b + 16 h + kk, 64 t + c)  ->  [t, b, h, c, kk]
    v = qp.reshape(NB, 2, 16, T, 64).transpose(3, 0, 1, 4, 2)
    # s index (b, n) = (b, 64 t + 16 g + i)  ->  [t, b, i, g]
    w = sp.reshape(NB, T, 4, 16).transpose(1, 0, 3, 2)
    return np.ascontiguousarray(v).ravel(), np.ascontiguousarray(w).ravel()


def unpack_ref(values: np.ndarray, scales: np.ndarray, K: int, N: int
               ) -> Tuple[np.ndarray, np.ndarray]:
    """The inverse of repack_ref: canonical ``(q, s)`` of the first N columns."""
    NB, Np = K // BLOCK, _padded(N)
    T = Np // 64
    v = np.asarray(values).view(np.int8)[: K * Np].reshape(T, NB, 2, 64, 16)
    w = np.asarray(scales, np.float32)[: NB * Np].reshape(T, NB, 16, 4)
    q = v.transpose(1, 2, 4, 0, 3).reshape(K, Np)
    s = w.transpose(1, 0, 3, 2).reshape(NB, Np)
    return np.ascontiguousarray(q[:, :N]), np.ascontiguousarray(s[:, :N])


def act_view_ref(xq: np.ndarray) -> np.ndarray:
    """The block-interleaved view of an ``m x K`` int8 activation, flat: every
    row's 32-value block b side by side, value ``(r, k)`` at
    ``((k // 32) * m + r) * 32 + k % 32`` (from_q8.rs, fn
    relayout_rows_to_q8_view: the rows' blocks of one K range brought
    together so that one block of every row is read as one piece)."""
    xq = _c(xq, np.int8)
    m, K = xq.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    return np.ascontiguousarray(xq.reshape(m, K // BLOCK, BLOCK).transpose(1, 0, 2)).ravel()


def view_rows(m: int, K: int) -> int:
    """Rows of the ``K/32 x 32`` activation view (from_q8.rs, fn q8_view_rows)."""
    return int(_load().q8o_view_rows(m, K))


def fold_bytes(m: int, K: int, N: int, wb: int, x_bytes: int) -> Tuple[int, int]:
    """``(weight, view_reads)`` bytes of the fold by the byte gate of
    from_q8.rs, fn q8_gemv (32-wide column tiles, 1024-row K chunks)."""
    w = _i64()
    v = _i64()
    _load().q8o_fold_bytes(m, K, N, wb, x_bytes, ctypes.byref(w), ctypes.byref(v))
    return int(w.value), int(v.value)


def tolerance_ok(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray,
                 rel: float = 1e-5, abs_: float = 1e-6) -> np.ndarray:
    """Elementwise ``|y_gpu - y_ref| <= rel * bound + abs_``."""
    return np.abs(np.asarray(y_gpu, np.float64) - y_ref) <= rel * bound + abs_
