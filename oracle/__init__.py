"""CPU oracle for the fused add + argmax readout (ctypes front of ``oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the package smoke
check and the benchmark's CPU-baseline leg import this module.  It shares no
code with the GPU library and the GPU library never calls it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C); this file only
builds it with gcc when no build is present and marshals numpy arrays.  What
the oracle computes is stated in the header comment of ``oracle.c``, with the
passages of the XPress kernels page it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_U16P = ctypes.POINTER(ctypes.c_uint16)
_I64P = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` to ``liboracle.so`` with plain gcc (no fast-math,
    no FMA contraction) and return the library path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        lib.oracle_bf16_from_double.restype = ctypes.c_uint16
        lib.oracle_bf16_sum.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        lib.oracle_bf16_sum.restype = ctypes.c_uint16
        lib.oracle_bf16_sum_many.argtypes = [_U16P, _U16P, _U16P, ctypes.c_int64]
        lib.oracle_bf16_sum_many.restype = None
        lib.oracle_bf16_sum_grid.argtypes = [_U16P, ctypes.c_int64, _U16P]
        lib.oracle_bf16_sum_grid.restype = None
        lib.oracle_add_argmax_row.argtypes = [_U16P, _U16P, ctypes.c_int64]
        lib.oracle_add_argmax_row.restype = ctypes.c_int64
        lib.oracle_add_argmax_to_blk.argtypes = [
            _U16P, _U16P, _I64P] + [ctypes.c_int64] * 5
        lib.oracle_add_argmax_to_blk.restype = ctypes.c_int
        lib.oracle_add_argmax_rows.argtypes = [
            _U16P, _U16P, _I64P] + [ctypes.c_int64] * 5
        lib.oracle_add_argmax_rows.restype = ctypes.c_int
        lib.oracle_topc_argmax_to_blk.argtypes = [
            _U16P, _U16P, _I64P, _I64P] + [ctypes.c_int64] * 3
        lib.oracle_topc_argmax_to_blk.restype = ctypes.c_int
        lib.oracle_dot_bf16.argtypes = [_U16P, _U16P, ctypes.c_int64]
        lib.oracle_dot_bf16.restype = ctypes.c_uint16
        lib.oracle_gemm_argmax_rows.argtypes = [
            _U16P, _U16P, _U16P, _I64P] + [ctypes.c_int64] * 5
        lib.oracle_gemm_argmax_rows.restype = ctypes.c_int
        _DP = ctypes.POINTER(ctypes.c_double)
        lib.oracle_bf16_to_double_many.argtypes = [_U16P, _DP, ctypes.c_int64]
        lib.oracle_bf16_to_double_many.restype = None
        lib.oracle_gemm_argmax_rows_decoded.argtypes = [
            _U16P, _DP, _DP, _I64P] + [ctypes.c_int64] * 5
        lib.oracle_gemm_argmax_rows_decoded.restype = ctypes.c_int
        lib.oracle_bf16_from_double_many.argtypes = [_DP, _U16P, ctypes.c_int64]
        lib.oracle_bf16_from_double_many.restype = None
        lib.oracle_latent_pass.argtypes = (
            [_I64P, _I64P] + [_U16P] * 7 + [_U16P] + [ctypes.c_int64] * 5 + [_DP] * 6)
        lib.oracle_latent_pass.restype = ctypes.c_int
        _lib = lib
        return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def _p16(a: np.ndarray):
    return a.ctypes.data_as(_U16P)


def bf16_to_double(h: int) -> float:
    """Exact value of one bf16 bit pattern."""
    return _load().oracle_bf16_to_double(int(h) & 0xFFFF)


def bf16_from_double(x: float) -> int:
    """Nearest bf16 (ties to even) of a binary64 value, as a bit pattern."""
    return int(_load().oracle_bf16_from_double(float(x)))


def bf16_from_double_many(x) -> np.ndarray:
    """bf16 patterns (uint16) of float64 values, each rounded once to nearest
    even; same shape as x."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_from_double_many(
        x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _p16(out), x.size)
    return out


def bf16_sum(a: int, b: int) -> int:
    """bf16(a + b) of two bf16 bit patterns."""
    return int(_load().oracle_bf16_sum(int(a) & 0xFFFF, int(b) & 0xFFFF))


def bf16_sum_many(a, b) -> np.ndarray:
    """Element-wise bf16(a + b) over two equal-shape uint16 arrays."""
    a = _u16(a)
    b = _u16(b)
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_bf16_sum_many(_p16(a), _p16(b), _p16(out), a.size)
    return out


def bf16_sum_grid(a_vals) -> np.ndarray:
    """``out[i, b] = bf16(a_vals[i] + b)`` for all 65536 patterns b."""
    a_vals = _u16(a_vals).reshape(-1)
    out = np.empty((a_vals.size, 65536), dtype=np.uint16)
    _load().oracle_bf16_sum_grid(_p16(a_vals), a_vals.size, _p16(out))
    return out


def add_argmax_row(base_row, bias_row) -> int:
    """First index of the maximum of bf16(base_row + bias_row)."""
    a = _u16(base_row).reshape(-1)
    b = _u16(bias_row).reshape(-1)
    if a.size != b.size or a.size < 1:
        raise ValueError("rows must be non-empty and of equal length")
    return int(_load().oracle_add_argmax_row(_p16(a), _p16(b), a.size))


def _check_layout(buf: np.ndarray, rows: int, V: int, stride: int, name: str):
    if stride < V:
        raise ValueError("%s row stride %d < V=%d" % (name, stride, V))
    need = (rows - 1) * stride + V if rows > 0 else 0
    if buf.size < need:
        raise ValueError("%s holds %d elements, layout needs %d" % (name, buf.size, need))


def add_argmax_to_blk(base, bias, blk: np.ndarray, N: int, B: int, V: int,
                      stride_base_r: int, stride_bias_r: int) -> None:
    """In-place oracle readout on host arrays; same argument meaning as the
    GPU entry point.  ``blk`` must be a C-contiguous int64 array of N*B."""
    base = _u16(base)
    bias = _u16(bias)
    if blk.dtype != np.int64 or not blk.flags.c_contiguous or blk.size != N * B:
        raise ValueError("blk must be a C-contiguous int64 array of N*B elements")
    rows = N * (B - 1)
    _check_layout(base, rows, V, stride_base_r, "base")
    _check_layout(bias, rows, V, stride_bias_r, "bias")
    rc = _load().oracle_add_argmax_to_blk(
        _p16(base), _p16(bias), blk.ctypes.data_as(_I64P),
        N, B, V, stride_base_r, stride_bias_r)
    if rc != 0:
        raise ValueError("oracle rejected the layout")


def add_argmax_rows(base, bias, r0: int, r1: int, V: int, stride_base_r: int,
                    stride_bias_r: int) -> np.ndarray:
    """Argmax of rows [r0, r1) as an int64 array (no blk scatter)."""
    base = _u16(base)
    bias = _u16(bias)
    _check_layout(base, r1, V, stride_base_r, "base")
    _check_layout(bias, r1, V, stride_bias_r, "bias")
    out = np.empty(max(r1 - r0, 0), dtype=np.int64)
    rc = _load().oracle_add_argmax_rows(
        _p16(base), _p16(bias), out.ctypes.data_as(_I64P), r0, r1, V,
        stride_base_r, stride_bias_r)
    if rc != 0:
        raise ValueError("oracle rejected the layout")
    return out


def add_argmax_rows_threaded(base, bias, rows: int, V: int, stride_base_r: int,
                             stride_bias_r: int, threads: int) -> np.ndarray:
    """The same per-row oracle, rows split evenly over ``threads`` host
    threads (ctypes releases the GIL during each call)."""
    base = _u16(base)
    bias = _u16(bias)
    out = np.empty(rows, dtype=np.int64)
    threads = max(1, min(int(threads), rows if rows > 0 else 1))
    bounds = [rows * t // threads for t in range(threads + 1)]

    def work(t):
        r0, r1 = bounds[t], bounds[t + 1]
        out[r0:r1] = add_argmax_rows(base, bias, r0, r1, V, stride_base_r,
                                     stride_bias_r)

    ts = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return out


def topc_argmax_to_blk(base_c, bias_c, cand, blk: np.ndarray, N: int, B: int, C: int) -> None:
    """In-place top-C oracle on host arrays: for draft row r = n*(B-1) + j,
    blk[n, 1+j] = cand[r, first argmax_c bf16(base_c[r, c] + bias_c[r, c])].
    base_c / bias_c: uint16 bf16 patterns, cand: int64, all [N*(B-1), C]
    contiguous; blk: C-contiguous int64 of N*B elements."""
    base_c = _u16(base_c).reshape(-1)
    bias_c = _u16(bias_c).reshape(-1)
    cand = np.ascontiguousarray(cand, dtype=np.int64).reshape(-1)
    rows = N * (B - 1)
    if C < 1 or base_c.size < rows * C or bias_c.size < rows * C or cand.size < rows * C:
        raise ValueError("top-C buffers do not hold N*(B-1)*C candidates")
    if blk.dtype != np.int64 or not blk.flags.c_contiguous or blk.size != N * B:
        raise ValueError("blk must be a C-contiguous int64 array of N*B elements")
    rc = _load().oracle_topc_argmax_to_blk(
        _p16(base_c), _p16(bias_c), cand.ctypes.data_as(_I64P), blk.ctypes.data_as(_I64P),
        N, B, C)
    if rc != 0:
        raise ValueError("oracle rejected the sizes")


def dot_bf16(x_row, w_row) -> int:
    """bf16 pattern of the dot product of two bf16 rows, rounded once."""
    a = _u16(x_row).reshape(-1)
    b = _u16(w_row).reshape(-1)
    if a.size != b.size or a.size < 1:
        raise ValueError("rows must be non-empty and of equal length")
    return int(_load().oracle_dot_bf16(_p16(a), _p16(b), a.size))


def bf16_to_double_many(h) -> np.ndarray:
    """binary64 values of an array of bf16 patterns (the oracle's decoding)."""
    h = _u16(h).reshape(-1)
    out = np.empty(h.size, dtype=np.float64)
    _load().oracle_bf16_to_double_many(_p16(h), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                       h.size)
    return out


def gemm_argmax_rows(base, x, w, rows, V: int, R: int, stride_base_r: int,
                     threads: int = 1) -> np.ndarray:
    """First argmax of bf16(base + bf16(x @ w.T)) for each row listed in
    ``rows`` (an iterable of row indices); base [.., stride], x [.., R] and
    w [V, R] are uint16 bf16 patterns.  x and w are decoded to binary64 once
    (``oracle_gemm_argmax_rows_decoded``: the same arithmetic as
    ``oracle_gemm_argmax_rows``); rows are spread over host threads."""
    base = _u16(base).reshape(-1)
    x = _u16(x).reshape(-1)
    w = _u16(w).reshape(-1)
    rows = [int(r) for r in rows]
    if w.size < V * R:
        raise ValueError("w must hold V*R elements")
    for r in rows:
        if r < 0 or (r + 1) * R > x.size or r * stride_base_r + V > base.size:
            raise ValueError("row %d outside the buffers" % r)
    out = np.empty(len(rows), dtype=np.int64)
    if not rows:
        return out
    lib = _load()
    dp = ctypes.POINTER(ctypes.c_double)
    wd = bf16_to_double_many(w[:V * R])
    xd = bf16_to_double_many(x[:(max(rows) + 1) * R])

    def work(idx):
        one = np.empty(1, dtype=np.int64)
        for j in idx:
            r = rows[j]
            rc = lib.oracle_gemm_argmax_rows_decoded(_p16(base), xd.ctypes.data_as(dp),
                                                     wd.ctypes.data_as(dp),
                                                     one.ctypes.data_as(_I64P), r, r + 1, V, R,
                                                     stride_base_r)
            if rc != 0:
                raise ValueError("oracle rejected the sizes")
            out[j] = one[0]

    threads = max(1, min(int(threads), len(rows)))
    parts = [list(range(t, len(rows), threads)) for t in range(threads)]
    ts = [threading.Thread(target=work, args=(p,)) for p in parts]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return out


def latent_pass(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, N: int, B: int, R: int,
                H: int, V: int, intermediates: bool = False, threads: int = 1):
    """Latent stage of one pass on host arrays (see ``oracle_latent_pass``).

    blk [N, B] and am1 [N] are int64; xh [N, B, R], w1 [V, R], wlat [R, R],
    mixl [B, B, R], wg / wu [H, R] and wd [R, H] are uint16 bf16 patterns.
    Returns out [N, B-1, R] as uint16 bf16 patterns, and with
    ``intermediates`` also a dict of the binary64 values before rounding:
    x / u [N, B, R], g / v / f [N, B-1, H], o [N, B-1, R].  Blocks are
    independent, so they are spread over host threads."""
    blk = np.ascontiguousarray(blk, dtype=np.int64).reshape(N, B)
    am1 = np.ascontiguousarray(am1, dtype=np.int64).reshape(N)
    xh = _u16(xh).reshape(N, B, R)
    w1 = _u16(w1).reshape(V, R)
    wlat = _u16(wlat).reshape(R, R)
    mixl = _u16(mixl).reshape(B, B, R)
    wg = _u16(wg).reshape(H, R)
    wu = _u16(wu).reshape(H, R)
    wd = _u16(wd).reshape(R, H)
    out = np.zeros((N, B - 1, R), dtype=np.uint16)
    inter = None
    if intermediates:
        inter = {"x": np.zeros((N, B, R)), "u": np.zeros((N, B, R)),
                 "g": np.zeros((N, B - 1, H)), "v": np.zeros((N, B - 1, H)),
                 "f": np.zeros((N, B - 1, H)), "o": np.zeros((N, B - 1, R))}
    lib = _load()
    dp = ctypes.POINTER(ctypes.c_double)
    errors = []

    def dptr(name, n0):
        if inter is None:
            return ctypes.cast(None, dp)
        return inter[name][n0:].ctypes.data_as(dp)

    def work(n0, n1):
        rc = lib.oracle_latent_pass(
            blk[n0:].ctypes.data_as(_I64P), am1[n0:].ctypes.data_as(_I64P),
            _p16(xh[n0:]), _p16(w1), _p16(wlat), _p16(mixl), _p16(wg), _p16(wu),
            _p16(wd), _p16(out[n0:]), n1 - n0, B, R, H, V,
            dptr("x", n0), dptr("u", n0), dptr("g", n0), dptr("v", n0),
            dptr("f", n0), dptr("o", n0))
        if rc != 0:
            errors.append(rc)

    threads = max(1, min(int(threads), N if N else 1))
    bounds = [(N * t // threads, N * (t + 1) // threads) for t in range(threads)]
    ts = [threading.Thread(target=work, args=b) for b in bounds if b[1] > b[0]]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errors:
        raise ValueError("oracle rejected the latent inputs (code %d)" % errors[0])
    return (out, inter) if intermediates else out
