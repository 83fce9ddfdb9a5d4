"""ctypes binding of ``libxpress_argmax.so`` (declared in include/xpress_argmax.h).

Argument marshalling only: every step of the readout runs in the library's
HIP kernels.  Entry points keep the C names.  Tensor arguments may be torch
tensors on a GPU (their ``data_ptr()`` is passed) or plain integer device
addresses; for a tensor the binding also checks that its storage covers the
bytes the call will touch, which a bare pointer cannot tell the library.  A
nonzero status raises :class:`XpressError`.  If the library has not been
built, the first call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxpress_argmax.so")

XPRESS_OK = 0
XPRESS_EINVAL = 1
XPRESS_EHIP = 2
XPRESS_ENOMEM = 3
XPRESS_ECAPTURE = 4
XPRESS_ESCRATCH = 5

XPRESS_COMBINE_AUTO = 0
XPRESS_COMBINE_SINGLE = 1
XPRESS_COMBINE_ATOMIC = 2
XPRESS_COMBINE_TWO_PASS = 3
XPRESS_COMBINE_BALANCED = 4

COMBINE_NAMES = {XPRESS_COMBINE_SINGLE: "single", XPRESS_COMBINE_ATOMIC: "atomic",
                 XPRESS_COMBINE_TWO_PASS: "two_pass", XPRESS_COMBINE_BALANCED: "balanced"}

_lock = threading.Lock()
_lib = None


class XpressError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s" % (where, xpress_error_string(status))
        if status == XPRESS_EHIP:
            msg += " (hipError %d)" % xpress_last_hip_error()
        super().__init__(msg)


def load():
    """Load the library (once).  Raises ImportError when it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libxpress_argmax.so is not built; run `python -m vocab_wide_add_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        ip = ctypes.POINTER(ctypes.c_int)
        lib.xpress_add_argmax_to_blk.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp]
        lib.xpress_add_argmax_to_blk.restype = i32
        lib.xpress_add_argmax_to_blk_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp]
        lib.xpress_add_argmax_to_blk_noalloc.restype = i32
        lib.xpress_topc_argmax_to_blk.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        lib.xpress_topc_argmax_to_blk.restype = i32
        lib.xpress_readout_gemm_argmax_to_blk.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64,
                                                          i64, vp]
        lib.xpress_readout_gemm_argmax_to_blk.restype = i32
        lib.xpress_latent_pass.argtypes = [vp] * 10 + [i64] * 5 + [vp]
        lib.xpress_latent_pass.restype = i32
        lib.xpress_latent_set_tiles.argtypes = [i32, i32, i32]
        lib.xpress_latent_set_tiles.restype = i32
        lib.xpress_latent_reserve.argtypes = [i64, i64, i64, i64, vp]
        lib.xpress_latent_reserve.restype = i32
        lib.xpress_reserve.argtypes = [i64, i64, i64, vp]
        lib.xpress_reserve.restype = i32
        lib.xpress_release.argtypes = []
        lib.xpress_release.restype = i32
        lib.xpress_set_workspace_limit.argtypes = [i64]
        lib.xpress_set_workspace_limit.restype = i32
        lib.xpress_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int64)]
        lib.xpress_workspace_bytes.restype = i32
        lib.xpress_set_plan.argtypes = [i32, i32, i32]
        lib.xpress_set_plan.restype = i32
        lib.xpress_set_reverse_order.argtypes = [i32]
        lib.xpress_set_reverse_order.restype = i32
        lib.xpress_describe_plan.argtypes = [vp, vp, i64, i64, i64, i64, i64,
                                             ip, ip, ip, ip, ip]
        lib.xpress_describe_plan.restype = i32
        lib.xpress_describe_gemm_plan.argtypes = [i64, i64, i64, ip, ip, ip, ip]
        lib.xpress_describe_gemm_plan.restype = i32
        lib.xpress_bf16_add_round_table.argtypes = [vp, i64, vp, vp]
        lib.xpress_bf16_add_round_table.restype = i32
        lib.xpress_read_probe.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp]
        lib.xpress_read_probe.restype = i32
        lib.xpress_last_hip_error.argtypes = []
        lib.xpress_last_hip_error.restype = i32
        lib.xpress_error_string.argtypes = [i32]
        lib.xpress_error_string.restype = ctypes.c_char_p
        lib.xpress_version.argtypes = []
        lib.xpress_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _ptr(x):
    """Device address of a torch tensor on a GPU, or an int address as is."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("expected a tensor on a GPU, got one on %s" % x.device)
        return x.data_ptr()
    raise TypeError("expected a GPU tensor or an integer address, got %r" % type(x))


def _span(t, nbytes: int, what: str):
    """Refuse a tensor whose storage ends before the ``nbytes`` the call
    will touch from its first element (integer addresses are the caller's
    responsibility, as in the C ABI)."""
    if nbytes <= 0 or t is None or isinstance(t, int) or not hasattr(t, "untyped_storage"):
        return
    avail = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if nbytes > avail:
        raise ValueError("%s: the call reads or writes %d bytes from the tensor's first "
                         "element, its storage holds %d" % (what, nbytes, avail))


def _stream(stream):
    """HIP stream handle: None means torch's current stream on the current device."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != XPRESS_OK:
        raise XpressError(status, where)


def xpress_add_argmax_to_blk(base, bias, blk, N: int, B: int, V: int,
                             stride_base_r: int, stride_bias_r: int, stream=None) -> None:
    """blk[n, 1+b] = argmax_v bf16(base[r, v] + bias[r, v]), r = n*(B-1) + b.

    Queued on ``stream`` (default: torch's current stream).  See the header
    for the layout rules and error behaviour.
    """
    rows = int(N) * (int(B) - 1)
    if rows > 0:
        _span(base, ((rows - 1) * int(stride_base_r) + int(V)) * 2, "base")
        _span(bias, ((rows - 1) * int(stride_bias_r) + int(V)) * 2, "bias")
        _span(blk, int(N) * int(B) * 8, "blk")
    lib = load()
    _check(lib.xpress_add_argmax_to_blk(_ptr(base), _ptr(bias), _ptr(blk), int(N), int(B),
                                        int(V), int(stride_base_r), int(stride_bias_r),
                                        _stream(stream)),
           "xpress_add_argmax_to_blk")


def bind_add_argmax_to_blk(base, bias, blk, N: int, B: int, V: int, stride_base_r: int,
                           stride_bias_r: int, stream=None):
    """xpress_add_argmax_to_blk with its arguments marshalled once: checks
    the tensors' spans and resolves pointers and the stream now, and returns
    a callable that queues the readout (the library validates the arguments
    again on every call and the callable raises on a nonzero status).  The
    tensors must stay alive and in place while the callable is used."""
    rows = int(N) * (int(B) - 1)
    if rows > 0:
        _span(base, ((rows - 1) * int(stride_base_r) + int(V)) * 2, "base")
        _span(bias, ((rows - 1) * int(stride_bias_r) + int(V)) * 2, "bias")
        _span(blk, int(N) * int(B) * 8, "blk")
    fn = load().xpress_add_argmax_to_blk
    args = (_ptr(base), _ptr(bias), _ptr(blk), int(N), int(B), int(V), int(stride_base_r),
            int(stride_bias_r), _stream(stream))

    def call():
        st = fn(*args)
        if st != XPRESS_OK:
            raise XpressError(st, "xpress_add_argmax_to_blk")
    return call


def xpress_add_argmax_to_blk_noalloc(base, bias, blk, N: int, B: int, V: int,
                                     stride_base_r: int, stride_bias_r: int, stream=None) -> None:
    """The same readout without any device allocation (a fixed key table
    built into the library, shared by every call on the GPU)."""
    rows = int(N) * (int(B) - 1)
    if rows > 0:
        _span(base, ((rows - 1) * int(stride_base_r) + int(V)) * 2, "base")
        _span(bias, ((rows - 1) * int(stride_bias_r) + int(V)) * 2, "bias")
        _span(blk, int(N) * int(B) * 8, "blk")
    lib = load()
    _check(lib.xpress_add_argmax_to_blk_noalloc(_ptr(base), _ptr(bias), _ptr(blk), int(N),
                                                int(B), int(V), int(stride_base_r),
                                                int(stride_bias_r), _stream(stream)),
           "xpress_add_argmax_to_blk_noalloc")


def xpress_topc_argmax_to_blk(base_c, bias_c, cand, blk, N: int, B: int, C: int,
                              stream=None) -> None:
    """blk[n, 1+j] = cand[r, argmax_c bf16(base_c[r, c] + bias_c[r, c])],
    r = n*(B-1) + j; base_c, bias_c, cand are [N, B-1, C] contiguous."""
    rows = int(N) * (int(B) - 1)
    if rows > 0:
        _span(base_c, rows * int(C) * 2, "base_c")
        _span(bias_c, rows * int(C) * 2, "bias_c")
        _span(cand, rows * int(C) * 8, "cand")
        _span(blk, int(N) * int(B) * 8, "blk")
    lib = load()
    _check(lib.xpress_topc_argmax_to_blk(_ptr(base_c), _ptr(bias_c), _ptr(cand), _ptr(blk),
                                         int(N), int(B), int(C), _stream(stream)),
           "xpress_topc_argmax_to_blk")


def xpress_readout_gemm_argmax_to_blk(base, x, w, blk, N: int, B: int, V: int, R: int,
                                      stride_base_r: int, stream=None) -> None:
    """blk[n, 1+b] = argmax_v bf16(base[r, v] + bf16(x[r] . w[v])), r = n*(B-1) + b;
    x is [rows, R], w is [V, R], all bf16 on the GPU."""
    rows = int(N) * (int(B) - 1)
    if rows > 0:
        _span(base, ((rows - 1) * int(stride_base_r) + int(V)) * 2, "base")
        _span(x, rows * int(R) * 2, "x")
        _span(w, int(V) * int(R) * 2, "w")
        _span(blk, int(N) * int(B) * 8, "blk")
    lib = load()
    _check(lib.xpress_readout_gemm_argmax_to_blk(_ptr(base), _ptr(x), _ptr(w), _ptr(blk),
                                                 int(N), int(B), int(V), int(R),
                                                 int(stride_base_r), _stream(stream)),
           "xpress_readout_gemm_argmax_to_blk")


def xpress_latent_pass(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, lat_out, N: int, B: int,
                       R: int, H: int, V: int, stream=None) -> None:
    """Latent stage of one pass: lat_out [N, B-1, R] from the block tokens
    blk [N, B], am1 [N] (int64), the hidden cache xh [N, B, R], the embedding
    w1 [V, R] and the out-major weights wlat [R, R], mixl [B, B, R],
    wg / wu [H, R], wd [R, H] (all bf16 on the GPU)."""
    n, b, r, h, v = int(N), int(B), int(R), int(H), int(V)
    if n > 0:
        for t, nb, what in ((blk, n * b * 8, "blk"), (am1, n * 8, "am1"),
                            (xh, n * b * r * 2, "xh"), (w1, v * r * 2, "w1"),
                            (wlat, r * r * 2, "wlat"), (mixl, b * b * r * 2, "mixl"),
                            (wg, h * r * 2, "wg"), (wu, h * r * 2, "wu"), (wd, r * h * 2, "wd"),
                            (lat_out, n * (b - 1) * r * 2, "lat_out")):
            _span(t, nb, what)
    lib = load()
    _check(lib.xpress_latent_pass(_ptr(blk), _ptr(am1), _ptr(xh), _ptr(w1), _ptr(wlat),
                                  _ptr(mixl), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(lat_out),
                                  int(N), int(B), int(R), int(H), int(V), _stream(stream)),
           "xpress_latent_pass")


def xpress_latent_reserve(N: int, B: int, R: int, H: int, stream=None) -> None:
    _check(load().xpress_latent_reserve(int(N), int(B), int(R), int(H), _stream(stream)),
           "xpress_latent_reserve")


def xpress_latent_set_tiles(mix: int = 0, gate: int = 0, down: int = 0) -> None:
    """Row-slab counts of the three latent kernels: 1, 2 or 4 (direct kernels),
    8 (LDS-staged kernels), 0 = automatic."""
    _check(load().xpress_latent_set_tiles(int(mix), int(gate), int(down)),
           "xpress_latent_set_tiles")


def xpress_reserve(N: int, B: int, V: int, stream=None) -> None:
    _check(load().xpress_reserve(int(N), int(B), int(V), _stream(stream)), "xpress_reserve")


def xpress_release() -> None:
    _check(load().xpress_release(), "xpress_release")


def xpress_set_workspace_limit(nbytes: int) -> None:
    """Cap on the library's workspace per device (0 = none); past it a call
    returns XPRESS_ENOMEM (raised as XpressError)."""
    _check(load().xpress_set_workspace_limit(int(nbytes)), "xpress_set_workspace_limit")


def xpress_workspace_bytes() -> int:
    """Bytes of workspace (live and retired) held on the current device."""
    out = ctypes.c_int64(0)
    _check(load().xpress_workspace_bytes(ctypes.byref(out)), "xpress_workspace_bytes")
    return int(out.value)


def xpress_set_plan(combine: int = XPRESS_COMBINE_AUTO, splits: int = 0,
                    block_threads: int = 0) -> None:
    _check(load().xpress_set_plan(int(combine), int(splits), int(block_threads)),
           "xpress_set_plan")


def xpress_set_reverse_order(reversed_: bool) -> None:
    """Debug: later launches visit their work units from last to first."""
    _check(load().xpress_set_reverse_order(1 if reversed_ else 0), "xpress_set_reverse_order")


def xpress_describe_plan(base, bias, N: int, B: int, V: int, stride_base_r: int,
                         stride_bias_r: int) -> dict:
    """The plan a call would use, from sizes and pointer alignment (host only)."""
    out = [ctypes.c_int(0) for _ in range(5)]
    _check(load().xpress_describe_plan(
        _ptr(base), _ptr(bias), int(N), int(B), int(V), int(stride_base_r),
        int(stride_bias_r), *[ctypes.byref(o) for o in out]), "xpress_describe_plan")
    combine, splits, threads, vec, launches = [o.value for o in out]
    return {"combine": COMBINE_NAMES.get(combine, combine), "splits": splits,
            "block_threads": threads, "vector_path": bool(vec), "launches": launches}


def xpress_describe_gemm_plan(N: int, B: int, V: int) -> dict:
    """Launch shape of the readout with in-place bias for (N, B, V): waves
    per workgroup, vocabulary ranges, workgroups per range and 32-id tiles."""
    out = [ctypes.c_int(0) for _ in range(4)]
    _check(load().xpress_describe_gemm_plan(int(N), int(B), int(V),
                                            *[ctypes.byref(o) for o in out]),
           "xpress_describe_gemm_plan")
    waves, ranges, row_wgs, tiles = [o.value for o in out]
    return {"waves": waves, "ranges": ranges, "row_wgs": row_wgs, "tiles": tiles}


def xpress_bf16_add_round_table(a_vals, n_a: int, out, stream=None) -> None:
    """out[i*65536 + b] = bf16(a_vals[i] + b) on the GPU, for every pattern b."""
    _span(a_vals, int(n_a) * 2, "a_vals")
    _span(out, int(n_a) * 65536 * 2, "out")
    _check(load().xpress_bf16_add_round_table(_ptr(a_vals), int(n_a), _ptr(out),
                                              _stream(stream)),
           "xpress_bf16_add_round_table")


XPRESS_READ_ROWS = 0
XPRESS_READ_FLAT = 1


def xpress_read_probe(base, bias, rows: int, V: int, stride: int, mode: int, sink,
                      stream=None) -> None:
    """Plain streaming read of base and bias (no arithmetic): the read
    ceiling the readout is measured against.  mode XPRESS_READ_ROWS (one
    workgroup per row) or XPRESS_READ_FLAT (grid-stride sweep)."""
    if int(rows) > 0:
        _span(base, ((int(rows) - 1) * int(stride) + int(V)) * 2, "base")
        _span(bias, ((int(rows) - 1) * int(stride) + int(V)) * 2, "bias")
        _span(sink, 4, "sink")
    _check(load().xpress_read_probe(_ptr(base), _ptr(bias), int(rows), int(V), int(stride),
                                    int(mode), _ptr(sink), _stream(stream)),
           "xpress_read_probe")


def xpress_last_hip_error() -> int:
    return int(load().xpress_last_hip_error())


def xpress_error_string(status: int) -> str:
    return load().xpress_error_string(int(status)).decode()


def xpress_version() -> str:
    return load().xpress_version().decode()
