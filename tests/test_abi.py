"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and its host-only calls (plan description, plan override,
error strings, argument validation ahead of any launch) behave as documented.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

from conftest import gpu_available
from vocab_wide_add_amd import native

# The argument-validation tests below pass made-up addresses that must be
# rejected before any launch.  They only run where there is no GPU, so a
# mistake in a test tuple can never put a kernel on a device with bad
# pointers; the GPU suite checks the same errors with real buffers.
no_gpu_only = pytest.mark.skipif(gpu_available(), reason="fake-pointer checks run without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xpress_argmax.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xpress_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = native.load()
    names = declared_functions()
    assert "xpress_add_argmax_to_blk" in names and len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    # the binding keeps the same names
    for name in names:
        assert callable(getattr(native, name)), name


def test_version_and_strings():
    assert native.xpress_version() == "0.1.0"
    for s in range(6):
        assert native.xpress_error_string(s) != "unknown status"
    assert native.xpress_error_string(99) == "unknown status"


def test_plan_for_the_pages_shape():
    # measured default: one 256-thread workgroup per row at 480 rows
    p = native.xpress_describe_plan(256, 256, 32, 16, 152064, 152064, 152064)
    assert p["vector_path"] and p["launches"] == 1
    assert (p["combine"], p["splits"], p["block_threads"]) == ("single", 1, 256)
    # 1024 threads per row from 1024 rows on
    p = native.xpress_describe_plan(256, 256, 256, 16, 152064, 152064, 152064)
    assert (p["combine"], p["block_threads"]) == ("single", 1024)
    # a few very wide rows are split and combined in a second pass
    p = native.xpress_describe_plan(256, 256, 1, 9, 152064, 152064, 152064)
    assert (p["combine"], p["launches"]) == ("two_pass", 2) and p["splits"] >= 2
    # short rows get a smaller workgroup
    p = native.xpress_describe_plan(256, 256, 2, 4, 1000, 1000, 1000)
    assert p["block_threads"] == 64
    p = native.xpress_describe_plan(258, 256, 32, 16, 152064, 152064, 152064)
    assert not p["vector_path"]
    p = native.xpress_describe_plan(256, 256, 32, 16, 152064, 152065, 152064)
    assert not p["vector_path"]
    p = native.xpress_describe_plan(256, 256, 0, 16, 152064, 152064, 152064)
    assert p["launches"] == 0


def test_plan_override_round_trip():
    try:
        native.xpress_set_plan(native.XPRESS_COMBINE_TWO_PASS, 5, 512)
        p = native.xpress_describe_plan(256, 256, 2, 4, 100000, 100000, 100000)
        assert (p["combine"], p["splits"], p["block_threads"], p["launches"]) == (
            "two_pass", 5, 512, 2)
        native.xpress_set_plan(native.XPRESS_COMBINE_SINGLE, 5, 64)
        p = native.xpress_describe_plan(256, 256, 2, 4, 100000, 100000, 100000)
        assert (p["combine"], p["splits"]) == ("single", 1)
        with pytest.raises(native.XpressError):
            native.xpress_set_plan(7, 0, 0)
        with pytest.raises(native.XpressError):
            native.xpress_set_plan(0, 0, 100)
    finally:
        native.xpress_set_plan(0, 0, 0)


@pytest.mark.parametrize("args", [
    (256, 256, 512, -1, 2, 8, 8, 8),       # N < 0
    (256, 256, 512, 1, 0, 8, 8, 8),        # B < 1
    (256, 256, 512, 1, 2, 0, 8, 8),        # V < 1
    (256, 256, 512, 1, 2, 8, 7, 8),        # stride_base < V
    (256, 256, 512, 1, 2, 8, 8, 7),        # stride_bias < V
    (0, 256, 512, 1, 2, 8, 8, 8),          # null base with rows
    (256, 0, 512, 1, 2, 8, 8, 8),          # null bias with rows
    (256, 256, 0, 1, 2, 8, 8, 8),          # null blk with rows
    (256, 4096, 260, 1, 2, 8, 8, 8),       # blk overlaps base
    (4096, 256, 268, 1, 2, 8, 8, 8),       # blk overlaps bias
    (256, 256, 512, 1, 2, 2 ** 31, 2 ** 31, 2 ** 31),  # V too large
])
@no_gpu_only
def test_invalid_arguments_rejected_before_launch(args):
    # validation happens before any HIP call, so this runs without a GPU
    lib = native.load()
    assert lib.xpress_add_argmax_to_blk(*args, None) == native.XPRESS_EINVAL


@no_gpu_only
def test_no_rows_is_ok_without_pointers():
    lib = native.load()
    assert lib.xpress_add_argmax_to_blk(0, 0, 0, 0, 16, 152064, 152064, 152064, None) == 0
    assert lib.xpress_add_argmax_to_blk(0, 0, 0, 32, 1, 152064, 152064, 152064, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(native, "_lib", None)
    monkeypatch.setattr(native, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        native.load()


@pytest.mark.parametrize("args", [
    (256, 256, 0, 4096, 1, 2, 8),          # null cand with rows
    (256, 256, 1024, 1040, 1, 2, 8),       # blk [1040, 1056) overlaps cand [1024, 1088)
    (256, 256, 1024, 4096, 1, 2, 0),       # C < 1
    (256, 256, 1024, 4096, -1, 2, 8),      # N < 0
    (0, 256, 1024, 4096, 1, 2, 8),         # null base_c
])
@no_gpu_only
def test_topc_invalid_arguments_rejected_before_launch(args):
    lib = native.load()
    assert lib.xpress_topc_argmax_to_blk(*args, None) == native.XPRESS_EINVAL


@no_gpu_only
def test_topc_no_rows_is_ok_without_pointers():
    lib = native.load()
    assert lib.xpress_topc_argmax_to_blk(0, 0, 0, 0, 0, 16, 256, None) == 0
    assert lib.xpress_topc_argmax_to_blk(0, 0, 0, 0, 32, 1, 256, None) == 0


@no_gpu_only
@pytest.mark.parametrize("args", [
    (256, 512, 1024, 4096, 1, 2, 8, 96, 8),     # R not 64/128/256
    (258, 512, 1024, 4096, 1, 2, 8, 64, 8),     # base not 16-byte aligned
    (256, 520, 1024, 4096, 1, 2, 8, 64, 8),     # x not 16-byte aligned
    (256, 512, 1032, 4096, 1, 2, 8, 64, 8),     # w not 16-byte aligned
    (256, 512, 1024, 4096, 1, 2, 8, 64, 12),    # stride not a multiple of 8
    (256, 512, 1024, 4096, 1, 2, 8, 64, 4),     # stride < V
    (256, 512, 1024, 520, 1, 2, 8, 64, 8),      # blk [520, 536) overlaps x [512, 640)
    (0, 512, 1024, 4096, 1, 2, 8, 64, 8),       # null base
    (256, 512, 0, 4096, 1, 2, 8, 64, 8),        # null w
    (256, 512, 1024, 4096, -1, 2, 8, 64, 8),    # N < 0
    (256, 512, 1024, 4096, 1, 0, 8, 64, 8),     # B < 1
    (256, 512, 1024, 4096, 1, 2, 0, 64, 8),     # V < 1
    (256, 512, 1024, 256, 1, 2, 8, 64, 8),      # blk on base
])
def test_gemm_invalid_arguments_rejected_before_launch(args):
    lib = native.load()
    assert lib.xpress_readout_gemm_argmax_to_blk(*args, None) == native.XPRESS_EINVAL


@no_gpu_only
def test_gemm_no_rows_is_ok_without_pointers():
    lib = native.load()
    assert lib.xpress_readout_gemm_argmax_to_blk(0, 0, 0, 0, 0, 16, 152064, 256, 152064,
                                                 None) == 0
    assert lib.xpress_readout_gemm_argmax_to_blk(0, 0, 0, 0, 32, 1, 152064, 256, 152064,
                                                 None) == 0


# latent pass: blk, am1, xh, w1, wlat, mixl, wg, wu, wd, lat_out, N, B, R, H, V
_LAT_PTRS = [0x10000, 0x20000, 0x30000, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000,
             0x600000, 0x700000]


def _lat(ptr_changes=None, **sizes):
    ptrs = list(_LAT_PTRS)
    for i, p in (ptr_changes or {}).items():
        ptrs[i] = p
    dims = dict(N=1, B=4, R=64, H=64, V=8)
    dims.update(sizes)
    return tuple(ptrs) + (dims["N"], dims["B"], dims["R"], dims["H"], dims["V"])


@no_gpu_only
@pytest.mark.parametrize("args", [
    _lat(N=-1), _lat(B=1), _lat(B=33), _lat(R=96), _lat(R=32), _lat(R=2048),
    _lat(H=96), _lat(H=16384), _lat(V=0), _lat(N=2 ** 30, B=4),
    _lat({2: 0}),                 # null xh
    _lat({0: 0}),                 # null blk
    _lat({9: 0}),                 # null lat_out
    _lat({3: 0x100008}),          # w1 not 16-byte aligned
    _lat({6: 0x400004}),          # wg not 16-byte aligned
    _lat({1: 0x20004}),           # am1 not 8-byte aligned
    _lat({9: 0x30000}),           # lat_out overlaps xh
    _lat({9: 0x100200}),          # lat_out inside w1 (1 KiB at 0x100000)
    _lat({9: 0x0FFFE}),           # lat_out runs into blk
])
def test_latent_invalid_arguments_rejected_before_launch(args):
    lib = native.load()
    assert lib.xpress_latent_pass(*args, None) == native.XPRESS_EINVAL


@no_gpu_only
def test_latent_no_blocks_is_ok_without_pointers():
    lib = native.load()
    assert lib.xpress_latent_pass(*([0] * 10), 0, 16, 256, 512, 152064, None) == 0
    assert lib.xpress_latent_reserve(0, 16, 256, 512, None) == 0
    assert lib.xpress_latent_reserve(1, 16, 96, 512, None) == native.XPRESS_EINVAL


def test_latent_tile_override_validates():
    try:
        native.xpress_latent_set_tiles(1, 2, 4)
        native.xpress_latent_set_tiles(8, 8, 8)
        native.xpress_latent_set_tiles(0, 0, 0)
        with pytest.raises(native.XpressError):
            native.xpress_latent_set_tiles(3, 0, 0)
        with pytest.raises(native.XpressError):
            native.xpress_latent_set_tiles(0, 16, 0)
    finally:
        native.xpress_latent_set_tiles(0, 0, 0)


def test_binding_refuses_tensors_shorter_than_the_call():
    """A tensor whose storage ends before the bytes a call touches is refused
    before the library is called (a kernel would read past it)."""
    import torch
    t = torch.zeros(10, dtype=torch.int16)
    native._span(t, 20, "t")
    with pytest.raises(ValueError, match="storage holds 20"):
        native._span(t, 22, "t")
    v = t[4:]                      # 12 bytes from its first element
    native._span(v, 12, "v")
    with pytest.raises(ValueError, match="storage holds 12"):
        native._span(v, 14, "v")
    base = torch.zeros(2 * 100, dtype=torch.int16)
    blk = torch.zeros(2 * 3, dtype=torch.int64)
    with pytest.raises(ValueError, match="base"):
        # 4 rows of 100 need 800 bytes, base holds 400
        native.xpress_add_argmax_to_blk(base, base, blk, 2, 3, 100, 100, 100)
    with pytest.raises(ValueError, match="lat_out"):
        small = torch.zeros(8, dtype=torch.int16)
        big = torch.zeros(1 << 20, dtype=torch.int16)
        ids = torch.zeros(64, dtype=torch.int64)
        native.xpress_latent_pass(ids, ids, big, big, big, big, big, big, big, small,
                                  2, 4, 64, 64, 10)

