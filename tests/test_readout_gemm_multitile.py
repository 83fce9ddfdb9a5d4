"""Parity of the readout with in-place bias on the pipelined tile loop,
every row, bit for bit.

The kernel's steady loop (copies two or three tiles ahead, fixed wait
counts) runs only on vocabulary ranges of at least three 32-id tiles, and
the exact rerun that follows a tagged-maximum pass replays the whole range.
These tests pick shapes whose ranges hold several tiles in each launch shape
(one, two and eight waves per workgroup), including a ragged last tile, and
compare every row against the oracle on dyadic inputs (x and w on the grid
k/8, so every fp32 partial sum is exact and the bias is the bf16 of the exact
dot product whatever the accumulation order).  Rows whose maximum is not
positive force the rerun after a multi-tile pass.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import say, to_dev, ORACLE_THREADS
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# (N, B, V): 300 rows (eight waves, one workgroup per range), 100 rows (two
# waves), 30 rows (one wave).  V is not a multiple of 32: a ragged last tile.
MULTI_TILE = [(20, 16, 32003), (10, 11, 100003), (2, 16, 100003)]


def _dyadic(rows, V, R, seed, pad):
    g = np.random.Generator(np.random.PCG64(seed))
    base = np.full((rows, V + pad), 0x42C8, np.uint16)      # +100 padding
    base[:, :V] = workloads.f32_to_bf16_bits(
        (g.integers(-16, 17, size=(rows, V)) / 4.0).astype(np.float32))
    x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, R)) / 8.0).astype(np.float32))
    wt = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(V, R)) / 8.0).astype(np.float32))
    return base, x, wt


def _run(base, x, wt, N, B, V, R, S, anchor):
    import torch
    rows = N * (B - 1)
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = anchor
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, S,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    blk_d = to_dev(blk0)
    native.xpress_readout_gemm_argmax_to_blk(to_dev(base), to_dev(x), to_dev(wt), blk_d,
                                             N, B, V, R, S)
    torch.cuda.synchronize()
    return blk_d.cpu().numpy(), want


def _mismatches(got, want, kinds=None, k=8):
    g, w = got[:, 1:].reshape(-1), want[:, 1:].reshape(-1)
    bad = np.nonzero(g != w)[0][:k]
    return [(int(r), None if kinds is None else kinds[r], int(g[r]), int(w[r])) for r in bad]


def _tiles_per_range(N, B, V):
    p = native.xpress_describe_gemm_plan(N, B, V)
    return p["tiles"] / p["ranges"], p


@pytest.mark.parametrize("R", [64, 128, 256])
@pytest.mark.parametrize("N,B,V", MULTI_TILE)
def test_gemm_multitile_every_row(N, B, V, R):
    rows = N * (B - 1)
    tpr, plan = _tiles_per_range(N, B, V)
    assert tpr >= 3.0, plan
    pad = (-V) % 8 + 8
    S = V + pad
    base, x, wt = _dyadic(rows, V, R, seed=rows * 31 + V + R, pad=pad)
    say("gemm multi-tile N=%d B=%d V=%d R=%d plan=%s" % (N, B, V, R, plan))
    got, want = _run(base, x, wt, N, B, V, R, S, anchor=7)
    assert np.array_equal(got, want), _mismatches(got, want)


@pytest.mark.parametrize("R", [64, 128, 256])
@pytest.mark.parametrize("N,B,V", MULTI_TILE)
def test_gemm_multitile_non_positive_maxima(N, B, V, R):
    """The five row kinds of the short-range test (positive; all negative
    with ties; maximum +0 from -0 and +0 base values; -inf but one; negative
    over the first part only) at several tiles per range, so that the exact
    rerun replays a pipelined multi-tile range."""
    rows = N * (B - 1)
    tpr, plan = _tiles_per_range(N, B, V)
    assert tpr >= 3.0, plan
    pad = (-V) % 8
    S = V + pad
    base, x, wt = _dyadic(rows, V, R, seed=9000 + rows + R, pad=pad)
    g = np.random.Generator(np.random.PCG64(9100 + rows + R))
    NEG_INF, NEG_ZERO = 0xFF80, 0x8000
    kinds = []
    for r in range(rows):
        k = r % 5
        kinds.append(k)
        if k == 1:       # all negative, many ties at the top value
            x[r, :] = 0
            base[r, :V] = workloads.f32_to_bf16_bits(
                (-g.integers(1, 5, size=V) / 4.0).astype(np.float32))
        elif k == 2:     # maximum +0, from -0 and +0 base values
            x[r, :] = 0
            base[r, :V] = workloads.f32_to_bf16_bits(np.full(V, -0.5, np.float32))
            zpos = g.choice(V, size=6, replace=False)
            base[r, zpos[:3]] = NEG_ZERO
            base[r, zpos[3:]] = 0
        elif k == 3:     # -inf everywhere but one negative value
            base[r, :V] = NEG_INF
            base[r, g.integers(0, V)] = workloads.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
        elif k == 4:     # negative over the first part, positive after
            cut = int(g.integers(V // 4, 3 * V // 4))
            x[r, :] = 0
            base[r, :cut] = workloads.f32_to_bf16_bits(np.full(cut, -1.0, np.float32))
    say("gemm multi-tile non-positive maxima N=%d B=%d V=%d R=%d" % (N, B, V, R))
    got, want = _run(base, x, wt, N, B, V, R, S, anchor=3)
    assert np.array_equal(got, want), _mismatches(got, want, kinds)


def test_gemm_full_size_dyadic_every_row():
    """All 480 rows of the pages' shape (152064 ids, R = 256) on dyadic
    inputs: every fp32 sum exact, so every row must match the oracle."""
    w = workloads.GEMM_WORKLOADS["gemm_dyadic_n32_b16_v152064_r256"]
    base, x, wt, blk0 = workloads.generate_gemm(w)
    say("gemm full-size dyadic, every row")
    import torch
    blk_d = to_dev(blk0)
    native.xpress_readout_gemm_argmax_to_blk(to_dev(base), to_dev(x), to_dev(wt), blk_d,
                                             w.N, w.B, w.V, w.R, w.V)
    torch.cuda.synchronize()
    got = blk_d.cpu().numpy()
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(w.rows), w.V, w.R, w.V,
                                          threads=ORACLE_THREADS).reshape(w.N, w.B - 1)
    assert np.array_equal(got, want), _mismatches(got, want)


@pytest.mark.parametrize("N,B,V,R", [(3, 8, 5000, 256),     # 21 rows: one wave
                                     (8, 16, 5000, 128),    # 120 rows: two waves
                                     (20, 16, 5003, 64)])   # 300 rows: eight waves
def test_gemm_nan_sums_never_win(N, B, V, R):
    """NaN sums are outside the contract; the reading taken is that a NaN
    never wins, as in the oracle.  Rows: x = +inf in channel 0 with the rest
    0, so bias[v] is +inf, -inf or NaN as w[v, 0] is positive, negative or 0
    (inf * 0); base = +inf where the bias is -inf (+inf + -inf is NaN), so
    early ids hold NaN sums with a larger bit pattern than +inf; a row with a
    NaN x channel (every sum NaN: index 0); rows beside them are ordinary."""
    rows = N * (B - 1)
    base, x, wt = _dyadic(rows, V, R, seed=4400 + rows, pad=(-V) % 8)
    S = base.shape[1]
    POS_INF, NAN = 0x7F80, 0x7FC0
    w0 = (wt[:, 0].astype(np.uint32) << 16).view(np.float32)
    for r in range(rows):
        k = r % 3
        if k == 1:
            x[r, :] = 0
            x[r, 0] = POS_INF
            base[r, :V][w0 < 0] = POS_INF
        elif k == 2 and r % 6 == 5:
            x[r, 0] = NAN
    say("gemm NaN sums N=%d B=%d V=%d R=%d" % (N, B, V, R))
    got, want = _run(base, x, wt, N, B, V, R, S, anchor=1)
    assert np.array_equal(got, want), _mismatches(got, want)


@pytest.mark.parametrize("N,B,V,R", [(20, 16, 32003, 256),    # 300 rows: eight waves
                                     (10, 11, 100003, 128)])  # 100 rows: two waves
def test_gemm_negative_rows_with_a_late_nan(N, B, V, R):
    """Rows whose sums are all negative (so their workgroups take the
    order-preserving mode after the first tile) holding one NaN base value
    at an id outside the first tile of its vocabulary range.  A NaN with the
    sign clear maps above every value there, so the check after the range
    must send the workgroup through the exact pass; one with the sign set
    maps below -inf and simply never wins.  Every row against the oracle
    (where a NaN sum never wins)."""
    rows = N * (B - 1)
    tpr, plan = _tiles_per_range(N, B, V)
    assert tpr >= 3.0, plan
    pad = (-V) % 8
    S = V + pad
    base, x, wt = _dyadic(rows, V, R, seed=9700 + rows + R, pad=pad)
    g = np.random.Generator(np.random.PCG64(9800 + rows + R))
    tiles, ranges = plan["tiles"], plan["ranges"]
    first_tiles = {r * tiles // ranges for r in range(ranges)}
    later_ids = np.array([v for v in range(V) if v // 32 not in first_tiles])
    eighth = workloads.f32_to_bf16_bits(np.array([0.125], np.float32))[0]
    for r in range(rows):
        x[r, :] = 0
        x[r, 0] = eighth                      # bias = w[v, 0] / 8, |bias| <= 1/8
        base[r, :V] = workloads.f32_to_bf16_bits(
            (-g.integers(8, 18, size=V) / 4.0).astype(np.float32))    # -2 .. -4.25
        if r % 3 == 0:
            base[r, int(g.choice(later_ids))] = 0x7FC0       # NaN, sign clear
        elif r % 3 == 1:
            base[r, int(g.choice(later_ids))] = 0xFFC0       # NaN, sign set
    say("gemm negative rows with a late NaN N=%d B=%d V=%d R=%d" % (N, B, V, R))
    got, want = _run(base, x, wt, N, B, V, R, S, anchor=2)
    assert np.array_equal(got, want), _mismatches(got, want)
