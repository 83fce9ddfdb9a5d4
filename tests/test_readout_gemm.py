"""Parity of the HIP readout-with-matmul (xpress_readout_gemm_argmax_to_blk)
with the CPU oracle.

Dyadic inputs (x, w on the grid k/8): every fp32 partial sum of the dot
products is exact, so the GPU's bias equals the bf16 of the exact dot product
whatever the matrix cores' accumulation order, and blk must match the oracle
bit for bit.  N(0, 1) inputs: fp32 accumulation can move a bias across a bf16
rounding boundary; the bias is then off by one bf16 ulp and the sum by at
most two (one for the bias, one for the second rounding), so the GPU's winner
must score within two bf16 ulps of the true maximum under the oracle's exact
definition, and most rows must match exactly.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import say, to_dev, ORACLE_THREADS
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def gpu_gemm(base_d, x_d, w_d, blk0, N, B, V, R, S):
    import torch
    blk_d = to_dev(blk0)
    native.xpress_readout_gemm_argmax_to_blk(base_d, x_d, w_d, blk_d, N, B, V, R, S)
    torch.cuda.synchronize()
    return blk_d.cpu().numpy()


def sample_rows(rows, k=24):
    picks = {0, 1, 31, 32, 33, 63, 64, rows - 1, rows - 2, rows // 2}
    g = np.random.Generator(np.random.PCG64(rows))
    picks |= set(int(r) for r in g.integers(0, rows, size=k))
    return sorted(r for r in picks if 0 <= r < rows)


@pytest.mark.parametrize("name", ["gemm_tiny_n2_b4_v1000_r64", "gemm_small_n8_b8_v32000_r256"])
def test_gemm_small_workloads_every_row(name):
    w = workloads.GEMM_WORKLOADS[name]
    base, x, wt, blk0 = workloads.generate_gemm(w)
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(w.rows), w.V, w.R, w.V,
                                          threads=ORACLE_THREADS).reshape(w.N, w.B - 1)
    say("gemm %s" % name)
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, w.N, w.B, w.V, w.R, w.V)
    assert np.array_equal(got, want)


def test_gemm_full_size_dyadic_sampled_rows():
    w = workloads.GEMM_WORKLOADS["gemm_dyadic_n32_b16_v152064_r256"]
    base, x, wt, blk0 = workloads.generate_gemm(w)
    say("gemm full-size dyadic")
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, w.N, w.B, w.V, w.R, w.V)
    assert np.array_equal(got[:, 0], blk0[:, 0])
    flat = got[:, 1:].reshape(-1)
    assert ((flat >= 0) & (flat < w.V)).all()
    rows = sample_rows(w.rows)
    want = oracle.gemm_argmax_rows(base, x, wt, rows, w.V, w.R, w.V, threads=ORACLE_THREADS)
    assert np.array_equal(flat[rows], want)


def _score(base, x, wt, r, v, V, R):
    """bf16(base[r, v] + bf16(x[r] . w[v])) under the oracle's definition."""
    bias = oracle.dot_bf16(x[r], wt[v])
    return oracle.bf16_to_double(oracle.bf16_sum(int(base[r, v]), bias))


@pytest.mark.parametrize("name", ["gemm_normal_n32_b16_v152064_r256",
                                  "gemm_normal_n1_b16_v152064_r256"])
def test_gemm_full_size_normal_within_derived_bound(name):
    w = workloads.GEMM_WORKLOADS[name]
    base, x, wt, blk0 = workloads.generate_gemm(w)
    say("gemm full-size N(0,1) %s" % name)
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, w.N, w.B, w.V, w.R, w.V)
    flat = got[:, 1:].reshape(-1)
    assert ((flat >= 0) & (flat < w.V)).all()
    rows = sample_rows(w.rows, k=40)
    want = oracle.gemm_argmax_rows(base, x, wt, rows, w.V, w.R, w.V, threads=ORACLE_THREADS)
    exact = 0
    for r, vo in zip(rows, want):
        vg = int(flat[r])
        if vg == vo:
            exact += 1
            continue
        s_best = _score(base, x, wt, r, int(vo), w.V, w.R)
        s_gpu = _score(base, x, wt, r, vg, w.V, w.R)
        ulp = 2.0 ** (np.floor(np.log2(abs(s_best))) - 7) if s_best != 0 else 2.0 ** -133
        assert s_gpu >= s_best - 2 * ulp, (r, vg, vo, s_gpu, s_best)
    assert exact >= 0.9 * len(rows)


def _dyadic(rows, V, R, seed, pad=0):
    g = np.random.Generator(np.random.PCG64(seed))
    base = workloads.f32_to_bf16_bits(
        (g.integers(-16, 17, size=(rows, V)) / 4.0).astype(np.float32))
    if pad:
        b = np.full((rows, V + pad), 0x42C8, np.uint16)
        b[:, :V] = base
        base = b
    x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, R)) / 8.0).astype(np.float32))
    wt = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(V, R)) / 8.0).astype(np.float32))
    return base, x, wt


@pytest.mark.parametrize("R", [64, 128, 256])
@pytest.mark.parametrize("N,B,V", [(1, 2, 1), (1, 2, 63), (1, 33, 64), (3, 12, 65),
                                   (2, 17, 1000), (5, 21, 4097), (1, 2, 130),
                                   # the launch shape changes at 64 and 128 rows
                                   (4, 17, 3000), (5, 14, 2999), (8, 17, 1001), (3, 44, 777)])
def test_gemm_ragged_shapes(R, N, B, V):
    rows = N * (B - 1)
    pad = (-V) % 8 + (8 if V % 3 == 0 else 0)   # strides a multiple of 8, sometimes padded
    S = V + pad
    base, x, wt = _dyadic(rows, V, R, seed=V * 7 + R + rows, pad=pad)
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 3
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, S,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    say("gemm ragged N=%d B=%d V=%d R=%d" % (N, B, V, R))
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, N, B, V, R, S)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("N,B,V,R", [(37, 15, 1001, 64),    # 518 rows: 2 workgroups per range, 6 rows in the second
                                     (40, 16, 3000, 256),   # 600 rows
                                     (70, 16, 2000, 128)])  # 1050 rows: 3 workgroups per range
def test_gemm_several_workgroups_per_range(N, B, V, R):
    """Above 512 rows each vocabulary range is covered by several 512-row
    workgroups placed on one XCD; the last one is partly empty."""
    rows = N * (B - 1)
    pad = (-V) % 8
    S = V + pad
    base, x, wt = _dyadic(rows, V, R, seed=rows + V + R, pad=pad)
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 11
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, S,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    say("gemm several workgroups per range N=%d B=%d V=%d R=%d" % (N, B, V, R))
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, N, B, V, R, S)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("R", [64, 256])
def test_gemm_special_values(R):
    """Special base values against the oracle (dyadic x and w, so the bias is
    exact): all -inf rows (id 0 wins), all +inf rows and +inf ties (the
    lowest id), -0 next to +0 sums, subnormal sums, the largest finite bf16
    next to a positive bias (overflow to +inf), winners in the ragged last
    tile, and zero x rows (bias exactly +0)."""
    N, B, V = 4, 9, 1000               # 32 rows, a ragged last tile
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(4040 + R))
    base = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, V)) / 4.0).astype(np.float32))
    x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, R)) / 8.0).astype(np.float32))
    wt = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(V, R)) / 8.0).astype(np.float32))
    NEG_INF, POS_INF, NEG_ZERO, MAX_FIN = 0xFF80, 0x7F80, 0x8000, 0x7F7F
    base[0, :] = NEG_INF                          # all -inf
    base[1, :] = POS_INF                          # all +inf
    base[2, [500, 700]] = POS_INF                 # +inf tie
    x[3, :] = 0                                   # bias +0 everywhere
    base[3, :] = NEG_ZERO                         # -0 + +0 = +0 everywhere: id 0
    x[4, :] = 0
    base[4, :] = 0xBF80                           # -1.0 ...
    base[4, 999] = 0x0001                         # ... a subnormal at the last id
    base[4, 998] = 0x8001
    base[5, [10, 20]] = MAX_FIN                   # overflow with a positive bias
    base[6, 992:] = POS_INF                       # only the ragged tile holds +inf
    base[7, :] = NEG_INF
    base[7, 31] = 0                               # one finite value at a tile edge
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 5
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, V,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    w1 = want[:, 1:].reshape(-1)
    assert w1[0] == 0 and w1[1] == 0 and w1[2] == 500 and w1[3] == 0 and w1[4] == 999
    assert w1[6] == 992 and w1[7] == 31
    say("gemm special values R=%d" % R)
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, N, B, V, R, V)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("N,B,R", [(3, 8, 256),     # 21 rows: one wave per workgroup
                                   (10, 10, 64),    # 90 rows: two waves
                                   (8, 16, 256),    # 120 rows: two waves
                                   (20, 16, 256),   # 300 rows: eight waves
                                   (20, 16, 128),
                                   (20, 16, 64),
                                   (40, 16, 256)])  # 600 rows: two workgroups per range
def test_gemm_non_positive_maxima(N, B, R):
    """Rows whose maximum is not positive, beside rows whose maximum is, in
    every launch shape: all-negative rows full of ties, rows whose maximum
    is +0 reached from -0 and +0 base values, -inf rows, and rows negative
    over the first part of the vocabulary only (so that some vocabulary
    ranges of a row have a positive maximum and others not).  Dyadic inputs,
    so the bias is exact and the oracle's result is the only correct one."""
    V = 3000                                   # a ragged last tile
    rows = N * (B - 1)
    base, x, wt = _dyadic(rows, V, R, seed=7000 + rows + R)
    g = np.random.Generator(np.random.PCG64(7100 + rows + R))
    NEG_INF, NEG_ZERO = 0xFF80, 0x8000
    kinds = []
    for r in range(rows):
        k = r % 5
        kinds.append(k)
        if k == 1:       # all negative, many ties at the top value
            x[r, :] = 0
            base[r, :] = workloads.f32_to_bf16_bits(
                (-g.integers(1, 5, size=V) / 4.0).astype(np.float32))
        elif k == 2:     # maximum +0, from -0 and +0 base values
            x[r, :] = 0
            base[r, :] = workloads.f32_to_bf16_bits(np.full(V, -0.5, np.float32))
            zpos = g.choice(V, size=6, replace=False)
            base[r, zpos[:3]] = NEG_ZERO
            base[r, zpos[3:]] = 0
        elif k == 3:     # -inf everywhere but one negative value
            base[r, :] = NEG_INF
            base[r, g.integers(0, V)] = workloads.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
        elif k == 4:     # negative over the first part, positive after
            cut = int(g.integers(V // 4, 3 * V // 4))
            x[r, :] = 0
            base[r, :cut] = workloads.f32_to_bf16_bits(np.full(cut, -1.0, np.float32))
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 3
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, V,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    say("gemm non-positive maxima N=%d B=%d R=%d" % (N, B, R))
    got = gpu_gemm(to_dev(base), to_dev(x), to_dev(wt), blk0, N, B, V, R, V)
    assert np.array_equal(got, want), [
        (r, kinds[r], got[:, 1:].reshape(-1)[r], want[:, 1:].reshape(-1)[r])
        for r in range(rows) if got[:, 1:].reshape(-1)[r] != want[:, 1:].reshape(-1)[r]][:8]


def test_gemm_repeated_calls_and_guard_cells():
    import torch
    N, B, V, R = 4, 16, 20000, 128
    rows = N * (B - 1)
    guard = 0x7E7E7E7E7E7E7E7E
    for seed in range(3):
        base, x, wt = _dyadic(rows, V, R, seed=100 + seed)
        blk0 = np.full((N, B), -1, dtype=np.int64)
        blk0[:, 0] = 9
        want = blk0.copy()
        want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, V,
                                              threads=ORACLE_THREADS).reshape(N, B - 1)
        buf = np.full(N * B + 64, guard, dtype=np.int64)
        buf[32:32 + N * B] = blk0.reshape(-1)
        buf_d = to_dev(buf)
        say("gemm guard cells seed=%d" % seed)
        native.xpress_readout_gemm_argmax_to_blk(to_dev(base), to_dev(x), to_dev(wt),
                                                 buf_d.data_ptr() + 32 * 8, N, B, V, R, V)
        torch.cuda.synchronize()
        out = buf_d.cpu().numpy()
        assert (out[:32] == guard).all() and (out[32 + N * B:] == guard).all()
        assert np.array_equal(out[32:32 + N * B].reshape(N, B), want)


def test_gemm_invalid_arguments_raise():
    import torch
    b = torch.zeros(4096, dtype=torch.int16, device="cuda")
    blk = torch.zeros(64, dtype=torch.int64, device="cuda")
    with pytest.raises(native.XpressError):   # R unsupported
        native.xpress_readout_gemm_argmax_to_blk(b, b, b, blk, 1, 2, 8, 96, 8)
    with pytest.raises(native.XpressError):   # misaligned x
        native.xpress_readout_gemm_argmax_to_blk(b, b.data_ptr() + 2, b, blk, 1, 2, 8, 64, 8)


@pytest.mark.parametrize("N,B,V,R", [(2, 8, 5000, 128),     # 14 rows: one wave per workgroup
                                     (12, 11, 3000, 64),    # 120 rows: two waves
                                     (10, 17, 2000, 256)])  # 160 rows: eight waves
def test_gemm_graph_replay_matches_eager(N, B, V, R):
    """One call outside capture sizes the (device, stream) workspace; the call
    captured into a HIP graph then replays on fresh inputs copied in between,
    each replay checked against an eager call and the oracle."""
    import torch
    rows = N * (B - 1)
    cases = [_dyadic(rows, V, R, seed=700 + k) for k in range(3)]
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 5
    base_d, x_d, w_d = (to_dev(a) for a in cases[0])
    blk_d = to_dev(blk0)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    native.xpress_readout_gemm_argmax_to_blk(base_d, x_d, w_d, blk_d, N, B, V, R, V, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("gemm graph capture N=%d B=%d V=%d R=%d" % (N, B, V, R))
    with torch.cuda.graph(g, stream=s):
        native.xpress_readout_gemm_argmax_to_blk(base_d, x_d, w_d, blk_d, N, B, V, R, V, stream=s)
    for rep in range(6):
        base, x, wt = cases[rep % 3]
        base_d.copy_(to_dev(base))
        x_d.copy_(to_dev(x))
        w_d.copy_(to_dev(wt))
        blk_d.copy_(to_dev(blk0))
        torch.cuda.synchronize()
        say("gemm graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = blk_d.cpu().numpy()
        eager = gpu_gemm(base_d, x_d, w_d, blk0, N, B, V, R, V)
        assert np.array_equal(got, eager), rep
        want = blk0.copy()
        want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, V,
                                              threads=ORACLE_THREADS).reshape(N, B - 1)
        assert np.array_equal(got, want), rep


def test_gemm_two_streams_at_once():
    """Calls on two streams at once each use their own (device, stream) key
    table: both results must match the oracle."""
    import torch
    cases = []
    for k, (N, B, V, R) in enumerate([(6, 16, 4000, 128), (9, 16, 3000, 128)]):
        rows = N * (B - 1)
        base, x, wt = _dyadic(rows, V, R, seed=900 + k)
        blk0 = np.full((N, B), -1, dtype=np.int64)
        blk0[:, 0] = k
        want = blk0.copy()
        want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, V,
                                              threads=ORACLE_THREADS).reshape(N, B - 1)
        cases.append((N, B, V, R, to_dev(base), to_dev(x), to_dev(wt), to_dev(blk0), want))
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say("gemm two streams")
    for _ in range(5):
        for (N, B, V, R, bd, xd, wd, blk, _), st in zip(cases, s):
            native.xpress_readout_gemm_argmax_to_blk(bd, xd, wd, blk, N, B, V, R, V, stream=st)
    torch.cuda.synchronize()
    for (N, B, V, R, bd, xd, wd, blk, want) in cases:
        assert np.array_equal(blk.cpu().numpy(), want)
