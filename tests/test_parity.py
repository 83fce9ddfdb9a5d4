"""Parity of the HIP readout with the CPU oracle, through the C-ABI.

blk must match the oracle bit for bit (integer output), with the anchor slot
and every byte outside blk[:, 1:] untouched.  Covered: the five synthetic
workloads at full size in the default plan (the one the benchmark times),
every combine / block size / split count on the smaller ones, the unaligned
scalar path, ragged and degenerate shapes, ties across workgroup
boundaries, special values, repeated calls, graph replay and two streams.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Plan, gpu_blk, oracle_blk, say, to_dev
from conftest import gpu_available
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

COMBINES = [native.XPRESS_COMBINE_SINGLE, native.XPRESS_COMBINE_ATOMIC,
            native.XPRESS_COMBINE_TWO_PASS, native.XPRESS_COMBINE_BALANCED]

_cache = {}


def workload_case(name, rows_limit=None):
    """Host buffers, device copies and the oracle's blk for one workload."""
    key = (name, rows_limit)
    if key not in _cache:
        w = workloads.WORKLOADS[name]
        base, bias, blk0 = workloads.generate(w, rows_limit=rows_limit)
        N = w.N if rows_limit is None else rows_limit // (w.B - 1)
        blk0 = blk0[:N].copy()
        want = oracle_blk(base, bias, blk0, N, w.B, w.V, w.stride_base, w.stride_bias)
        _cache[key] = (w, N, base, bias, blk0, to_dev(base), to_dev(bias), want)
    return _cache[key]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_default_plan(name):
    w, N, base, bias, blk0, base_d, bias_d, want = workload_case(name)
    say("%s default plan %s" % (name, native.xpress_describe_plan(
        base_d, bias_d, N, w.B, w.V, w.stride_base, w.stride_bias)))
    got = gpu_blk(base_d, bias_d, blk0, N, w.B, w.V, w.stride_base, w.stride_bias)
    assert np.array_equal(got[:, 0], blk0[:, 0]), "anchor slot changed"
    assert (got[:, 1:] >= 0).all() and (got[:, 1:] < w.V).all()
    mism = np.argwhere(got != want)
    assert mism.size == 0, "first mismatches %s" % mism[:5].tolist()


@pytest.mark.parametrize("name", ["tiny_n2_b4_v1000", "small_n8_b8_v32000",
                                  "ties_strided_n32_b16_v151936"])
@pytest.mark.parametrize("combine", COMBINES)
@pytest.mark.parametrize("threads,splits", [(64, 0), (256, 0), (1024, 0), (256, 1),
                                            (256, 3), (128, 37), (512, 200)])
def test_every_plan(name, combine, threads, splits):
    w, N, base, bias, blk0, base_d, bias_d, want = workload_case(name)
    say("%s combine=%d threads=%d splits=%d" % (name, combine, threads, splits))
    with Plan(combine, splits, threads):
        got = gpu_blk(base_d, bias_d, blk0, N, w.B, w.V, w.stride_base, w.stride_bias)
    assert np.array_equal(got, want)


def _random_rows(N, B, V, seed, pad=0, kind="normal"):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = N * (B - 1)
    if kind == "normal":
        x = g.standard_normal((rows, V), dtype=np.float32) * np.float32(3.0)
        y = g.standard_normal((rows, V), dtype=np.float32)
    else:  # small integers: many exact ties
        x = g.integers(-2, 3, size=(rows, V)).astype(np.float32)
        y = g.integers(-2, 3, size=(rows, V)).astype(np.float32)
    base = np.full((rows, V + pad), 0x42C8, dtype=np.uint16)
    bias = np.full((rows, V + pad), 0x42C8, dtype=np.uint16)
    base[:, :V] = workloads.f32_to_bf16_bits(x)
    bias[:, :V] = workloads.f32_to_bf16_bits(y)
    blk = np.full((N, B), -1, dtype=np.int64)
    blk[:, 0] = g.integers(0, V, size=N)
    return base, bias, blk


@pytest.mark.parametrize("V", [1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 511, 513, 2047,
                               2048, 2049, 4095, 4096, 4097, 8191, 65537])
@pytest.mark.parametrize("combine", COMBINES)
def test_ragged_vocab(V, combine):
    N, B = 3, 5
    base, bias, blk0 = _random_rows(N, B, V, seed=V, kind="ties" if V % 2 else "normal")
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    base_d, bias_d = to_dev(base), to_dev(bias)
    say("ragged V=%d combine=%d" % (V, combine))
    for splits in (0, 2, 9):
        with Plan(combine, splits, 64 if V < 100 else 256):
            got = gpu_blk(base_d, bias_d, blk0, N, B, V, V, V)
        assert np.array_equal(got, want), (V, combine, splits)


@pytest.mark.parametrize("offset_base,offset_bias,pad", [(1, 0, 0), (0, 3, 0), (1, 1, 1),
                                                         (0, 0, 5), (2, 6, 3)])
@pytest.mark.parametrize("combine", COMBINES)
def test_unaligned_layouts_take_the_scalar_path(offset_base, offset_bias, pad, combine):
    N, B, V = 4, 4, 3001
    base, bias, blk0 = _random_rows(N, B, V, seed=17, pad=pad, kind="ties")
    want = oracle_blk(base, bias, blk0, N, B, V, V + pad, V + pad)
    big_b = np.zeros(base.size + 16, np.uint16)
    big_i = np.zeros(bias.size + 16, np.uint16)
    big_b[offset_base:offset_base + base.size] = base.reshape(-1)
    big_i[offset_bias:offset_bias + bias.size] = bias.reshape(-1)
    bd, id_ = to_dev(big_b), to_dev(big_i)
    pb = bd.data_ptr() + 2 * offset_base
    pi = id_.data_ptr() + 2 * offset_bias
    plan = native.xpress_describe_plan(pb, pi, N, B, V, V + pad, V + pad)
    aligned = offset_base % 8 == 0 and offset_bias % 8 == 0 and (V + pad) % 8 == 0
    assert plan["vector_path"] == aligned
    say("unaligned ob=%d oi=%d pad=%d combine=%d" % (offset_base, offset_bias, pad, combine))
    with Plan(combine, 0, 0):
        got = gpu_blk(pb, pi, blk0, N, B, V, V + pad, V + pad)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("N,B,V", [(1, 2, 1), (1, 2, 152064), (7, 2, 1000), (1, 33, 4000),
                                   (64, 3, 256), (300, 2, 40)])
def test_degenerate_shapes(N, B, V):
    base, bias, blk0 = _random_rows(N, B, V, seed=N * B + V)
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    bd, id_ = to_dev(base), to_dev(bias)
    for combine in [0] + COMBINES:
        say("degenerate N=%d B=%d V=%d combine=%d" % (N, B, V, combine))
        with Plan(combine, 0, 0):
            got = gpu_blk(bd, id_, blk0, N, B, V, V, V)
        assert np.array_equal(got, want)


def test_no_rows_writes_nothing():
    import torch
    blk = torch.full((4, 1), 5, dtype=torch.int64, device="cuda")
    say("no rows (B=1)")
    native.xpress_add_argmax_to_blk(0, 0, blk, 4, 1, 100, 100, 100)
    native.xpress_add_argmax_to_blk(0, 0, 0, 0, 16, 100, 100, 100)
    torch.cuda.synchronize()
    assert (blk.cpu() == 5).all()


def test_invalid_arguments_raise():
    import torch
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    blk = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(native.XpressError) as e:
        native.xpress_add_argmax_to_blk(x, x, blk, 1, 2, 32, 16, 32)
    assert e.value.status == native.XPRESS_EINVAL
    with pytest.raises(native.XpressError):
        native.xpress_add_argmax_to_blk(x, x, x, 1, 2, 8, 8, 8)  # blk aliases base
    with pytest.raises(ValueError):
        native.xpress_add_argmax_to_blk(x.cpu(), x, blk, 1, 2, 8, 8, 8)


@pytest.mark.parametrize("combine", [0] + COMBINES)
def test_guard_cells_and_anchor_untouched(combine):
    import torch
    N, B, V = 5, 6, 20000
    base, bias, blk0 = _random_rows(N, B, V, seed=99)
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    guard = 0x5A5A5A5A5A5A5A5A
    buf = np.full(N * B + 64, guard, dtype=np.int64)
    buf[32:32 + N * B] = blk0.reshape(-1)
    buf_d = to_dev(buf)
    say("guard cells combine=%d" % combine)
    with Plan(combine, 0, 0):
        native.xpress_add_argmax_to_blk(to_dev(base), to_dev(bias), buf_d.data_ptr() + 32 * 8,
                                        N, B, V, V, V)
    torch.cuda.synchronize()
    out = buf_d.cpu().numpy()
    assert (out[:32] == guard).all() and (out[32 + N * B:] == guard).all()
    assert np.array_equal(out[32:32 + N * B].reshape(N, B), want)


@pytest.mark.parametrize("N,B,V,pad", [(2, 4, 1000, 0), (3, 5, 77, 9), (5, 3, 4097, 64),
                                       (32, 16, 152064, 0)])
def test_planted_closed_form(N, B, V, pad):
    base, bias, blk0 = workloads.planted(N, B, V, seed=N * 100 + V, pad=pad)
    bd, id_ = to_dev(base), to_dev(bias)
    want = blk0.copy()
    want[:, 1:] = (np.arange(N * (B - 1)) % V).reshape(N, B - 1)
    for combine in [0] + COMBINES:
        say("planted N=%d B=%d V=%d combine=%d" % (N, B, V, combine))
        with Plan(combine, 0, 0):
            got = gpu_blk(bd, id_, blk0, N, B, V, V + pad, V + pad)
        assert np.array_equal(got, want)


def _tie_rows(V, positions, value_bits, fill_bits, rows):
    base = np.full((rows, V), fill_bits, dtype=np.uint16)
    bias = np.zeros((rows, V), dtype=np.uint16)
    for r in range(rows):
        for p in positions[r]:
            base[r, p] = value_bits
    return base, bias


@pytest.mark.parametrize("combine", COMBINES)
@pytest.mark.parametrize("splits", [2, 3, 7, 16, 64])
def test_equal_maxima_across_workgroups(combine, splits):
    """Equal maxima on both sides of every boundary that could reorder them:
    vector (8), wave (64 x 8), workgroup split edges and 4096-element chunks;
    the lowest index must win whatever the split."""
    V = 3 * 4096 + 517
    nvec = V // 8
    edges = sorted({8, 512, 4096, 8192, 12288} |
                   {(s * nvec // splits) * 8 for s in range(1, splits)})
    positions = []
    for e in edges:
        positions.append([e - 1, e])      # straddles the edge: e - 1 wins
        positions.append([e, V - 1])      # later copy at the tail
        positions.append([V - 1 - (e % 5), V - 1])
    rows = len(positions)
    N, B = rows, 2
    base, bias = _tie_rows(V, positions, 0x4000, 0x3F80, rows)  # 2.0 among 1.0
    blk0 = np.full((N, B), -7, dtype=np.int64)
    want = blk0.copy()
    want[:, 1] = [min(p) for p in positions]
    say("ties across workgroups combine=%d splits=%d" % (combine, splits))
    with Plan(combine, splits, 64):
        got = gpu_blk(to_dev(base), to_dev(bias), blk0, N, B, V, V, V)
    assert np.array_equal(got, want)
    assert np.array_equal(want, oracle_blk(base, bias, blk0, N, B, V, V, V))


@pytest.mark.parametrize("splits", [65, 200, 513, 1100])
def test_two_pass_many_splits(splits):
    """More keys per row than one wave holds, which the second pass loads in
    batches of 512: equal maxima planted at the starts of two splits, on
    either side of key 64 and key 512, must still give the lowest index."""
    V = 40000
    nvec = V // 8
    N, B = 4, 4
    rows = N * (B - 1)
    rng = np.random.default_rng(900 + splits)
    base = workloads.f32_to_bf16_bits(rng.normal(0.0, 4.0, (rows, V)).astype(np.float32))
    bias = workloads.f32_to_bf16_bits(rng.normal(0.0, 0.5, (rows, V)).astype(np.float32))
    marks = sorted({s for s in (0, 1, 63, 64, 65, 511, 512, 513, splits - 1) if s < splits})
    start = lambda s: (s * nvec // splits) * 8
    want = np.full((N, B), -3, dtype=np.int64)
    blk0 = want.copy()
    for r in range(rows):
        s1 = marks[r % len(marks)]
        s2 = marks[(r * 5 + 3) % len(marks)]
        s1, s2 = min(s1, s2), max(s1, s2)
        for s in {s1, s2}:
            base[r, start(s)] = 0x4220   # 40.0: above every Gaussian sum here
            bias[r, start(s)] = 0x0000
        want[r // (B - 1), 1 + r % (B - 1)] = start(s1)
    assert np.array_equal(want, oracle_blk(base, bias, blk0, N, B, V, V, V))
    say("two-pass many splits=%d" % splits)
    with Plan(native.XPRESS_COMBINE_TWO_PASS, splits, 64):
        got = gpu_blk(to_dev(base), to_dev(bias), blk0, N, B, V, V, V)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("combine", COMBINES)
def test_signed_zero_and_special_rows(combine):
    """-0 before +0 in another workgroup, all -inf rows, +inf ties, subnormal
    sums, overflow to +inf: every case against the oracle."""
    V = 5000
    rows = []

    def row():
        a = np.full(V, 0xFF80, dtype=np.uint16)   # -inf
        b = np.zeros(V, dtype=np.uint16)
        rows.append((a, b))
        return a, b

    a, b = row()                                    # all -inf -> 0
    a, b = row(); a[100] = 0x8000; b[100] = 0x8000; a[4000] = 0; b[4000] = 0      # -0 first
    a, b = row(); a[100] = 0; a[4000] = 0x8000; b[4000] = 0x8000                  # +0 first
    a, b = row(); a[7] = 0x7F80; a[4999] = 0x7F80                                 # +inf tie
    a, b = row(); a[10] = 0x0001; a[4900] = 0x0001; b[4900] = 0x0001              # subnormals
    a, b = row(); a[3] = 0x7F7F; b[3] = 0x7F7F; a[2] = 0x7F7F                     # max+max = +inf beats max
    a, b = row(); a[:] = 0x3F80; b[4096] = 0x3B80; b[4097] = 0x3BC0               # RNE tie/round
    a, b = row(); a[:] = 0xBF80; b[:] = 0x3F80                                    # all zero sums
    base = np.stack([r[0] for r in rows])
    bias = np.stack([r[1] for r in rows])
    N, B = len(rows), 2
    blk0 = np.full((N, B), 3, dtype=np.int64)
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    assert list(want[:, 1]) == [0, 100, 100, 7, 4900, 3, 4097, 0]
    for splits in (1, 2, 5):
        say("special rows combine=%d splits=%d" % (combine, splits))
        with Plan(combine, splits, 64):
            got = gpu_blk(to_dev(base), to_dev(bias), blk0, N, B, V, V, V)
        assert np.array_equal(got, want), splits


@pytest.mark.parametrize("combine", [native.XPRESS_COMBINE_ATOMIC,
                                     native.XPRESS_COMBINE_TWO_PASS,
                                     native.XPRESS_COMBINE_BALANCED])
def test_repeated_calls_leave_a_clean_workspace(combine):
    import torch
    N, B, V = 6, 9, 30000
    cases = [_random_rows(N, B, V, seed=s, kind="ties" if s % 2 else "normal")
             for s in range(4)]
    with Plan(combine, 11, 256):
        for it in range(3):
            for s, (base, bias, blk0) in enumerate(cases):
                say("repeat combine=%d it=%d case=%d" % (combine, it, s))
                got = gpu_blk(to_dev(base), to_dev(bias), blk0, N, B, V, V, V)
                want = oracle_blk(base, bias, blk0, N, B, V, V, V)
                assert np.array_equal(got, want), (it, s)
    torch.cuda.synchronize()


def test_graph_replay_matches_eager():
    import torch
    N, B, V = 8, 9, 40000
    cases = [_random_rows(N, B, V, seed=50 + s) for s in range(3)]
    base_d = to_dev(cases[0][0])
    bias_d = to_dev(cases[0][1])
    blk_d = to_dev(cases[0][2])
    s = torch.cuda.Stream()
    native.xpress_reserve(N, B, V, stream=s)
    g = torch.cuda.CUDAGraph()
    say("graph capture")
    with torch.cuda.graph(g, stream=s):
        native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V, stream=s)
    for rep in range(6):
        base, bias, blk0 = cases[rep % 3]
        base_d.copy_(to_dev(base))
        bias_d.copy_(to_dev(bias))
        blk_d.copy_(to_dev(blk0))
        torch.cuda.synchronize()
        say("graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        got = blk_d.cpu().numpy()
        eager = gpu_blk(base_d, bias_d, blk0, N, B, V, V, V)
        assert np.array_equal(got, eager), rep
        assert np.array_equal(got, oracle_blk(base, bias, blk0, N, B, V, V, V)), rep


def test_two_streams_at_once():
    import torch
    N, B, V = 16, 16, 60000
    c0 = _random_rows(N, B, V, seed=1)
    c1 = _random_rows(N, B, V, seed=2, kind="ties")
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    d0 = [to_dev(x) for x in c0]
    d1 = [to_dev(x) for x in c1]
    torch.cuda.synchronize()
    say("two streams")
    with Plan(native.XPRESS_COMBINE_ATOMIC, 13, 256):
        for _ in range(5):
            native.xpress_add_argmax_to_blk(d0[0], d0[1], d0[2], N, B, V, V, V, stream=s0)
            native.xpress_add_argmax_to_blk(d1[0], d1[1], d1[2], N, B, V, V, V, stream=s1)
        torch.cuda.synchronize()
    assert np.array_equal(d0[2].cpu().numpy(), oracle_blk(*c0, N, B, V, V, V))
    assert np.array_equal(d1[2].cpu().numpy(), oracle_blk(*c1, N, B, V, V, V))


def test_element_step_every_bf16_pair():
    """The device element step (the code every readout kernel inlines) equals
    the oracle's rounded sum for all 2^32 pairs of bf16 patterns; NaN
    results only need to be NaN on both sides."""
    import threading
    import torch
    chunk = 2048
    a_all = np.arange(65536, dtype=np.uint16)
    out_d = torch.empty(chunk * 65536, dtype=torch.int16, device="cuda")
    bad = 0
    for s in range(0, 65536, chunk):
        say("element table a=[%d, %d)" % (s, s + chunk))
        a_d = to_dev(a_all[s:s + chunk])
        native.xpress_bf16_add_round_table(a_d, chunk, out_d)
        torch.cuda.synchronize()
        got = out_d.cpu().numpy().view(np.uint16).reshape(chunk, 65536)
        want = np.empty_like(got)
        nthr = 16
        part = chunk // nthr

        def work(t):
            want[t * part:(t + 1) * part] = oracle.bf16_sum_grid(
                a_all[s + t * part:s + (t + 1) * part])

        ts = [threading.Thread(target=work, args=(t,)) for t in range(nthr)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
        assert np.array_equal(nan_g, nan_w), s
        bad += int(np.count_nonzero((got != want) & ~nan_w))
    assert bad == 0


def _balanced_edges(rows, V, per_cu):
    """Range boundaries (row, vector) of the balanced plan for these sizes."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    g = cus * per_cu
    nvec = V // 8
    q = rows * nvec
    edges = sorted({(k * q) // g for k in range(1, g)})
    return [(x // nvec, x % nvec) for x in edges]


@pytest.mark.parametrize("per_cu,threads", [(1, 256), (2, 256), (3, 128), (2, 1024)])
def test_balanced_ties_on_range_edges(per_cu, threads):
    """Equal maxima placed on both sides of the balanced plan's range edges
    (the last vector of one workgroup's range and the first of the next):
    the lower index must win, and rows shared by 2-3 ranges must fold to the
    same answer as the oracle."""
    rows, V = 300, 9000 + 5   # V % 8 != 0: the tail follows the row's last vector
    S = V + 3                 # row stride a multiple of 8 elements (16-byte rows)
    g = np.random.Generator(np.random.PCG64(per_cu * 7 + threads))
    base = np.full((rows, S), 0x42C8, dtype=np.uint16)   # +100 poison in the padding
    bias = np.zeros((rows, S), dtype=np.uint16)
    base[:, :V] = 0x3F80                                  # 1.0
    for r, qv in _balanced_edges(rows, V, per_cu):
        e = qv * 8
        base[r, e] = 0x4000                 # 2.0 at the first element of the range
        if e >= 1:
            base[r, e - 1] = 0x4000         # and at the last element of the previous one
    # some rows: maximum only in the tail, or a single copy anywhere
    for r in range(0, rows, 17):
        base[r, V - 1] = 0x4040
    for r in range(5, rows, 23):
        base[r, :V] = 0x3F80
        base[r, int(g.integers(0, V))] = 0x4000
    N, B = rows, 2
    blk0 = np.full((N, B), 11, dtype=np.int64)
    want = oracle_blk(base, bias, blk0, N, B, V, S, S)
    bd, id_ = to_dev(base), to_dev(bias)
    with Plan(native.XPRESS_COMBINE_BALANCED, per_cu, threads):
        plan = native.xpress_describe_plan(bd, id_, N, B, V, S, S)
        assert plan["combine"] == "balanced", plan
        say("balanced range edges per_cu=%d threads=%d" % (per_cu, threads))
        for _ in range(3):
            got = gpu_blk(bd, id_, blk0, N, B, V, S, S)
            assert np.array_equal(got, want)


@pytest.mark.parametrize("combine", COMBINES)
def test_nan_sums_never_win(combine):
    """NaN sums are outside the contract; the reading taken (the oracle's) is
    that a NaN never wins: NaN at index 0, NaN beside +inf, +inf + -inf,
    NaN with the sign set, and a row of NaN and -inf sums (index 0)."""
    V = 5000
    a = np.zeros((6, V), dtype=np.uint16)
    b = np.zeros((6, V), dtype=np.uint16)
    a[0, 0] = 0x7FC0; a[0, 4000] = 0x3F80                       # NaN first, 1 later
    a[1, :] = 0xBF80; a[1, 3] = 0x7F80; b[1, 3] = 0xFF80       # +inf + -inf, rest -1
    a[1, 4500] = 0x3F00
    a[2, 10] = 0x7FC0; a[2, 11] = 0x7F80; a[2, 4999] = 0x7F80  # NaN before +inf
    a[3, :] = 0xFF80; a[3, 7] = 0xFFC0; a[3, 4097] = 0x7FC0    # -inf and NaN only
    a[4, 100] = 0xFFC0; a[4, 4096] = 0x3F80; a[4, 4097] = 0x3F80
    a[5, :] = 0x7FC1                                            # every sum NaN
    N, B = 6, 2
    blk0 = np.full((N, B), 4, dtype=np.int64)
    want = oracle_blk(a, b, blk0, N, B, V, V, V)
    assert list(want[:, 1]) == [4000, 4500, 11, 0, 4096, 0]
    for splits in (1, 2, 5):
        say("NaN rows combine=%d splits=%d" % (combine, splits))
        with Plan(combine, splits, 64):
            got = gpu_blk(to_dev(a), to_dev(b), blk0, N, B, V, V, V)
        assert np.array_equal(got, want), splits
