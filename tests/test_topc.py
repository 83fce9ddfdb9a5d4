"""Parity of the HIP top-C readout with the CPU oracle, through the C-ABI.

blk[n, 1+j] must equal cand[r, first argmax_c bf16(base_c + bias_c)] bit for
bit, with slot 0 and everything outside blk's draft slots untouched.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import Plan, say, to_dev
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

COMBINES = [native.XPRESS_COMBINE_SINGLE, native.XPRESS_COMBINE_ATOMIC,
            native.XPRESS_COMBINE_TWO_PASS, native.XPRESS_COMBINE_BALANCED]


def oracle_topc(base_c, bias_c, cand, blk0, N, B, C):
    want = blk0.copy()
    oracle.topc_argmax_to_blk(base_c, bias_c, cand, want, N, B, C)
    return want


def gpu_topc(base_d, bias_d, cand_d, blk0, N, B, C):
    import torch
    blk_d = to_dev(blk0)
    native.xpress_topc_argmax_to_blk(base_d, bias_d, cand_d, blk_d, N, B, C)
    torch.cuda.synchronize()
    return blk_d.cpu().numpy()


_cache = {}


def case(name):
    if name not in _cache:
        w = workloads.TOPC_WORKLOADS[name]
        base_c, bias_c, cand, blk0 = workloads.generate_topc(w)
        want = oracle_topc(base_c, bias_c, cand, blk0, w.N, w.B, w.C)
        _cache[name] = (w, blk0, to_dev(base_c), to_dev(bias_c), to_dev(cand), want)
    return _cache[name]


@pytest.mark.parametrize("name", list(workloads.TOPC_WORKLOADS))
def test_topc_workload_default_plan(name):
    w, blk0, bd, id_, cd, want = case(name)
    say("topc %s default plan" % name)
    got = gpu_topc(bd, id_, cd, blk0, w.N, w.B, w.C)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["topc_n32_b16_c256", "topc_ties_n32_b16_c256",
                                  "topc_n32_b16_c4096"])
@pytest.mark.parametrize("combine", COMBINES)
@pytest.mark.parametrize("threads,splits", [(64, 0), (256, 0), (1024, 0), (64, 3), (128, 2)])
def test_topc_every_plan(name, combine, threads, splits):
    w, blk0, bd, id_, cd, want = case(name)
    say("topc %s combine=%d threads=%d splits=%d" % (name, combine, threads, splits))
    with Plan(combine, splits, threads):
        got = gpu_topc(bd, id_, cd, blk0, w.N, w.B, w.C)
    assert np.array_equal(got, want)


def _rows(rows, C, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.integers(-3, 4, size=(rows, C)).astype(np.float32)
    b = g.integers(-3, 4, size=(rows, C)).astype(np.float32)
    cand = g.integers(0, 2 ** 40, size=(rows, C), dtype=np.int64)
    return workloads.f32_to_bf16_bits(a), workloads.f32_to_bf16_bits(b), cand


@pytest.mark.parametrize("C", [1, 2, 7, 8, 9, 63, 64, 65, 100, 1000, 4097])
@pytest.mark.parametrize("combine", COMBINES)
def test_topc_ragged_candidates(C, combine):
    N, B = 5, 9
    base_c, bias_c, cand = _rows(N * (B - 1), C, C)
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 123
    want = oracle_topc(base_c, bias_c, cand, blk0, N, B, C)
    bd, id_, cd = to_dev(base_c), to_dev(bias_c), to_dev(cand)
    say("topc ragged C=%d combine=%d" % (C, combine))
    for splits in (0, 2):
        with Plan(combine, splits, 64):
            got = gpu_topc(bd, id_, cd, blk0, N, B, C)
        assert np.array_equal(got, want), (C, combine, splits)


def test_topc_planted_and_guard_cells():
    import torch
    N, B, C = 32, 16, 512
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(5))
    base = (g.integers(-64, 64, size=(rows, C)) / 16.0).astype(np.float32)
    base[np.arange(rows), np.arange(rows) % C] = 64.0
    bias = (g.integers(-64, 64, size=(rows, C)) / 16.0).astype(np.float32)
    cand = g.integers(0, 152064, size=(rows, C), dtype=np.int64)
    guard = 0x3C3C3C3C3C3C3C3C
    buf = np.full(N * B + 64, guard, dtype=np.int64)
    buf[32:32 + N * B] = np.tile(np.array([9] + [-1] * (B - 1)), N)
    buf_d = to_dev(buf)
    say("topc planted + guard cells")
    native.xpress_topc_argmax_to_blk(to_dev(workloads.f32_to_bf16_bits(base)),
                                     to_dev(workloads.f32_to_bf16_bits(bias)), to_dev(cand),
                                     buf_d.data_ptr() + 32 * 8, N, B, C)
    torch.cuda.synchronize()
    out = buf_d.cpu().numpy()
    assert (out[:32] == guard).all() and (out[32 + N * B:] == guard).all()
    blk = out[32:32 + N * B].reshape(N, B)
    assert (blk[:, 0] == 9).all()
    assert np.array_equal(blk[:, 1:].reshape(-1), cand[np.arange(rows), np.arange(rows) % C])


def test_topc_invalid_arguments_raise():
    import torch
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    c = torch.zeros(64, dtype=torch.int64, device="cuda")
    blk = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(native.XpressError):
        native.xpress_topc_argmax_to_blk(x, x, 0, blk, 1, 2, 8)
    with pytest.raises(native.XpressError):
        native.xpress_topc_argmax_to_blk(x, x, c, c, 1, 2, 8)  # blk aliases cand


@pytest.mark.parametrize("C", [1, 2, 7, 8, 9, 63, 64, 65, 100, 1000, 4096, 4097])
@pytest.mark.parametrize("offset", [0, 1])
def test_topc_default_plan_ragged_and_unaligned(C, offset):
    """The default top-C plan (one wave per row carrying the ids, up to 4096
    candidates; the streaming readout above) on ragged counts, with aligned
    buffers and with base_c / bias_c / cand shifted off 16-byte alignment."""
    import torch
    N, B = 7, 5
    rows = N * (B - 1)
    base_c, bias_c, cand = _rows(rows, C, 1000 + C)
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 55
    want = oracle_topc(base_c, bias_c, cand, blk0, N, B, C)
    big_a = np.zeros(base_c.size + 8, np.uint16)
    big_b = np.zeros(bias_c.size + 8, np.uint16)
    big_c = np.zeros(cand.size + 2, np.int64)
    big_a[offset:offset + base_c.size] = base_c.reshape(-1)
    big_b[offset:offset + bias_c.size] = bias_c.reshape(-1)
    big_c[offset:offset + cand.size] = cand.reshape(-1)
    da, db, dc = to_dev(big_a), to_dev(big_b), to_dev(big_c)
    blk_d = to_dev(blk0)
    say("topc default plan C=%d offset=%d" % (C, offset))
    native.xpress_topc_argmax_to_blk(da.data_ptr() + 2 * offset, db.data_ptr() + 2 * offset,
                                     dc.data_ptr() + 8 * offset, blk_d, N, B, C)
    torch.cuda.synchronize()
    assert np.array_equal(blk_d.cpu().numpy(), want)


@pytest.mark.parametrize("C", [64, 256, 1024])    # one wave per row up to 256, else streaming
def test_topc_special_values(C):
    """Special values against the oracle on both top-C paths: all -inf rows
    (position 0's id wins), +inf ties (the lowest position), -0 before +0,
    subnormal sums, overflow to +inf, and a winner at the last position;
    candidate ids are large and distinct so that a position slip shows."""
    N, B = 3, 9
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(5050 + C))
    base_c = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, C)) / 4.0).astype(np.float32))
    bias_c = workloads.f32_to_bf16_bits((g.integers(-4, 5, size=(rows, C)) / 8.0).astype(np.float32))
    cand = (g.permutation(rows * C).astype(np.int64).reshape(rows, C) + (1 << 33))
    NEG_INF, POS_INF, NEG_ZERO, MAX_FIN = 0xFF80, 0x7F80, 0x8000, 0x7F7F
    base_c[0, :] = NEG_INF
    bias_c[0, :] = 0
    base_c[1, [C // 3, C - 1]] = POS_INF
    base_c[2, :] = NEG_ZERO
    bias_c[2, :] = NEG_ZERO                       # every sum is -0: position 0 wins
    base_c[3, :] = NEG_ZERO
    bias_c[3, :] = 0
    bias_c[3, C // 2] = NEG_ZERO                  # -0 + -0 = -0 ties +0: position 0
    base_c[4, :] = 0xBF80
    bias_c[4, :] = 0
    base_c[4, C - 1] = 0x0001                     # a subnormal at the last position
    base_c[5, [1, C - 2]] = MAX_FIN
    bias_c[5, [1, C - 2]] = MAX_FIN               # both overflow to +inf: position 1
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 77
    want = oracle_topc(base_c, bias_c, cand, blk0, N, B, C)
    w1 = want[:, 1:].reshape(-1)
    assert w1[0] == cand[0, 0] and w1[1] == cand[1, C // 3] and w1[2] == cand[2, 0]
    assert w1[3] == cand[3, 0] and w1[4] == cand[4, C - 1] and w1[5] == cand[5, 1]
    say("topc special values C=%d" % C)
    got = gpu_topc(to_dev(base_c), to_dev(bias_c), to_dev(cand), blk0, N, B, C)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("C", [64, 256, 1024])    # one wave per row up to 256, else streaming
def test_topc_nan_sums_never_win(C):
    """A NaN sum never wins on either top-C path (the oracle's reading of a
    case outside the contract): NaN at position 0 of every lane, NaN from
    +inf + -inf before +inf, NaN with the sign set, and rows whose sums are
    all NaN or NaN and -inf (position 0's id)."""
    N, B = 2, 5
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(6060 + C))
    base_c = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, C)) / 4.0).astype(np.float32))
    bias_c = np.zeros((rows, C), dtype=np.uint16)
    cand = (g.permutation(rows * C).astype(np.int64).reshape(rows, C) + (1 << 34))
    base_c[0, :64] = 0x7FC0                       # each lane's first candidate is NaN
    base_c[1, 5] = 0x7F80; bias_c[1, 5] = 0xFF80  # +inf + -inf = NaN ...
    base_c[1, C - 1] = 0x7F80                     # ... before the only +inf
    base_c[2, ::3] = 0xFFC0                       # NaN with the sign set
    base_c[3, :] = 0x7FC0                         # every sum NaN: position 0
    base_c[4, :] = 0xFF80
    base_c[4, 1::2] = 0x7FC0                      # -inf and NaN: position 0
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = 12
    want = oracle_topc(base_c, bias_c, cand, blk0, N, B, C)
    w1 = want[:, 1:].reshape(-1)
    assert w1[1] == cand[1, C - 1] and w1[3] == cand[3, 0] and w1[4] == cand[4, 0]
    say("topc NaN sums C=%d" % C)
    got = gpu_topc(to_dev(base_c), to_dev(bias_c), to_dev(cand), blk0, N, B, C)
    assert np.array_equal(got, want)
