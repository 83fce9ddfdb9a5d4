"""Results do not depend on the order in which workgroups run.

xpress_set_reverse_order makes every later launch visit its work units from
last to first (the streaming readout's (row, split) units or balanced
ranges; the readout with in-place bias's (range, row block) pairs), so the
combines receive their keys in another order: the atomic and balanced
combines fold into each row's word in a different sequence, the two-pass
table is filled by different workgroups first.  Each case runs in both
orders, twice each, and every result must equal the oracle's bit for bit.
The workgroups do the same work either way; every launch is valid for its
buffers."""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import Plan, gpu_blk, oracle_blk, say, to_dev, ORACLE_THREADS
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(autouse=True)
def default_order():
    yield
    native.xpress_set_reverse_order(False)
    native.xpress_set_plan(0, 0, 0)


def _rows_with_ties(N, B, V, seed):
    """Rows whose maximum occurs several times, spread over the row, so that
    a combine taking the wrong tie would show."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = N * (B - 1)
    base = workloads.f32_to_bf16_bits(g.integers(-8, 8, size=(rows, V)).astype(np.float32))
    bias = np.zeros((rows, V), np.uint16)
    for r in range(rows):
        pos = np.sort(g.choice(V, size=5, replace=False))
        base[r, pos] = workloads.f32_to_bf16_bits(np.full(5, 64.0, np.float32))
    blk = np.full((N, B), -1, dtype=np.int64)
    blk[:, 0] = g.integers(0, V, size=N)
    return base, bias, blk


@pytest.mark.parametrize("combine,splits", [
    (native.XPRESS_COMBINE_SINGLE, 0),
    (native.XPRESS_COMBINE_ATOMIC, 7),
    (native.XPRESS_COMBINE_TWO_PASS, 13),
    (native.XPRESS_COMBINE_BALANCED, 2),
    (native.XPRESS_COMBINE_AUTO, 0)])
@pytest.mark.parametrize("N,B,V", [(2, 4, 100003), (4, 8, 50008), (8, 16, 20000), (32, 16, 4099)])
def test_readout_either_order(combine, splits, N, B, V):
    base, bias, blk0 = _rows_with_ties(N, B, V, seed=N * 1000 + V % 997)
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    base_d, bias_d = to_dev(base), to_dev(bias)
    with Plan(combine, splits, 0):
        for rev in (False, True, False, True):
            say("readout combine=%d splits=%d N=%d B=%d V=%d reversed=%s"
                % (combine, splits, N, B, V, rev))
            native.xpress_set_reverse_order(rev)
            got = gpu_blk(base_d, bias_d, blk0, N, B, V, V, V)
            assert np.array_equal(got, want), (rev, combine, splits)


@pytest.mark.parametrize("N,B,V,R", [(2, 8, 40003, 64),      # 14 rows: one wave
                                     (8, 16, 30000, 128),    # 120 rows: two waves
                                     (20, 16, 32003, 256)])  # 300 rows: eight waves
def test_gemm_readout_either_order(N, B, V, R):
    import torch
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(rows + V + R))
    S = V + (-V) % 8                     # row stride: a multiple of 8
    base = np.zeros((rows, S), np.uint16)
    base[:, :V] = workloads.f32_to_bf16_bits((g.integers(-16, 17, size=(rows, V)) / 4.0)
                                             .astype(np.float32))
    x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, R)) / 8.0).astype(np.float32))
    wt = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(V, R)) / 8.0).astype(np.float32))
    blk0 = np.full((N, B), -1, dtype=np.int64)
    want = blk0.copy()
    want[:, 1:] = oracle.gemm_argmax_rows(base, x, wt, range(rows), V, R, S,
                                          threads=ORACLE_THREADS).reshape(N, B - 1)
    bd, xd, wd = to_dev(base), to_dev(x), to_dev(wt)
    for rev in (False, True, False, True):
        say("gemm readout N=%d B=%d V=%d R=%d reversed=%s" % (N, B, V, R, rev))
        native.xpress_set_reverse_order(rev)
        blk_d = to_dev(blk0)
        native.xpress_readout_gemm_argmax_to_blk(bd, xd, wd, blk_d, N, B, V, R, S)
        torch.cuda.synchronize()
        assert np.array_equal(blk_d.cpu().numpy(), want), rev
