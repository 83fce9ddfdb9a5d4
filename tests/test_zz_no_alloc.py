"""xpress_add_argmax_to_blk_noalloc: the readout without any device
allocation, checked through the C-ABI against xpress_add_argmax_to_blk (and
the oracle) on two calls in a row, the second with a smaller input, on a
graph captured without a reserve, and on the table-size limit.  Runs last:
its calls share the library's fixed key table on the GPU."""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import Plan, oracle_blk, say, to_dev
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _case(N, B, V, seed, pad=0):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = N * (B - 1)
    base = np.full((rows, V + pad), 0x42C8, np.uint16)
    bias = np.full((rows, V + pad), 0x42C8, np.uint16)
    base[:, :V] = workloads.f32_to_bf16_bits(g.standard_normal((rows, V), dtype=np.float32) * 3)
    bias[:, :V] = workloads.f32_to_bf16_bits(g.integers(-2, 3, size=(rows, V)).astype(np.float32))
    blk = np.full((N, B), -1, dtype=np.int64)
    blk[:, 0] = g.integers(0, V, size=N)
    return base, bias, blk


def _both(base, bias, blk0, N, B, V, S):
    import torch
    bd, id_ = to_dev(base), to_dev(bias)
    ref = to_dev(blk0)
    got = to_dev(blk0)
    native.xpress_add_argmax_to_blk(bd, id_, ref, N, B, V, S, S)
    native.xpress_add_argmax_to_blk_noalloc(bd, id_, got, N, B, V, S, S)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    ((2, 9, 150000, 0), (1, 4, 70000, 8)),      # both split in two passes
    ((32, 16, 20000, 0), (3, 5, 65537, 0)),     # one workgroup per row, then split
    ((4, 17, 100003, 1), (1, 2, 9, 0))])        # unaligned scalar path, then a tiny row
def test_noalloc_matches_the_allocating_entry(first, second):
    for k, (N, B, V, pad) in enumerate((first, second)):
        base, bias, blk0 = _case(N, B, V, seed=100 * k + V, pad=pad)
        plan = native.xpress_describe_plan(256, 256, N, B, V, V + pad, V + pad)
        say("noalloc call %d N=%d B=%d V=%d plan=%s" % (k, N, B, V, plan))
        got, ref = _both(base, bias, blk0, N, B, V, V + pad)
        assert np.array_equal(got, ref), k
        assert np.array_equal(got, oracle_blk(base, bias, blk0, N, B, V, V + pad, V + pad)), k


def test_noalloc_allocates_nothing_and_captures_without_reserve():
    import torch
    N, B, V = 2, 9, 150000
    torch.cuda.synchronize()
    native.xpress_release()
    cases = [_case(N, B, V, seed=7 + k) for k in range(3)]
    bd, id_, blk_d = (to_dev(a) for a in cases[0])
    # one eager call (looks the table up on this device); no workspace appears
    native.xpress_add_argmax_to_blk_noalloc(bd, id_, blk_d, N, B, V, V, V)
    torch.cuda.synchronize()
    assert native.xpress_workspace_bytes() == 0
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    say("noalloc capture without reserve")
    with torch.cuda.graph(g, stream=s):
        native.xpress_add_argmax_to_blk_noalloc(bd, id_, blk_d, N, B, V, V, V, stream=s)
    assert native.xpress_workspace_bytes() == 0
    for rep in range(4):
        base, bias, blk0 = cases[rep % 3]
        bd.copy_(to_dev(base))
        id_.copy_(to_dev(bias))
        blk_d.copy_(to_dev(blk0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(blk_d.cpu().numpy(), oracle_blk(base, bias, blk0, N, B, V, V, V)), rep


def test_noalloc_rejects_a_table_beyond_its_size():
    import torch
    N, B, V = 2, 9, 150000                 # 16 rows
    base, bias, blk0 = _case(N, B, V, seed=3)
    bd, id_, blk_d = to_dev(base), to_dev(bias), to_dev(blk0)
    torch.cuda.synchronize()
    with Plan(native.XPRESS_COMBINE_TWO_PASS, 300, 64):      # 16 x 300 = 4800 keys
        with pytest.raises(native.XpressError) as ei:
            native.xpress_add_argmax_to_blk_noalloc(bd, id_, blk_d, N, B, V, V, V)
        assert ei.value.status == native.XPRESS_ESCRATCH
        torch.cuda.synchronize()
        assert np.array_equal(blk_d.cpu().numpy(), blk0)
    with Plan(native.XPRESS_COMBINE_TWO_PASS, 256, 64):      # 4096 keys: the limit
        got, ref = _both(base, bias, blk0, N, B, V, V)
        assert np.array_equal(got, ref)
    with Plan(native.XPRESS_COMBINE_ATOMIC, 7, 128):         # runs as two-pass here
        got, ref = _both(base, bias, blk0, N, B, V, V)
        assert np.array_equal(got, ref)
