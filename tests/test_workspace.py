"""The library's device workspace: error paths and lifetime, through the
C-ABI on a GPU.

- a call captured into a HIP graph that would have to grow the workspace
  returns XPRESS_ECAPTURE and queues nothing;
- after xpress_reserve the same capture succeeds and replays match the oracle;
- growth retires the old allocation instead of freeing it, so a graph
  captured before a larger eager call still replays correctly;
- XPRESS_ENOMEM through the test cap (xpress_set_workspace_limit), with
  nothing queued and blk untouched;
- xpress_release frees live and retired workspace and the next call
  allocates afresh.

Every call here is valid for the buffers it gets; the error paths return
before any launch.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import Plan, gpu_blk, oracle_blk, say, to_dev
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

# 6 rows of 100000: the automatic plan splits each row over 3 workgroups and
# combines in two passes through the workspace's key table
N, B, V = 2, 4, 100000


def _case(seed):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = N * (B - 1)
    base = workloads.f32_to_bf16_bits(g.standard_normal((rows, V), dtype=np.float32) * 3)
    bias = workloads.f32_to_bf16_bits(g.standard_normal((rows, V), dtype=np.float32))
    blk = np.full((N, B), -1, dtype=np.int64)
    blk[:, 0] = g.integers(0, V, size=N)
    return base, bias, blk


@pytest.fixture(autouse=True)
def fresh_workspace():
    import torch
    torch.cuda.synchronize()
    native.xpress_set_workspace_limit(0)
    native.xpress_release()
    yield
    native.xpress_set_plan(0, 0, 0)
    native.xpress_set_workspace_limit(0)
    torch.cuda.synchronize()
    native.xpress_release()


def test_plan_uses_the_workspace():
    p = native.xpress_describe_plan(256, 256, N, B, V, V, V)
    assert p["combine"] == "two_pass" and p["launches"] == 2, p


def test_capture_that_must_grow_returns_ecapture_and_queues_nothing():
    import torch
    base, bias, blk0 = _case(1)
    base_d, bias_d, blk_d = to_dev(base), to_dev(bias), to_dev(blk0)
    marker = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    assert native.xpress_workspace_bytes() == 0
    g = torch.cuda.CUDAGraph()
    say("capture with an empty workspace")
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(native.XpressError) as ei:
            native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V, stream=s)
        marker.add_(1)                     # the graph holds this and nothing else
    assert ei.value.status == native.XPRESS_ECAPTURE
    assert native.xpress_workspace_bytes() == 0
    g.replay()
    torch.cuda.synchronize()
    assert marker.cpu().tolist() == [1, 1, 1, 1]
    assert np.array_equal(blk_d.cpu().numpy(), blk0)


def test_reserve_then_capture_replays_match_the_oracle():
    import torch
    cases = [_case(10 + k) for k in range(3)]
    base_d, bias_d, blk_d = (to_dev(a) for a in cases[0])
    s = torch.cuda.Stream()
    native.xpress_reserve(N, B, V, stream=s)
    assert native.xpress_workspace_bytes() > 0
    g = torch.cuda.CUDAGraph()
    say("capture after reserve")
    with torch.cuda.graph(g, stream=s):
        native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V, stream=s)
    for rep in range(4):
        base, bias, blk0 = cases[rep % 3]
        base_d.copy_(to_dev(base))
        bias_d.copy_(to_dev(bias))
        blk_d.copy_(to_dev(blk0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(blk_d.cpu().numpy(), oracle_blk(base, bias, blk0, N, B, V, V, V)), rep


def test_graph_captured_before_growth_still_replays():
    """Capture at a small shape, then an eager call on the same stream that
    grows the key table (a two-pass plan with 1100 splits per row), then
    more device allocations; the captured graph still holds the old table,
    which was retired rather than freed, and its replays stay correct."""
    import torch
    base, bias, blk0 = _case(20)
    base_d, bias_d, blk_d = to_dev(base), to_dev(bias), to_dev(blk0)
    s = torch.cuda.Stream()
    native.xpress_reserve(N, B, V, stream=s)
    before = native.xpress_workspace_bytes()
    g = torch.cuda.CUDAGraph()
    say("capture before growth")
    with torch.cuda.graph(g, stream=s):
        native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V, stream=s)
    # the larger call: 120 rows x 1100 splits = 132000 table entries
    Nl, Bl, Vl = 8, 16, 300000
    gl = np.random.Generator(np.random.PCG64(21))
    rows_l = Nl * (Bl - 1)
    bl = workloads.f32_to_bf16_bits(gl.standard_normal((rows_l, Vl), dtype=np.float32))
    il = workloads.f32_to_bf16_bits(gl.standard_normal((rows_l, Vl), dtype=np.float32))
    blkl0 = np.full((Nl, Bl), -1, dtype=np.int64)
    with torch.cuda.stream(s):
        bl_d, il_d = to_dev(bl), to_dev(il)
    torch.cuda.synchronize()
    say("eager call that grows the table")
    with Plan(native.XPRESS_COMBINE_TWO_PASS, 1100, 64):
        blkl_d = to_dev(blkl0)
        native.xpress_add_argmax_to_blk(bl_d, il_d, blkl_d, Nl, Bl, Vl, Vl, Vl, stream=s)
        torch.cuda.synchronize()
    assert np.array_equal(blkl_d.cpu().numpy(), oracle_blk(bl, il, blkl0, Nl, Bl, Vl, Vl, Vl))
    grown = native.xpress_workspace_bytes()
    assert grown > before
    # fresh device memory of about the old table's size: with the old table
    # freed it could have landed there
    junk = [torch.full((65536,), -1, dtype=torch.int64, device="cuda") for _ in range(8)]
    for rep in range(3):
        blk_d.copy_(to_dev(blk0))
        torch.cuda.synchronize()
        say("replay after growth %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(blk_d.cpu().numpy(), oracle_blk(base, bias, blk0, N, B, V, V, V)), rep
    assert all(int((j != -1).sum()) == 0 for j in junk)
    native.xpress_release()
    assert native.xpress_workspace_bytes() == 0


def test_enomem_through_the_workspace_cap():
    import torch
    base, bias, blk0 = _case(30)
    base_d, bias_d, blk_d = to_dev(base), to_dev(bias), to_dev(blk0)
    torch.cuda.synchronize()
    native.xpress_set_workspace_limit(1024)
    say("calls under a 1 KiB workspace cap")
    with pytest.raises(native.XpressError) as ei:
        native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V)
    assert ei.value.status == native.XPRESS_ENOMEM
    with pytest.raises(native.XpressError) as ei:
        native.xpress_reserve(N, B, V)
    assert ei.value.status == native.XPRESS_ENOMEM
    torch.cuda.synchronize()
    assert np.array_equal(blk_d.cpu().numpy(), blk0)
    assert native.xpress_workspace_bytes() == 0
    # the single-workgroup plan needs no workspace and still runs under the cap
    Ns, Bs, Vs = 20, 16, 5000
    bs, is_, blks = _case_rows(Ns, Bs, Vs, 31)
    assert native.xpress_describe_plan(256, 256, Ns, Bs, Vs, Vs, Vs)["combine"] == "single"
    got = gpu_blk(to_dev(bs), to_dev(is_), blks, Ns, Bs, Vs, Vs, Vs)
    assert np.array_equal(got, oracle_blk(bs, is_, blks, Ns, Bs, Vs, Vs, Vs))
    native.xpress_set_workspace_limit(0)
    got = gpu_blk(base_d, bias_d, blk0, N, B, V, V, V)
    assert np.array_equal(got, oracle_blk(base, bias, blk0, N, B, V, V, V))


def _case_rows(n, b, v, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = n * (b - 1)
    base = workloads.f32_to_bf16_bits(g.standard_normal((rows, v), dtype=np.float32) * 3)
    bias = workloads.f32_to_bf16_bits(g.standard_normal((rows, v), dtype=np.float32))
    blk = np.full((n, b), -1, dtype=np.int64)
    blk[:, 0] = 5
    return base, bias, blk


def test_release_round_trip():
    base, bias, blk0 = _case(40)
    base_d, bias_d = to_dev(base), to_dev(bias)
    want = oracle_blk(base, bias, blk0, N, B, V, V, V)
    for k in range(3):
        say("release round trip %d" % k)
        assert np.array_equal(gpu_blk(base_d, bias_d, blk0, N, B, V, V, V), want)
        assert native.xpress_workspace_bytes() > 0
        native.xpress_release()
        assert native.xpress_workspace_bytes() == 0


def test_gemm_capture_without_a_sized_workspace_returns_ecapture():
    import torch
    rows_n, rows_b, v, r = 2, 8, 3000, 64
    g = np.random.Generator(np.random.PCG64(50))
    rows = rows_n * (rows_b - 1)
    base = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, v)) / 4.0).astype(np.float32))
    x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(rows, r)) / 8.0).astype(np.float32))
    wt = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(v, r)) / 8.0).astype(np.float32))
    blk0 = np.full((rows_n, rows_b), -1, dtype=np.int64)
    bd, xd, wd, blk_d = to_dev(base), to_dev(x), to_dev(wt), to_dev(blk0)
    marker = torch.zeros(2, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    say("gemm capture with an empty workspace")
    with torch.cuda.graph(cg, stream=s):
        with pytest.raises(native.XpressError) as ei:
            native.xpress_readout_gemm_argmax_to_blk(bd, xd, wd, blk_d, rows_n, rows_b, v, r, v,
                                                     stream=s)
        marker.add_(2)
    assert ei.value.status == native.XPRESS_ECAPTURE
    cg.replay()
    torch.cuda.synchronize()
    assert marker.cpu().tolist() == [2, 2]
    assert np.array_equal(blk_d.cpu().numpy(), blk0)
