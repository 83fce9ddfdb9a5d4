"""Several readout passes inside one captured HIP graph, each reading the
previous pass's blk in place.

The XPress kernels page runs a Jacobi pass as a few launches inside a captured
graph, and the next pass reads blk where the readout left it.  Here a pass is
the readout followed by a small scatter that knocks the pass's winners out of
base (sets them to -inf), so pass p finds every row's p-th best token.  The
oracle reproduces the same sequence on the host.  The graph is replayed
several times with eager work between replays, and every replay must give
the oracle's tokens -- which also checks that the split plans' workspaces
come back clean between passes inside one graph.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import Plan, say, to_dev
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

NEG_INF = 0xFF80


def oracle_passes(base, bias, blk0, N, B, V, S, passes):
    """Winners of each pass: readout, then the winners set to -inf in base."""
    base = base.copy()
    rows = N * (B - 1)
    out = []
    for _ in range(passes):
        blk = blk0.copy()
        oracle.add_argmax_to_blk(base, bias, blk, N, B, V, S, S)
        win = blk[:, 1:].reshape(-1)
        base[np.arange(rows), win] = NEG_INF
        out.append(blk)
    return out


@pytest.mark.parametrize("combine,splits", [(0, 0), (native.XPRESS_COMBINE_ATOMIC, 3),
                                            (native.XPRESS_COMBINE_TWO_PASS, 4),
                                            (native.XPRESS_COMBINE_BALANCED, 2)])
def test_graph_of_passes_reads_blk_in_place(combine, splits):
    import torch
    N, B, V, P = 8, 16, 20000, 5
    rows = N * (B - 1)
    g = np.random.Generator(np.random.PCG64(31 + combine))
    # integer-valued logits: the knocked-out winners are followed by ties
    base = workloads.f32_to_bf16_bits(g.integers(-6, 7, size=(rows, V)).astype(np.float32))
    bias = workloads.f32_to_bf16_bits(g.integers(-2, 3, size=(rows, V)).astype(np.float32))
    blk0 = np.full((N, B), -1, dtype=np.int64)
    blk0[:, 0] = g.integers(0, V, size=N)
    want = oracle_passes(base, bias, blk0, N, B, V, V, P)

    base_d = to_dev(base)
    bias_d = to_dev(bias)
    blk_d = to_dev(blk0)
    hist_d = torch.zeros((P, N, B), dtype=torch.int64, device="cuda")
    row_ids = torch.arange(rows, device="cuda")
    neg_inf = torch.tensor(NEG_INF - 65536, dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()
    with Plan(combine, splits, 256):
        native.xpress_reserve(N, B, V, stream=s)
        graph = torch.cuda.CUDAGraph()
        say("multipass capture combine=%d splits=%d" % (combine, splits))
        with torch.cuda.graph(graph, stream=s):
            for p in range(P):
                native.xpress_add_argmax_to_blk(base_d, bias_d, blk_d, N, B, V, V, V, stream=s)
                hist_d[p].copy_(blk_d)
                win = blk_d[:, 1:].reshape(-1)
                base_d.view(rows, V)[row_ids, win] = neg_inf
        for rep in range(3):
            base_d.copy_(to_dev(base))
            blk_d.copy_(to_dev(blk0))
            hist_d.fill_(-9)
            torch.cuda.synchronize()
            say("multipass replay %d" % rep)
            graph.replay()
            torch.cuda.synchronize()
            got = hist_d.cpu().numpy()
            for p in range(P):
                assert np.array_equal(got[p], want[p]), (rep, p)
            # eager work between replays
            native.xpress_add_argmax_to_blk(to_dev(base), bias_d, to_dev(blk0), N, B, V, V, V)
            torch.cuda.synchronize()
