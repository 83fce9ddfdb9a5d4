"""Whole passes through the C-ABI: the latent stage (reading blk) feeding the
readout with in-place bias (writing blk in place), chained pass after pass,
eagerly and captured in one HIP graph.

Each stage is checked against the oracle by its own tests; here the chain is
checked for what composing them adds: both entry points share the stream's
workspace, blk is read by one stage and rewritten by the next, and a graph
of several passes must replay exactly the eager sequence (every kernel is
deterministic), replay after replay, with the anchors untouched.
"""
import numpy as np
import pytest

from gpu_util import say
from conftest import gpu_available
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KEYS = ("blk", "am1", "xh", "w1", "wlat", "mixl", "wg", "wu", "wd")


def _inputs(N, B, R, H, V, seed):
    lw = workloads.LatentWorkload("pass_test", N, B, R, H, V, seed=seed)
    d = workloads.generate_latent(lw)
    gw = workloads.GemmWorkload("pass_test", N, B, V, R, seed + 1, False)
    base, _, wt, _ = workloads.generate_gemm(gw)
    return d, base, wt


def _device(d, base, wt):
    import torch
    dev = {k: torch.from_numpy(np.ascontiguousarray(
        d[k].view(np.int16) if d[k].dtype == np.uint16 else d[k])).cuda() for k in KEYS}
    dev["base"] = torch.from_numpy(base.view(np.int16)).cuda()
    dev["wt"] = torch.from_numpy(wt.view(np.int16)).cuda()
    return dev


def _pass(dev, lat, N, B, R, H, V, stream):
    native.xpress_latent_pass(*(dev[k] for k in KEYS), lat, N, B, R, H, V, stream=stream)
    native.xpress_readout_gemm_argmax_to_blk(dev["base"], lat, dev["wt"], dev["blk"], N, B, V,
                                             R, V, stream=stream)


@pytest.mark.parametrize("N,B,R,H,V", [(6, 16, 256, 512, 3000),    # 90 rows: two waves
                                       (40, 12, 128, 256, 2000),   # 440 rows: eight waves
                                       (3, 8, 64, 128, 1000)])     # 21 rows: one wave
def test_pass_chain_graph_replays_eager(N, B, R, H, V):
    import torch
    P = 3
    d, base, wt = _inputs(N, B, R, H, V, seed=500 + N + B + R)
    s = torch.cuda.Stream()

    # eager: 2P passes, blk and the last latent rows kept after P and 2P
    dev = _device(d, base, wt)
    lat = torch.empty((N, B - 1, R), dtype=torch.int16, device="cuda")
    native.xpress_latent_reserve(N, B, R, H, stream=s)
    say("pass chain eager N=%d B=%d R=%d H=%d V=%d" % (N, B, R, H, V))
    want = []
    for rep in range(2):
        for _ in range(P):
            _pass(dev, lat, N, B, R, H, V, s)
        torch.cuda.synchronize()
        want.append((dev["blk"].cpu().numpy().copy(), lat.cpu().numpy().copy()))
    first = want[0][0]
    assert np.array_equal(first[:, 0], d["blk"][:, 0]), "anchor slot changed"
    assert ((first[:, 1:] >= 0) & (first[:, 1:] < V)).all()

    # graph of P passes on fresh buffers; the workspace is sized by one
    # eager pass on the capture stream on scratch copies of blk first
    dev = _device(d, base, wt)
    lat = torch.empty((N, B - 1, R), dtype=torch.int16, device="cuda")
    warm = dict(dev)
    warm["blk"] = dev["blk"].clone()
    _pass(warm, lat, N, B, R, H, V, s)
    torch.cuda.synchronize()
    say("pass chain capture P=%d" % P)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(P):
            _pass(dev, lat, N, B, R, H, V, s)
    for rep in range(2):
        say("pass chain replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays
        _ = (dev["xh"].float() * 2).sum().item()
        got_blk = dev["blk"].cpu().numpy()
        got_lat = lat.cpu().numpy()
        assert np.array_equal(got_blk, want[rep][0]), rep
        assert np.array_equal(got_lat, want[rep][1]), rep
