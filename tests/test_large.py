"""Maximum-size cases on the GPU: buffers past 2^31 elements, so every row
offset needs 64-bit arithmetic.

Inputs are drawn on the device from a seeded torch generator (the host would
need tens of GB to hold them); the rows the oracle checks -- the first and
last rows, the rows on either side of element 2^31 and a seeded random
sample -- are copied back and recomputed on the CPU.
"""
import numpy as np
import pytest

from conftest import gpu_available
from gpu_util import say, ORACLE_THREADS
import latent_bound
import oracle
from vocab_wide_add_amd import native, workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

N, B, V = 1024, 16, 152064
ROWS = N * (B - 1)   # 15360 rows: 2.34e9 elements per [rows, V] buffer


def sample_rows(rows, V, seed, k=24):
    edge = (1 << 31) // V
    picks = {0, 1, rows - 1, rows - 2, edge - 1, edge, edge + 1}
    g = np.random.Generator(np.random.PCG64(seed))
    picks |= set(int(r) for r in g.integers(0, rows, size=k))
    return sorted(r for r in picks if 0 <= r < rows)


def host_rows(t, rows):
    import torch
    idx = torch.tensor(rows, dtype=torch.int64, device=t.device)
    return t.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def big_inputs():
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    base = (torch.randn((ROWS, V), device="cuda", generator=g) * 4.0).to(torch.bfloat16)
    bias = (torch.randn((ROWS, V), device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    torch.cuda.synchronize()
    yield base, bias
    del base, bias
    torch.cuda.empty_cache()


def test_readout_past_2g_elements(big_inputs):
    import torch
    base, bias = big_inputs
    assert base.numel() > (1 << 31)
    blk = torch.full((N, B), -1, dtype=torch.int64, device="cuda")
    blk[:, 0] = torch.arange(N, device="cuda") * 7
    say("readout N=%d rows=%d V=%d" % (N, ROWS, V))
    native.xpress_add_argmax_to_blk(base.view(torch.int16), bias.view(torch.int16), blk, N, B,
                                    V, V, V)
    torch.cuda.synchronize()
    got = blk.cpu().numpy()
    assert np.array_equal(got[:, 0], np.arange(N) * 7)
    rows = sample_rows(ROWS, V, 1)
    hb, hi = host_rows(base, rows), host_rows(bias, rows)
    want = oracle.add_argmax_rows_threaded(hb, hi, len(rows), V, V, V, ORACLE_THREADS)
    flat = got[:, 1:].reshape(-1)
    assert np.array_equal(flat[rows], want)


def test_readout_gemm_past_2g_elements(big_inputs):
    """Dyadic x and w (k/8): every fp32 partial sum is exact, so the sampled
    rows must match the oracle bit for bit."""
    import torch
    base, _ = big_inputs
    R = 256
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    x = (torch.randint(-8, 9, (ROWS, R), device="cuda", generator=g).float() / 8).to(torch.bfloat16)
    w = (torch.randint(-8, 9, (V, R), device="cuda", generator=g).float() / 8).to(torch.bfloat16)
    blk = torch.full((N, B), -1, dtype=torch.int64, device="cuda")
    say("readout with in-place bias N=%d rows=%d V=%d R=%d" % (N, ROWS, V, R))
    native.xpress_readout_gemm_argmax_to_blk(base.view(torch.int16), x.view(torch.int16),
                                             w.view(torch.int16), blk, N, B, V, R, V)
    torch.cuda.synchronize()
    got = blk.cpu().numpy()[:, 1:].reshape(-1)
    rows = sample_rows(ROWS, V, 2, k=9)
    hb = host_rows(base, rows)
    hx = host_rows(x, rows)
    hw = w.view(torch.int16).cpu().numpy().view(np.uint16)
    want = oracle.gemm_argmax_rows(hb, hx, hw, range(len(rows)), V, R, V,
                                   threads=ORACLE_THREADS)
    assert np.array_equal(got[rows], want)


def test_latent_2048_blocks_sampled():
    """2048 blocks (30720 latent rows, the staged kernels); blocks are
    independent, so the oracle recomputes a sample of them alone."""
    import torch
    w = workloads.LatentWorkload("latent_n2048_b16_r256_h512_v152064", 2048, 16, 256, 512,
                                 152064, seed=41)
    d = workloads.generate_latent(w)
    keys = ("blk", "am1", "xh", "w1", "wlat", "mixl", "wg", "wu", "wd")
    dd = {k: torch.from_numpy(d[k].view(np.int16) if d[k].dtype == np.uint16 else d[k]).cuda()
          for k in keys}
    out = torch.empty((w.N, w.B - 1, w.R), dtype=torch.int16, device="cuda")
    say("latent N=%d" % w.N)
    native.xpress_latent_pass(*(dd[k] for k in keys), out, w.N, w.B, w.R, w.H, w.V)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    blocks = sorted({0, 1, 7, 8, 1023, 1024, 2046, 2047} |
                    set(int(b) for b in np.random.default_rng(3).integers(0, w.N, 8)))
    sub = dict(d)
    for k in ("blk", "am1", "xh"):
        sub[k] = np.ascontiguousarray(d[k][blocks])
    want, inter = oracle.latent_pass(*(sub[k] for k in keys), len(blocks), w.B, w.R, w.H, w.V,
                                     intermediates=True, threads=ORACLE_THREADS)
    ok, exact, worst = latent_bound.check(got[blocks], want, sub, inter, w.B, w.R, w.H)
    say("  exact fraction %.5f" % exact)
    assert ok, worst
    assert exact >= 0.99, exact
