"""The latent-stage acceptance test (tests/latent_bound.py) on the CPU.

The GPU parity test accepts an output when every element lies in the
propagated fp32 error interval around the oracle's exact value and at least
99% of the elements are bit-equal.  Here that check is run on outputs whose
provenance is known:
  * the oracle's own output and an fp32 evaluation of the stage with torch
    (sums in torch's order, bf16 roundings at the same three places) must
    pass;
  * outputs with a planted mistake -- the residual dropped, u or m left
    unrounded, the residual rounded -- must fail; and where the sums are
    exact (so the interval holds one value) one element off by one bf16 step
    must fail too.
"""
import numpy as np
import pytest
import torch

import latent_bound
import oracle
from vocab_wide_add_amd import workloads

W = workloads.LatentWorkload("bound_n6_b8_r128_h256_v500", 6, 8, 128, 256, 500, seed=50)
KEYS = ("blk", "am1", "xh", "w1", "wlat", "mixl", "wg", "wu", "wd")


def _f32(bits):
    return torch.from_numpy(latent_bound.values(bits).astype(np.float32))


def emulate(d, w, mistake=None):
    """The stage in fp32 with torch, with an optional planted mistake."""
    N, B, R = w.N, w.B, w.R
    toks = np.concatenate([d["am1"][:, None], d["blk"][:, :B - 1]], axis=1)
    x = _f32(d["xh"]) + _f32(d["w1"][toks]) @ _f32(d["wlat"]).T
    u = torch.einsum("bjr,njr->nbr", _f32(d["mixl"]), x)[:, 1:]
    ub = u if mistake == "ub_unrounded" else u.to(torch.bfloat16).float()
    g = ub @ _f32(d["wg"]).T
    v = ub @ _f32(d["wu"]).T
    f = g / (1 + torch.exp(-g)) * v
    m = f if mistake == "m_unrounded" else f.to(torch.bfloat16).float()
    res = {"residual_dropped": torch.zeros_like(u), "residual_rounded": ub}.get(mistake, u)
    o = (res + m @ _f32(d["wd"]).T).to(torch.bfloat16)
    return o.view(torch.int16).numpy().view(np.uint16).reshape(N, B - 1, R)


@pytest.fixture(scope="module")
def case():
    d = workloads.generate_latent(W)
    want, inter = oracle.latent_pass(*(d[k] for k in KEYS), W.N, W.B, W.R, W.H, W.V,
                                     intermediates=True)
    return d, want, inter


def _accepts(got, want, d, inter):
    ok, exact, _ = latent_bound.check(got, want, d, inter, W.B, W.R, W.H)
    return ok and exact >= 0.99


def test_oracle_output_is_accepted(case):
    d, want, inter = case
    ok, exact, _ = latent_bound.check(want, want, d, inter, W.B, W.R, W.H)
    assert ok and exact == 1.0


def test_fp32_evaluation_is_accepted(case):
    d, want, inter = case
    got = emulate(d, W)
    ok, exact, worst = latent_bound.check(got, want, d, inter, W.B, W.R, W.H)
    assert ok, worst
    assert exact >= 0.99


@pytest.mark.parametrize("mistake", ["residual_dropped", "ub_unrounded", "m_unrounded",
                                     "residual_rounded"])
def test_planted_mistakes_are_rejected(case, mistake):
    d, want, inter = case
    assert not _accepts(emulate(d, W, mistake), want, d, inter)


def test_one_step_off_is_rejected_where_the_sums_are_exact():
    """With x, u, g and v exact (the mlp_dyadic recipe) most intervals hold a
    single bf16 value: moving one such element by one step must fail, while
    the fp32 evaluation still passes."""
    w = workloads.LatentWorkload("bound_dyadic_n4_b8_r128_h256_v500", 4, 8, 128, 256, 500,
                                 seed=51, kind="mlp_dyadic")
    d = workloads.generate_latent(w)
    want, inter = oracle.latent_pass(*(d[k] for k in KEYS), w.N, w.B, w.R, w.H, w.V,
                                     intermediates=True)
    ok, exact, worst = latent_bound.check(emulate(d, w), want, d, inter, w.B, w.R, w.H, "gv")
    assert ok and exact >= 0.99, worst
    lo, hi = latent_bound.interval(d, inter, w.B, w.R, w.H, "gv")
    single = np.argwhere(lo == hi)
    assert len(single) > 0.8 * lo.size
    idx = tuple(single[0])
    bad = want.copy()
    bad[idx] = np.uint16(int(bad[idx]) + 1)
    ok, _, _ = latent_bound.check(bad, want, d, inter, w.B, w.R, w.H, "gv")
    assert not ok
