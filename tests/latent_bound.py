"""Per-element acceptance interval for the GPU latent stage (tests only).

The GPU forms every sum of the latent stage in fp32, in an order of its own
(the matrix cores' accumulation, partial sums over K split across waves), and
rounds to bf16 at the same three places as the definition: u before the MLP,
the SwiGLU product, and the output.  Its output therefore differs from the
oracle's (the exact values, rounded) only through fp32 rounding of sums, and
through the bf16 roundings those small differences can tip.  This module
bounds that difference element by element from the oracle's exact
intermediates and the magnitudes of the inputs:

  * a sum of n terms t_i formed in fp32 in any order is within
    gamma(n) * sum |t_i| of the exact sum, gamma(n) = n*u / (1 - n*u); u is
    taken as 2^-23 (twice fp32's unit roundoff, so the bound also covers an
    accumulator that truncates instead of rounding to nearest);
  * bf16 rounding is monotone, so a value known to lie in [a - e, a + e]
    rounds into [bf16(a - e), bf16(a + e)];
  * silu(g) * v changes by at most 1.1 * |v| per unit of g (the derivative of
    g * sigmoid(g) lies in [-0.1, 1.1]) and |g| per unit of v, and its fp32
    evaluation (exp, add, reciprocal, two multiplies) adds at most 64 fp32 ulps of
    relative error, plus 1e-30 absolute for underflow.

The stages, with X, U, G, V, F, O the oracle's exact values:
  E1 = gamma(R+1) * (|xh| + |emb| @ |wlat|^T)                  (x)
  E2 = sum_j |L| E1_j + gamma(B) * sum_j |L| (|X_j| + E1_j)      (u)
  ub in [bf16(U - E2), bf16(U + E2)]  ->  D3 = its distance from bf16(U)
  EG = D3 @ |wg|^T + gamma(R) * A3 @ |wg|^T, EV likewise          (g, v)
  E5 = 1.1 (|V| + EV) EG + (|G| + EG) EV + rounding               (f)
  m in [bf16(F - E5), bf16(F + E5)]   ->  D5, A5
  E6 = E2 + D5 @ |wd|^T + gamma(H+1) (|U| + E2 + A5 @ |wd|^T)     (o)
  accepted output: any bf16 in [bf16(O - E6), bf16(O + E6)].
"""
from __future__ import annotations

import numpy as np

import oracle

UNIT = 2.0 ** -23
F32_ULP = 2.0 ** -24


def gamma(n: int) -> float:
    return n * UNIT / (1.0 - n * UNIT)


def values(bits) -> np.ndarray:
    """Exact values of bf16 patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def rounded(x) -> np.ndarray:
    """Values of the bf16 roundings (to nearest even) of float64 values."""
    return values(oracle.bf16_from_double_many(x))


def interval(d, inter, B: int, R: int, H: int, exact_through: str = ""):
    """(lo, hi): float64 arrays [N, B-1, R] bounding the GPU output's value.

    exact_through names the last stage whose fp32 sums are exact for the
    inputs at hand (every partial sum representable in fp32, so any
    summation order gives the exact value): "" (none), "u" (x and u), or
    "gv" (x, u, g and v).  The workload recipes state when that holds."""
    N = d["blk"].shape[0]
    toks = np.concatenate([d["am1"].reshape(N, 1), d["blk"][:, :B - 1]], axis=1)
    emb = np.abs(values(d["w1"][toks]))                        # [N, B, R]
    wlat = np.abs(values(d["wlat"]))
    S1 = np.abs(values(d["xh"])) + emb @ wlat.T
    E1 = gamma(R + 1) * S1
    if exact_through in ("u", "gv"):
        E1 = 0.0 * S1
    L = np.abs(values(d["mixl"]))                               # [B, B, R]
    X = np.abs(inter["x"])
    E2 = (np.einsum("bjr,njr->nbr", L, E1)
          + gamma(B) * np.einsum("bjr,njr->nbr", L, X + E1))[:, 1:, :]
    if exact_through in ("u", "gv"):
        E2 = 0.0 * E2
    U = inter["u"][:, 1:, :]
    UB = rounded(U)
    lo3, hi3 = rounded(U - E2), rounded(U + E2)
    D3 = np.maximum(hi3 - UB, UB - lo3)
    A3 = np.maximum(np.abs(lo3), np.abs(hi3))
    wg, wu, wd = (np.abs(values(d[k])) for k in ("wg", "wu", "wd"))
    EG = D3 @ wg.T + gamma(R) * (A3 @ wg.T)
    EV = D3 @ wu.T + gamma(R) * (A3 @ wu.T)
    if exact_through == "gv":
        EG, EV = 0.0 * EG, 0.0 * EV
    G, V, F = inter["g"], inter["v"], inter["f"]
    prop = 1.1 * (np.abs(V) + EV) * EG + (np.abs(G) + EG) * EV
    E5 = prop + 64 * F32_ULP * (np.abs(F) + prop) + 1e-30 * (1 + (np.abs(G) + EG) * (np.abs(V) + EV))
    M = rounded(F)
    lo5, hi5 = rounded(F - E5), rounded(F + E5)
    D5 = np.maximum(hi5 - M, M - lo5)
    A5 = np.maximum(np.abs(lo5), np.abs(hi5))
    E6 = E2 + D5 @ wd.T + gamma(H + 1) * (np.abs(U) + E2 + A5 @ wd.T)
    O = inter["o"]
    return rounded(O - E6), rounded(O + E6)


def check(gpu_bits, oracle_bits, d, inter, B: int, R: int, H: int, exact_through: str = ""):
    """Returns (ok, exact_fraction, worst) for a GPU output [N, B-1, R]."""
    lo, hi = interval(d, inter, B, R, H, exact_through)
    got = values(gpu_bits)
    inside = (got >= lo) & (got <= hi)
    exact = float(np.mean(np.asarray(gpu_bits) == np.asarray(oracle_bits)))
    bad = np.argwhere(~inside)
    worst = None
    if bad.size:
        idx = tuple(bad[0])
        worst = dict(index=idx, got=float(got[idx]), lo=float(lo[idx]), hi=float(hi[idx]),
                     oracle=float(values(np.asarray(oracle_bits)[idx])))
    return bool(inside.all()), exact, worst
