"""Pins of the latent-stage oracle against facts that do not come from it.

The latent stage (XPress kernels page, "_xpress_latent_kernel") is pinned by
  * hand-derived outputs (tests/golden/latent_cases.txt): the rounding points
    (u before the MLP, the SwiGLU product, the output), the tie rule, the sign
    of the gate, which token each slot reads, the projection's and the MLP
    matrices' orientation and the per-channel mixer;
  * the MLP switched off (wg = wu = 0, so g = v = 0 and the MLP adds exactly
    0): the output is then bf16 of the projection and the full mixer, which
    is computed here in exact rational arithmetic and rounded by the
    exact-search rounding of tests/exact_bf16.py;
  * the embedding and the mixer switched off (wlat = 0, mixer = I, so u = xh):
    the output is then the SwiGLU MLP alone, computed with numpy matmuls and
    scipy's logistic function, its two roundings done by exact search;
  * invariants that hold for any weights: the last slot's token is never
    read, a slot's token only changes later slots, and blocks are independent
    (permuting blocks permutes the outputs).
test_oracle_mutations.py checks that these pins catch plausible mistakes.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import exact_bf16
import oracle
from vocab_wide_add_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex(field):
    return np.array([int(t, 16) for t in field.split()], dtype=np.uint16)


def load_latent_cases():
    cases = []
    with open(os.path.join(GOLDEN, "latent_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split(";", 13)]
            name, dims, blk, am1 = parts[:4]
            N, B, R, H, V = (int(t) for t in dims.split())
            xh, w1, wlat, mixl, wg, wu, wd, out = (_hex(p) for p in parts[4:12])
            cases.append(dict(
                name=name, N=N, B=B, R=R, H=H, V=V,
                blk=np.array([int(t) for t in blk.split()], dtype=np.int64).reshape(N, B),
                am1=np.array([int(t) for t in am1.split()], dtype=np.int64),
                xh=xh.reshape(N, B, R), w1=w1.reshape(V, R), wlat=wlat.reshape(R, R),
                mixl=mixl.reshape(B, B, R), wg=wg.reshape(H, R), wu=wu.reshape(H, R),
                wd=wd.reshape(R, H), out=out.reshape(N, B - 1, R), why=parts[13]))
    return cases


LATENT_CASES = load_latent_cases()


def _bits(rng, shape, scale):
    return workloads.f32_to_bf16_bits(
        rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def _values(bits):
    """Exact values of bf16 patterns as a float64 array (every bf16 is exact)."""
    return np.vectorize(lambda h: float(exact_bf16.value(int(h))), otypes=[np.float64])(bits)


def random_inputs(seed, N, B, R, H, V, causal=False):
    """Random small inputs; the mixer is full unless ``causal`` zeroes it
    above the diagonal."""
    rng = np.random.default_rng(seed)
    d = dict(
        blk=rng.integers(0, V, size=(N, B)).astype(np.int64),
        am1=rng.integers(0, V, size=N).astype(np.int64),
        xh=_bits(rng, (N, B, R), 1.0), w1=_bits(rng, (V, R), 1.0),
        wlat=_bits(rng, (R, R), 1 / np.sqrt(R)), mixl=_bits(rng, (B, B, R), 0.5),
        wg=_bits(rng, (H, R), 1 / np.sqrt(R)), wu=_bits(rng, (H, R), 1 / np.sqrt(R)),
        wd=_bits(rng, (R, H), 1 / np.sqrt(H)))
    if causal:
        d["mixl"][np.triu_indices(B, 1)] = 0
    return d


def run(call, d, N, B, R, H, V):
    return call(d["blk"], d["am1"], d["xh"], d["w1"], d["wlat"], d["mixl"], d["wg"],
                d["wu"], d["wd"], N, B, R, H, V)


def oracle_call(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, N, B, R, H, V):
    return oracle.latent_pass(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, N, B, R, H, V)


# --- the pins, each a predicate over a latent-pass callable ------------------

def golden_ok(call):
    for c in LATENT_CASES:
        got = run(call, c, c["N"], c["B"], c["R"], c["H"], c["V"])
        if not np.array_equal(got, c["out"]):
            return False
    return True


def no_mlp_expected(d, N, B, R, H):
    """bf16 of the exact projection and full mixer (the MLP adds 0)."""
    val = lambda h: exact_bf16.value(int(h))  # noqa: E731
    wlat = [[val(d["wlat"][r, k]) for k in range(R)] for r in range(R)]
    out = np.zeros((N, B - 1, R), dtype=np.uint16)
    for n in range(N):
        toks = [int(d["am1"][n])] + [int(t) for t in d["blk"][n, :B - 1]]
        x = []
        for b in range(B):
            emb = [val(h) for h in d["w1"][toks[b]]]
            x.append([val(d["xh"][n, b, r]) + sum(emb[k] * wlat[r][k] for k in range(R))
                      for r in range(R)])
        for b in range(1, B):
            for r in range(R):
                u = sum(val(d["mixl"][b, j, r]) * x[j][r] for j in range(B))
                out[n, b - 1, r] = exact_bf16.round_exact(Fraction(u))
    return out


def no_mlp_ok(call, seed=5, N=3, B=4, R=6, H=3, V=9):
    d = random_inputs(seed, N, B, R, H, V)
    d["wg"][:] = 0
    d["wu"][:] = 0
    return np.array_equal(run(call, d, N, B, R, H, V), no_mlp_expected(d, N, B, R, H))


def mlp_only_expected(d, N, B, R, H):
    """u = xh; out = bf16(u + bf16(g * logistic(g) * v) @ wd.T)."""
    rnd = np.vectorize(lambda x: exact_bf16.round_exact(Fraction(float(x))), otypes=[np.uint16])
    u = _values(d["xh"])[:, 1:, :]
    g = u @ _values(d["wg"]).T
    v = u @ _values(d["wu"]).T
    m = _values(rnd(g * scipy.special.expit(g) * v))
    return rnd(u + m @ _values(d["wd"]).T)


def mlp_only_ok(call, seed=6, N=2, B=3, R=8, H=5, V=4):
    d = random_inputs(seed, N, B, R, H, V)
    d["wlat"][:] = 0
    d["mixl"][:] = 0
    for b in range(B):
        d["mixl"][b, b, :] = 0x3F80
    return np.array_equal(run(call, d, N, B, R, H, V), mlp_only_expected(d, N, B, R, H))


def invariants_ok(call, seed=7, N=3, B=5, R=4, H=3, V=11):
    d = random_inputs(seed, N, B, R, H, V, causal=True)
    base = run(call, d, N, B, R, H, V)
    # the last slot's token is never read
    e = {k: v.copy() for k, v in d.items()}
    e["blk"][:, B - 1] = (e["blk"][:, B - 1] + 1) % V
    if not np.array_equal(run(call, e, N, B, R, H, V), base):
        return False
    # slot s's token is read by slot s+1 only: outputs of slots 1..s stay,
    # slot s+1's changes
    for s in range(B - 1):
        e = {k: v.copy() for k, v in d.items()}
        e["blk"][1, s] = (e["blk"][1, s] + 3) % V
        got = run(call, e, N, B, R, H, V)
        if not np.array_equal(got[:, :s], base[:, :s]) or np.array_equal(got[1, s], base[1, s]):
            return False
        if not np.array_equal(got[[0, 2]], base[[0, 2]]):
            return False
    # blocks are independent: permuting them permutes the outputs
    perm = np.array([2, 0, 1])
    e = {k: v.copy() for k, v in d.items()}
    for k in ("blk", "am1", "xh"):
        e[k] = np.ascontiguousarray(d[k][perm])
    if not np.array_equal(run(call, e, N, B, R, H, V), base[perm]):
        return False
    return True


def latent_pins_pass(call) -> bool:
    return golden_ok(call) and no_mlp_ok(call) and mlp_only_ok(call) and invariants_ok(call)


# --- the tests -----------------------------------------------------------------

@pytest.mark.parametrize("case", LATENT_CASES, ids=[c["name"] for c in LATENT_CASES])
def test_golden_latent_case(case):
    got = run(oracle_call, case, case["N"], case["B"], case["R"], case["H"], case["V"])
    assert np.array_equal(got, case["out"]), (case["why"], got, case["out"])


def test_no_mlp_is_exact_projection_and_mixer():
    assert no_mlp_ok(oracle_call)
    # a second, larger draw with a full (non-causal) mixer
    assert no_mlp_ok(oracle_call, seed=15, N=2, B=6, R=8, H=2, V=30)


def test_mlp_only_is_library_swiglu():
    assert mlp_only_ok(oracle_call)
    assert mlp_only_ok(oracle_call, seed=16, N=3, B=5, R=16, H=24, V=2)


def test_invariants():
    assert invariants_ok(oracle_call)


def test_intermediates_are_consistent():
    d = random_inputs(8, 2, 4, 8, 6, 10)
    out, it = oracle.latent_pass(d["blk"], d["am1"], d["xh"], d["w1"], d["wlat"], d["mixl"],
                                 d["wg"], d["wu"], d["wd"], 2, 4, 8, 6, 10, intermediates=True)
    rnd = np.vectorize(lambda x: exact_bf16.round_exact(Fraction(float(x))), otypes=[np.uint16])
    assert np.array_equal(rnd(it["o"]), out)
    g, v = it["g"], it["v"]
    np.testing.assert_allclose(it["f"], g * scipy.special.expit(g) * v, rtol=1e-13, atol=1e-300)


def test_rejects_bad_ids_and_sizes():
    d = random_inputs(9, 2, 3, 4, 2, 5)
    bad = dict(d, blk=d["blk"].copy())
    bad["blk"][1, 0] = 5
    with pytest.raises(ValueError):
        run(oracle_call, bad, 2, 3, 4, 2, 5)
    bad = dict(d, am1=np.array([0, -1], dtype=np.int64))
    with pytest.raises(ValueError):
        run(oracle_call, bad, 2, 3, 4, 2, 5)


def test_workload_recipes_match_their_kind():
    w = workloads.LATENT_WORKLOADS["latent_tiny_n2_b4_r64_h128_v1000"]
    d = workloads.generate_latent(w)
    assert d["mixl"].shape == (w.B, w.B, w.R) and (d["mixl"][0, 1:] != 0).any()  # full mixer
    w = workloads.LATENT_WORKLOADS["latent_small_n8_b8_r128_h256_v32000"]
    d = workloads.generate_latent(w)
    assert not np.triu(_values(d["mixl"][:, :, 0]), 1).any()  # causal mixer
    assert ((0 <= d["blk"]) & (d["blk"] < w.V)).all() and ((0 <= d["am1"]) & (d["am1"] < w.V)).all()
    w = workloads.LATENT_WORKLOADS["latent_exact_n64_b16_r256_h512_v152064"]
    d = workloads.generate_latent(w)
    assert not d["wg"].any() and not d["wu"].any()


def test_vector_rounding_matches_the_pinned_scalar_rounding():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 40, 2000),
                        [0.0, -0.0, 1e300, -1e300, 2.0 ** -134, 3 * 2.0 ** -134, 1.00390625]])
    got = oracle.bf16_from_double_many(x)
    assert got.shape == x.shape
    assert all(int(g) == oracle.bf16_from_double(float(v)) for g, v in zip(got, x))
    # and the exact-search rounding agrees on the finite ones
    for g, v in zip(got[:200], x[:200]):
        assert int(g) == exact_bf16.round_exact(Fraction(float(v)))
