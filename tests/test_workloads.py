"""The seeded input generator: reproducible, shaped as stated, padded with
poison, anchors in range.  CPU only."""
import numpy as np
import pytest

from vocab_wide_add_amd import workloads

PAD_BITS = 0x42C8  # bf16 of +100


def test_five_workloads_shapes():
    w = workloads.WORKLOADS
    assert [(x.N, x.B, x.V, x.rows) for x in w.values()] == [
        (2, 4, 1000, 6), (8, 8, 32000, 56), (32, 16, 152064, 480),
        (32, 16, 151936, 480), (256, 16, 152064, 3840)]
    # the pages' ~146 MB of avoided bf16 logits at N = 32, V = 152k, B = 16
    pages = w["spike_n32_b16_v152064"]
    assert pages.rows * pages.V * 2 == 145_981_440
    ties = w["ties_strided_n32_b16_v151936"]
    assert (ties.stride_base, ties.stride_bias) == (151936 + 64, 151936 + 128)


@pytest.mark.parametrize("name", ["tiny_n2_b4_v1000", "small_n8_b8_v32000"])
def test_reproducible(name):
    w = workloads.WORKLOADS[name]
    a = workloads.generate(w)
    b = workloads.generate(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_rows_limit_is_a_prefix():
    w = workloads.WORKLOADS["small_n8_b8_v32000"]
    full = workloads.generate(w)
    part = workloads.generate(w, rows_limit=5)
    assert np.array_equal(full[0][:5], part[0])
    assert np.array_equal(full[1][:5], part[1])
    assert np.array_equal(full[2], part[2])


def test_padding_poison_and_anchors():
    w = workloads.WORKLOADS["ties_strided_n32_b16_v151936"]
    base, bias, blk = workloads.generate(w, rows_limit=16)
    assert base.shape == (16, w.stride_base) and bias.shape == (16, w.stride_bias)
    assert (base[:, w.V:] == PAD_BITS).all() and (bias[:, w.V:] == PAD_BITS).all()
    vals = (base[:, :w.V].astype(np.uint32) << 16).view(np.float32)
    assert vals.min() == -8 and vals.max() == 8 and (vals == np.round(vals)).all()
    assert blk.shape == (w.N, w.B)
    assert ((blk[:, 0] >= 0) & (blk[:, 0] < w.V)).all()
    assert (blk[:, 1:] == -1).all()


def test_spike_and_spread():
    w = workloads.WORKLOADS["spike_n32_b16_v152064"]
    base, bias, _ = workloads.generate(w, rows_limit=4)
    b = (base.astype(np.uint32) << 16).view(np.float32)
    s = (bias.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(b.std()) - 4.0) < 0.1 and abs(float(s.std()) - 0.5) < 0.02
    # the planted +20 stands far above a N(0, 4^2) row of this length
    assert (b.max(axis=1) > 18).all()


def test_planted_layout():
    base, bias, blk = workloads.planted(3, 5, 77, pad=9)
    assert base.shape == (12, 86) and (base[:, 77:] == PAD_BITS).all()
    for r in range(12):
        v = (base[r, :77].astype(np.uint32) << 16).view(np.float32)
        assert int(np.argmax(v)) == r % 77 and v.max() == 64.0


def test_generated_inputs_match_their_stored_digests():
    """SHA-256 of every benchmarked input (whole for the small workloads, a
    prefix of rows for the large ones) against tests/golden/workload_digests.json,
    written by tests/golden/make_workload_digests.py: a change in the
    generators, the conversions or the recipes fails here rather than
    silently changing the inputs."""
    import importlib.util
    import json
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_workload_digests",
                                                  os.path.join(here, "make_workload_digests.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(here, "workload_digests.json")) as f:
        stored = json.load(f)
    now = mod.digests()
    assert sorted(now) == sorted(stored)
    for key in stored:
        assert now[key] == stored[key], key
