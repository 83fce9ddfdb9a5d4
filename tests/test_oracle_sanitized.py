"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, -fno-sanitize-recover=all), run over its pins through a small driver
(tests/oracle_sanitize_driver.c) that allocates every buffer at exactly the
size a call may touch.  Any out-of-bounds access or undefined arithmetic
stops the driver; its answers must also equal the ordinary build's and the
pins' expected values.  CPU only; the sanitizers instrument host code."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import exact_bf16
import oracle
from test_oracle import ARGMAX_ROWS, GEMM_ROWS, NAN_ROWS, ROUNDING, TOPC_ROWS
from test_oracle_latent import latent_pins_pass
from vocab_wide_add_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("san") / "oracle_san")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return exe


def _run(exe, jobs):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], input="\n".join(jobs) + "\n", capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout.split("\n")[:len(jobs)]


def _ints(a):
    return " ".join(str(int(v)) for v in np.asarray(a).reshape(-1))


def test_sanitized_rounding_and_rows(driver):
    g = np.random.Generator(np.random.PCG64(77))
    pairs = [(a, b) for a, b, _, _ in ROUNDING]
    pairs += [(int(a), int(b)) for a, b in g.integers(0, 65536, size=(3000, 2))]
    jobs = ["sum %d %d" % p for p in pairs]
    out = _run(driver, jobs)
    for (a, b), o in zip(pairs, out):
        assert int(o) == oracle.bf16_sum(a, b), (a, b)
    for (a, b, e, why) in ROUNDING:
        assert int(out[pairs.index((a, b))]) == e, why
    rows = [(base, bias, idx) for _, base, bias, idx, _ in ARGMAX_ROWS + NAN_ROWS]
    for _ in range(300):
        V = int(g.integers(1, 40))
        a = g.integers(0, 0x7F80, size=V).astype(np.uint16) | \
            (g.integers(0, 2, size=V).astype(np.uint16) << 15)
        b = g.integers(0, 0x7F80, size=V).astype(np.uint16) | \
            (g.integers(0, 2, size=V).astype(np.uint16) << 15)
        rows.append((a, b, exact_bf16.first_argmax(a, b)))
    out = _run(driver, ["row %d %s %s" % (len(a), _ints(a), _ints(b)) for a, b, _ in rows])
    for (a, b, idx), o in zip(rows, out):
        assert int(o) == idx


def test_sanitized_blk_layouts(driver):
    cases = [(3, 5, 77, 9), (5, 3, 4097, 64), (2, 1, 10, 0), (1, 2, 1, 0), (4, 2, 33, 7)]
    jobs, wants = [], []
    for (N, B, V, pad) in cases:
        base, bias, blk = workloads.planted(N, B, V, seed=V, pad=pad)
        S = V + pad
        want = blk.copy()
        if N * (B - 1) > 0:
            oracle.add_argmax_to_blk(base, bias, want, N, B, V, S, S)
        jobs.append("blk %d %d %d %d %d %s %s %s" % (N, B, V, S, S, _ints(base), _ints(bias),
                                                     _ints(blk)))
        wants.append(want)
    for o, want in zip(_run(driver, jobs), wants):
        vals = [int(t) for t in o.split()]
        assert vals[0] == 0 and vals[1:] == list(want.reshape(-1))


def test_sanitized_topc_and_gemm(driver):
    jobs, wants = [], []
    for _, base, bias, cand, tok, _ in TOPC_ROWS:
        jobs.append("topc %d %s %s %s" % (base.size, _ints(base), _ints(bias), _ints(cand)))
        wants.append(("topc", tok))
    g = np.random.Generator(np.random.PCG64(78))
    gemm = [(x, w, base, idx) for _, x, w, base, idx, _ in GEMM_ROWS]
    for _ in range(40):
        V, R = int(g.integers(1, 30)), int(g.integers(1, 20))
        x = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=R) / 8.0).astype(np.float32))
        w = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=(V, R)) / 8.0).astype(np.float32))
        base = workloads.f32_to_bf16_bits((g.integers(-8, 9, size=V) / 4.0).astype(np.float32))
        gemm.append((x, w, base, int(oracle.gemm_argmax_rows(base, x, w, [0], V, R, V)[0])))
    for x, w, base, idx in gemm:
        V, R = w.shape
        jobs.append("gemm %d %d %s %s %s" % (V, R, _ints(x), _ints(w), _ints(base)))
        wants.append(("gemm", idx))
    for o, (kind, want) in zip(_run(driver, jobs), wants):
        vals = [int(t) for t in o.split()]
        if kind == "topc":
            assert vals == [0, -7, want]
        else:
            assert vals == [0, want, 0, want]


def test_sanitized_latent_pins(driver):
    """Every latent-stage pin (golden cases, exact special cases, invariants)
    through the sanitized build."""
    def call(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, N, B, R, H, V):
        job = "latent %d %d %d %d %d %s" % (N, B, R, H, V, " ".join(
            _ints(a) for a in (blk, am1, xh, w1, wlat, mixl, wg, wu, wd)))
        vals = [int(t) for t in _run(driver, [job])[0].split()]
        if vals[0] != 0:
            raise ValueError("rejected")
        return np.array(vals[1:], dtype=np.uint16).reshape(N, B - 1, R)
    assert latent_pins_pass(call)
