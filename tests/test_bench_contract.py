"""The benchmark's host-side contract, on the CPU: one GPU only, a JSON line
with the fields the roofline and traffic reports need, and traffic figures
reported only while the kernel code they were counted on is unchanged."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2


@pytest.mark.skipif(gpu_available(), reason="checks the no-GPU exit")
def test_no_gpu_exits_with_a_message():
    r = _run(["--steps", "1", "--warmup", "0"])
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr


def test_code_digest_ignores_comments_only(tmp_path):
    b = _bench()
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n/* block */\n")
    c = tmp_path / "c.hip"
    c.write_text("// another comment\nint f(int x)\n{\n    return x + 1;\n}\n")
    d = tmp_path / "d.hip"
    d.write_text("int f(int x) { return x + 2; }\n")
    assert b.source_digest(str(a)) == b.source_digest(str(c))
    assert b.source_digest(str(a)) != b.source_digest(str(d))


def test_traffic_records_are_reported_only_for_their_code():
    """A committed counter record is reported while the kernel code it was
    counted on is unchanged, and not otherwise; its figures add up."""
    b = _bench()
    assert b.traffic_for("no_such_workload") is None
    for name, src in (("spike_n32_b16_v152064", b.SRC),
                      ("gemm_normal_n32_b16_v152064_r256", b.GEMM_SRC)):
        with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % name)) as f:
            t = json.load(f)
        fresh = t["kernel_source_sha256"] == b.source_digest(src)
        assert b.traffic_for(name, src) == (t["hbm_bytes_per_launch"] if fresh else None)
        assert t["hbm_bytes_per_launch"] == t["hbm_fetch_bytes_per_launch"] + \
            t["hbm_write_bytes_per_launch"]
        ratio = t["hbm_bytes_per_launch"] / t["algorithmic_bytes_per_launch"]
        assert abs(ratio - t["traffic_over_algorithmic"]) < 1e-3


def test_result_line_fields():
    b = _bench()
    out = b.result_line("m", "w", {"workload": "w"}, bytes_per_call=4_000_000, rows=10,
                        steps=100, warmup=5, wall=1e-3, region_gpu=0.9e-3,
                        durs=[9e-6] * 100, launches=1, traffic=None)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in out, k
    r = out["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # 4 MB per launch over 9 us per launch of GPU time
    assert abs(r["achieved"] - 4_000_000 / 9e-6 / 1e9) < 1.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # whole-job rate over the wall clock: 100 steps of 4 MB in 1 ms
    assert abs(out["value"] - 400.0) < 1e-6
    assert out["n_gpus"] == 1 and out["steps"] == 100
    k = out["kernel_us_event_pairs"]
    assert k["min"] <= k["p10"] <= k["p50"] <= k["p90"]


def test_digest_covers_every_source_of_the_kernel(tmp_path):
    """A code change in any file the kernel is built from (a shared header
    included) invalidates the counter records; comments anywhere do not."""
    b = _bench()
    main = tmp_path / "k.hip"
    main.write_text("int k() { return h(); }\n")
    h1 = tmp_path / "h.h"
    h1.write_text("int h() { return 1; }\n")
    base = b.source_digest([str(main), str(h1)])
    h1.write_text("// note\nint h() { return 1; }\n")
    assert b.source_digest([str(main), str(h1)]) == base
    h1.write_text("int h() { return 2; }\n")
    assert b.source_digest([str(main), str(h1)]) != base
    # the readout's and the GEMM readout's lists name their shared sources
    for name in ("device_common.h", "host_common.h", "xpress_argmax.h", "xpress_argmax.hip"):
        assert any(p.endswith(name) for p in b.SRC), name
        assert any(p.endswith(name) for p in b.GEMM_SRC), name
    assert any(p.endswith("readout_gemm.hip") for p in b.GEMM_SRC)


def test_cpu_baseline_legs_on_a_small_workload():
    """The CPU baseline reports the all-cores median of three runs, the
    single-thread median of three, the core count and the CPU model, and its
    answers are the oracle's."""
    import numpy as np
    import oracle
    from vocab_wide_add_amd import workloads
    b = _bench()
    w = workloads.WORKLOADS["tiny_n2_b4_v1000"]
    base, bias, _ = workloads.generate(w)
    res, rows, ans = b.cpu_baseline(base, bias, w, 0.6)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["cores"] >= 1
    assert len(res["runs"]) == 3 and len(res["single_thread"]["runs"]) == 3
    assert sorted(res["runs"])[1] == res["value"]
    assert sorted(res["single_thread"]["runs"])[1] == res["single_thread"]["value"]
    assert isinstance(res["cpu_model"], str) and res["cpu_model"]
    assert 1 <= rows <= w.rows
    want = oracle.add_argmax_rows(base, bias, 0, rows, w.V, w.stride_base, w.stride_bias)
    assert np.array_equal(ans, want)


def test_result_line_labels_the_traffic_source():
    """roofline.traffic comes from a committed counter record, and the line
    says so (or says that no record matches the kernel's source)."""
    import bench
    args = ("m", "spike_n32_b16_v152064", {"workload": "w"}, 291962880, 480, 20, 5,
            20 * 45e-6, 20 * 44.6e-6, [44.6e-6] * 20, 1)
    out = bench.result_line(*args, 292059898)
    assert out["roofline"]["traffic"] == 292059898
    assert "profiles/traffic_spike_n32_b16_v152064.json" in out["traffic_source"]
    out = bench.result_line(*args, None)
    assert out["roofline"]["traffic"] is None
    assert out["traffic_source"] == "no counter record for this kernel source"
