"""Writes tests/golden/workload_digests.json: SHA-256 digests of the seeded
synthetic inputs (vocab_wide_add_amd.workloads), so that a change in numpy's
or torch's generators or conversions, or in the recipes, shows up as a
failing test instead of silently changing every benchmarked input.

The small workloads are digested whole; the large ones by a prefix of rows
(the generator draws any prefix alone), which keeps the check to seconds.

Usage: python tests/golden/make_workload_digests.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from vocab_wide_add_amd import workloads  # noqa: E402

PREFIX_ROWS = 32


def sha(a) -> str:
    import numpy as np
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def digests() -> dict:
    out = {}
    for name, w in workloads.WORKLOADS.items():
        lim = None if w.rows <= 64 else PREFIX_ROWS
        base, bias, blk = workloads.generate(w, rows_limit=lim)
        out["readout/" + name] = {"rows": base.shape[0], "base": sha(base), "bias": sha(bias),
                                  "blk": sha(blk)}
    for name in ("topc_n32_b16_c64", "topc_ties_n32_b16_c256"):
        w = workloads.TOPC_WORKLOADS[name]
        base_c, bias_c, cand, blk = workloads.generate_topc(w)
        out["topc/" + name] = {"base_c": sha(base_c), "bias_c": sha(bias_c), "cand": sha(cand),
                               "blk": sha(blk)}
    for name in ("gemm_tiny_n2_b4_v1000_r64", "gemm_dyadic_n32_b16_v152064_r256",
                 "gemm_normal_n32_b16_v152064_r256", "gemm_negative_n32_b16_v152064_r256"):
        w = workloads.GEMM_WORKLOADS[name]
        lim = None if w.rows <= 64 else PREFIX_ROWS
        base, x, wt, blk = workloads.generate_gemm(w, rows_limit=lim)
        out["gemm/" + name] = {"rows": base.shape[0], "base": sha(base), "x": sha(x),
                               "w": sha(wt), "blk": sha(blk)}
    for name in ("latent_tiny_n2_b4_r64_h128_v1000", "latent_n32_b16_r256_h512_v152064"):
        w = workloads.LATENT_WORKLOADS[name]
        d = workloads.generate_latent(w)
        out["latent/" + name] = {k: sha(d[k]) for k in sorted(d)}
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "workload_digests.json")
    with open(path, "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)
