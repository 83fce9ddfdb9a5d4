"""The oracle's pins must catch plausible mistakes in the oracle.

Each case below rebuilds oracle.c with one deliberate mistake (a wrong
comparison, a wrong rounding rule, a flushed subnormal, a wrong slot or row
mapping, an ignored stride), loads the mutant on the CPU and checks that at
least one pin fails on it.  Nothing here touches a GPU.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import exact_bf16
from test_oracle import ARGMAX_ROWS, GEMM_ROWS, NAN_ROWS, ROUNDING, TOPC_ROWS
from test_oracle_latent import latent_pins_pass
from vocab_wide_add_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

U16P = ctypes.POINTER(ctypes.c_uint16)
I64P = ctypes.POINTER(ctypes.c_int64)

MUTATIONS = {
    "last_max_wins": ("if (s > best) {", "if (s >= best) {"),
    "ties_round_up": ("m = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "m = lo + 1.0;"),
    "ties_round_down": ("m = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "m = lo;"),
    "truncate": ("if (frac > 0.5) {", "if (frac > 2.0) {"),
    "flush_subnormal_inputs": ("mag = ldexp((double)f, -133);", "mag = 0.0;"),
    "wrong_exponent_bias": ("mag = ldexp((double)(128 + f), e - 127 - 7);",
                            "mag = ldexp((double)(128 + f), e - 126 - 7);"),
    "overflow_saturates": ("return sign | 0x7F80; /* overflow to infinity */",
                           "return sign | 0x7F7F; /* overflow to infinity */"),
    "anchor_overwritten": ("blk[n * B + 1 + b] =", "blk[n * B + b] ="),
    "row_to_block_by_B": ("int64_t n = r / (B - 1);\n        int64_t b = r % (B - 1);",
                          "int64_t n = r / B;\n        int64_t b = r % (B - 1);"),
    "stride_ignored": ("oracle_add_argmax_row(base + r * stride_base_r,\n"
                       "                                                   bias + r * stride_bias_r, V);",
                       "oracle_add_argmax_row(base + r * V,\n"
                       "                                                   bias + r * V, V);"),
    "sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "topc_position_not_id": ("blk[n * B + 1 + j] = cand[r * C + best];",
                             "blk[n * B + 1 + j] = best;"),
    "topc_wrong_row": ("blk[n * B + 1 + j] = cand[r * C + best];",
                       "blk[n * B + 1 + j] = cand[best];"),
    "nan_at_first_index_wins": ("if (s > best) {", "if (s > best || v == 0) {"),
    "gemm_bias_dropped": ("oracle_bf16_sum(base_row[v], bias)", "oracle_bf16_sum(base_row[v], 0)"),
    "gemm_x_row_ignored": ("gemm_scan_row(base + r * stride_base_r, xd + r * R, wd, V, R)",
                           "gemm_scan_row(base + r * stride_base_r, xd, wd, V, R)"),
    "gemm_bias_unrounded": ("uint16_t bias = oracle_bf16_from_double(acc);",
                            "uint16_t bias = oracle_bf16_from_double(acc) | 1;"),
    "gemm_last_max_wins": ("if (sum > best) {", "if (sum >= best) {"),
    "gemm_w_row_stride": ("const double* wv = w + v * R;", "const double* wv = w + v;"),
    # latent stage
    "latent_prev_is_same_slot": ("int64_t tok = (b == 0) ? am1[n] : blk[n * B + b - 1];",
                                 "int64_t tok = (b == 0) ? am1[n] : blk[n * B + b];"),
    "latent_anchor_not_am1": ("int64_t tok = (b == 0) ? am1[n] : blk[n * B + b - 1];",
                              "int64_t tok = (b == 0) ? blk[n * B] : blk[n * B + b - 1];"),
    "latent_cache_dropped": ("double acc = oracle_bf16_to_double(xh[(n * B + b) * R + r]);",
                             "double acc = 0.0;"),
    "latent_wlat_transposed": ("acc += emb[k] * dlat[r * R + k];",
                               "acc += emb[k] * dlat[k * R + r];"),
    "latent_mixer_transposed": ("acc += dmix[(b * B + j) * R + r] * x[j * R + r];",
                                "acc += dmix[(j * B + b) * R + r] * x[j * R + r];"),
    "latent_mixer_causal_only": ("for (int64_t j = 0; j < B; ++j) {\n                    acc += dmix",
                                 "for (int64_t j = 0; j <= b; ++j) {\n                    acc += dmix"),
    "latent_ub_unrounded": ("ub[r] = oracle_bf16_to_double(oracle_bf16_from_double(u[b * R + r]));",
                            "ub[r] = u[b * R + r];"),
    "latent_gate_reads_up": ("g += ub[r] * dg[h * R + r];", "g += ub[r] * du[h * R + r];"),
    "latent_silu_sign": ("double f = g / (1.0 + exp(-g)) * v;",
                         "double f = g / (1.0 + exp(g)) * v;"),
    "latent_m_unrounded": ("m[h] = oracle_bf16_to_double(oracle_bf16_from_double(f));",
                           "m[h] = f;"),
    "latent_residual_dropped": ("double acc = u[b * R + r];\n                for (int64_t h",
                                "double acc = 0.0;\n                for (int64_t h"),
    "latent_residual_rounded": ("double acc = u[b * R + r];\n                for (int64_t h",
                                "double acc = ub[r];\n                for (int64_t h"),
    "latent_down_transposed": ("acc += m[h] * dd[r * H + h];", "acc += m[h] * dd[h * R + r];"),
    "latent_block_stride_B": ("int64_t row = n * (B - 1) + b - 1;", "int64_t row = n * B + b - 1;"),
}


def _bind(lib):
    lib.oracle_bf16_sum.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.oracle_bf16_sum.restype = ctypes.c_uint16
    lib.oracle_add_argmax_row.argtypes = [U16P, U16P, ctypes.c_int64]
    lib.oracle_add_argmax_row.restype = ctypes.c_int64
    lib.oracle_add_argmax_to_blk.argtypes = [U16P, U16P, I64P] + [ctypes.c_int64] * 5
    lib.oracle_add_argmax_to_blk.restype = ctypes.c_int
    lib.oracle_topc_argmax_to_blk.argtypes = [U16P, U16P, I64P, I64P] + [ctypes.c_int64] * 3
    lib.oracle_topc_argmax_to_blk.restype = ctypes.c_int
    lib.oracle_gemm_argmax_rows.argtypes = [U16P, U16P, U16P, I64P] + [ctypes.c_int64] * 5
    lib.oracle_gemm_argmax_rows.restype = ctypes.c_int
    DP = ctypes.POINTER(ctypes.c_double)
    lib.oracle_latent_pass.argtypes = [I64P, I64P] + [U16P] * 8 + [ctypes.c_int64] * 5 + [DP] * 6
    lib.oracle_latent_pass.restype = ctypes.c_int
    return lib


def _latent_caller(lib):
    """A latent-pass callable over a (possibly mutated) library.  The output
    buffer is padded to N*B*R so that a mutant writing past N*(B-1)*R stays
    inside memory it owns; only the first N*(B-1)*R elements are compared."""
    DP = ctypes.POINTER(ctypes.c_double)

    def call(blk, am1, xh, w1, wlat, mixl, wg, wu, wd, N, B, R, H, V):
        arrs = [np.ascontiguousarray(a) for a in (xh, w1, wlat, mixl, wg, wu, wd)]
        blk = np.ascontiguousarray(blk, dtype=np.int64)
        am1 = np.ascontiguousarray(am1, dtype=np.int64)
        out = np.zeros(N * B * R + 1, dtype=np.uint16)
        null = ctypes.cast(None, DP)
        rc = lib.oracle_latent_pass(blk.ctypes.data_as(I64P), am1.ctypes.data_as(I64P),
                                    *[a.ctypes.data_as(U16P) for a in arrs],
                                    out.ctypes.data_as(U16P), N, B, R, H, V,
                                    null, null, null, null, null, null)
        if rc != 0:
            raise ValueError("rejected")
        return out[:N * (B - 1) * R].reshape(N, B - 1, R)
    return call


def _build_mutant(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not unique/present" % name
    path_c = os.path.join(tmp_path, "mut.c")
    path_so = os.path.join(tmp_path, "libmut.so")
    open(path_c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-w", "-o", path_so, path_c, "-lm"], check=True)
    return _bind(ctypes.CDLL(path_so))


def _pins_pass(lib) -> bool:
    for a, b, e, _ in ROUNDING:
        if lib.oracle_bf16_sum(a, b) != e:
            return False
    for _, base, bias, idx, _ in ARGMAX_ROWS + NAN_ROWS:
        base = np.ascontiguousarray(base)
        bias = np.ascontiguousarray(bias)
        if lib.oracle_add_argmax_row(base.ctypes.data_as(U16P), bias.ctypes.data_as(U16P),
                                     base.size) != idx:
            return False
    g = np.random.Generator(np.random.PCG64(1))
    for _ in range(200):
        V = int(g.integers(1, 24))
        a = g.integers(0, 0x7F80, size=V).astype(np.uint16) | \
            (g.integers(0, 2, size=V).astype(np.uint16) << 15)
        b = g.integers(0, 0x7F80, size=V).astype(np.uint16) | \
            (g.integers(0, 2, size=V).astype(np.uint16) << 15)
        got = lib.oracle_add_argmax_row(a.ctypes.data_as(U16P), b.ctypes.data_as(U16P), V)
        if got != exact_bf16.first_argmax(a, b):
            return False
    for (N, B, V, pad) in [(3, 5, 77, 9), (5, 3, 4097, 64)]:
        base, bias, blk = workloads.planted(N, B, V, seed=V, pad=pad)
        anchors = blk[:, 0].copy()
        lib.oracle_add_argmax_to_blk(base.ctypes.data_as(U16P), bias.ctypes.data_as(U16P),
                                     blk.ctypes.data_as(I64P), N, B, V, V + pad, V + pad)
        want = (np.arange(N * (B - 1)) % V).reshape(N, B - 1)
        if not np.array_equal(blk[:, 1:], want) or not np.array_equal(blk[:, 0], anchors):
            return False
    for _, base, bias, cand, tok, _ in TOPC_ROWS:
        blk = np.array([[-3, -1]], dtype=np.int64)
        base, bias, cand = (np.ascontiguousarray(x) for x in (base, bias, cand))
        lib.oracle_topc_argmax_to_blk(base.ctypes.data_as(U16P), bias.ctypes.data_as(U16P),
                                      cand.ctypes.data_as(I64P), blk.ctypes.data_as(I64P),
                                      1, 2, base.size)
        if blk[0, 1] != tok or blk[0, 0] != -3:
            return False
    # two rows of two candidates: row 1's winner must come from row 1's ids
    base = np.array([0x3F80, 0x4000, 0x4000, 0x3F80], dtype=np.uint16)
    bias = np.zeros(4, dtype=np.uint16)
    cand = np.array([10, 11, 20, 21], dtype=np.int64)
    blk = np.full((1, 3), -1, dtype=np.int64)
    lib.oracle_topc_argmax_to_blk(base.ctypes.data_as(U16P), bias.ctypes.data_as(U16P),
                                  cand.ctypes.data_as(I64P), blk.ctypes.data_as(I64P), 1, 3, 2)
    if list(blk[0]) != [-1, 11, 20]:
        return False
    for _, x, w, base, idx, _ in GEMM_ROWS:
        V, R = w.shape
        out = np.empty(1, dtype=np.int64)
        x, w, base = (np.ascontiguousarray(t) for t in (x, w, base))
        lib.oracle_gemm_argmax_rows(base.ctypes.data_as(U16P), x.ctypes.data_as(U16P),
                                    w.ctypes.data_as(U16P), out.ctypes.data_as(I64P),
                                    0, 1, V, R, V)
        if out[0] != idx:
            return False
    # two rows whose x differ: row 1 must use its own x
    x = np.array([0x3F80, 0x0000, 0x0000, 0x3F80], dtype=np.uint16)      # [[1,0],[0,1]]
    w = np.array([0x3F80, 0x0000, 0x0000, 0x3F80], dtype=np.uint16)      # [[1,0],[0,1]]
    base = np.zeros(4, dtype=np.uint16)
    out = np.empty(2, dtype=np.int64)
    lib.oracle_gemm_argmax_rows(base.ctypes.data_as(U16P), x.ctypes.data_as(U16P),
                                w.ctypes.data_as(U16P), out.ctypes.data_as(I64P), 0, 2, 2, 2, 2)
    if list(out) != [0, 1]:
        return False
    try:
        if not latent_pins_pass(_latent_caller(lib)):
            return False
    except ValueError:
        return False
    return True


def test_unmutated_oracle_passes_the_pins(tmp_path):
    # the same harness on the real source must pass, or the mutants prove nothing
    src = open(SRC).read()
    path_c = os.path.join(tmp_path, "orig.c")
    path_so = os.path.join(tmp_path, "liborig.so")
    open(path_c, "w").write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", path_so, path_c, "-lm"], check=True)
    assert _pins_pass(_bind(ctypes.CDLL(path_so)))


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(str(tmp_path), name)
    assert not _pins_pass(lib), "pins did not catch mutation %r" % name
