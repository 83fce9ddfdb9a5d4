"""Seeded synthetic inputs for the fused add + argmax readout.

This module holds only random-number plumbing and buffer layout: it draws
values, converts them to bf16 storage and lays rows out with their strides.  It
contains none of the readout's arithmetic (no sums, no rounding of sums, no
argmax), so the GPU path and the CPU oracle can both be fed from it.

Shapes follow the XPress kernels page: a pass drafts B-1 slots in each of N
blocks, the vocabulary is about 152k wide, and the materialised logits the
fused readout avoids come to about 146 MB at N = 32, which at 2 bytes per bf16
and V = 152064 pins B = 16 (480 draft rows).

Recipe: ``numpy.random.SeedSequence(seed).spawn(3)`` gives three independent
PCG64 streams -- one for base, one for bias, one for ids -- so that the first
rows of a workload can be drawn without drawing the rest.  Draws:
  1. base stream: ``rows x V`` values in row-major order -- float32 standard
     normals times sigma, or integers uniform on the closed range [lo, hi];
  2. bias stream: the same for bias, with its own sigma or range;
  3. id stream: for workloads with a spike, one vocabulary id per row,
     uniform on [0, V) (``spike`` is added to base at that id in float32,
     before rounding to bf16); then the anchors, one id per block, uniform on
     [0, V), stored in blk[:, 0].
Float32 values become bf16 with torch's round-to-nearest-even conversion on
the CPU; integer values in [-8, 8] are exact in bf16.  Rows are laid out with
their row strides; every element between V and the stride (including after
the last row) holds the poison value ``pad`` so that any read past V changes
the answer.  blk slots 1..B-1 start at -1 so that a missing write shows.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    B: int
    V: int
    seed: int
    base_dist: Tuple  # ("normal", sigma) or ("int", lo, hi)
    bias_dist: Tuple
    spike: Optional[float] = None
    base_pad: int = 0  # row stride = V + pad (elements)
    bias_pad: int = 0
    pad_value: float = 100.0

    @property
    def rows(self) -> int:
        return self.N * (self.B - 1)

    @property
    def stride_base(self) -> int:
        return self.V + self.base_pad

    @property
    def stride_bias(self) -> int:
        return self.V + self.bias_pad

    @property
    def bytes_read(self) -> int:
        """Algorithmic bytes of one readout: two bf16 streams of rows x V."""
        return self.rows * self.V * 4


# The five synthetic workloads.  The names state what each one is.
WORKLOADS = {
    w.name: w
    for w in [
        # 6 rows, V not a multiple of any chunk width.
        Workload("tiny_n2_b4_v1000", 2, 4, 1000, 0, ("normal", 4.0), ("normal", 0.5)),
        # 56 rows of a 32k vocabulary.
        Workload("small_n8_b8_v32000", 8, 8, 32000, 1, ("normal", 3.0), ("normal", 1.0)),
        # The readout shape the pages size: 480 rows of a 152064 vocabulary,
        # one +20 spike per row.
        Workload("spike_n32_b16_v152064", 32, 16, 152064, 2, ("normal", 4.0),
                 ("normal", 0.5), spike=20.0),
        # Integer values in [-8, 8]: exact ties everywhere; padded row strides
        # with +100 poison in the padding.
        Workload("ties_strided_n32_b16_v151936", 32, 16, 151936, 3, ("int", -8, 8),
                 ("int", -8, 8), base_pad=64, bias_pad=128),
        # 3840 rows; bias wide enough that bf16 rounding of the sum often
        # decides the winner.
        Workload("large_n256_b16_v152064", 256, 16, 152064, 4, ("normal", 4.0),
                 ("normal", 2.0)),
    ]
}

# The workload the benchmark times by default (the pages' shape).
BENCH_WORKLOAD = "spike_n32_b16_v152064"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's CPU conversion (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _draw(g: np.random.Generator, dist: Tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
        x *= np.float32(dist[1])
        return x
    if kind == "int":
        lo, hi = dist[1], dist[2]
        return g.integers(lo, hi + 1, size=shape).astype(np.float32)
    raise ValueError("unknown distribution %r" % (dist,))


def _lay_out(bits: np.ndarray, stride: int, pad_bits: int) -> np.ndarray:
    rows, V = bits.shape
    out = np.full((rows, stride), pad_bits, dtype=np.uint16)
    out[:, :V] = bits
    return out


def generate(w: Workload, rows_limit: Optional[int] = None):
    """Build one workload on the host.

    Returns ``(base, bias, blk)``: ``base`` is a uint16 array of shape
    ``[rows, stride_base]`` holding bf16 bit patterns, ``bias`` likewise with
    ``stride_bias``, and ``blk`` an int64 ``[N, B]`` array with the anchors in
    column 0 and -1 elsewhere.  ``rows_limit`` draws only the first rows;
    each buffer has its own stream filled row-major, so those rows are
    identical to the full workload's first rows.
    """
    s_base, s_bias, s_ids = np.random.SeedSequence(w.seed).spawn(3)
    g_ids = np.random.Generator(np.random.PCG64(s_ids))
    rows, V = w.rows, w.V
    keep = rows if rows_limit is None else min(rows, rows_limit)
    base = _draw(np.random.Generator(np.random.PCG64(s_base)), w.base_dist, (keep, V))
    if w.spike is not None:
        ids = g_ids.integers(0, V, size=rows)[:keep]
        base[np.arange(keep), ids] += np.float32(w.spike)
    anchors = g_ids.integers(0, V, size=w.N)
    pad_bits = int(f32_to_bf16_bits(np.array([w.pad_value], dtype=np.float32))[0])
    base_bits = _lay_out(f32_to_bf16_bits(base), w.stride_base, pad_bits)
    del base
    bias = _draw(np.random.Generator(np.random.PCG64(s_bias)), w.bias_dist, (keep, V))
    bias_bits = _lay_out(f32_to_bf16_bits(bias), w.stride_bias, pad_bits)
    del bias
    blk = np.full((w.N, w.B), -1, dtype=np.int64)
    blk[:, 0] = anchors
    return base_bits, bias_bits, blk


def planted(N: int, B: int, V: int, seed: int = 0, pad: int = 0):
    """Rows whose unique maximum sits at v = r mod V (r = draft row index).

    Every element is a bf16 in [-4, 4) drawn on the grid of multiples of 1/16
    (exact in bf16, and so are their sums); row r gets base = 64 at v = r mod V,
    which no other element of the row can reach.  The expected readout is then
    ``blk[n, 1 + b] = (n*(B-1) + b) mod V`` in closed form.
    """
    g = np.random.Generator(np.random.PCG64(seed))
    rows = N * (B - 1)
    base = (g.integers(-64, 64, size=(rows, V)) / 16.0).astype(np.float32)
    bias = (g.integers(-64, 64, size=(rows, V)) / 16.0).astype(np.float32)
    if rows:
        base[np.arange(rows), np.arange(rows) % V] = 64.0
    pad_bits = int(f32_to_bf16_bits(np.array([100.0], dtype=np.float32))[0])
    base_bits = _lay_out(f32_to_bf16_bits(base), V + pad, pad_bits)
    bias_bits = _lay_out(f32_to_bf16_bits(bias), V + pad, pad_bits)
    blk = np.full((N, B), -1, dtype=np.int64)
    blk[:, 0] = g.integers(0, V, size=N)
    return base_bits, bias_bits, blk


# ---------------------------------------------------------------------------
# Top-C readout inputs: per draft row, C candidates with their base logits,
# refiner bias and vocabulary ids, all [N*(B-1), C] contiguous.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class TopCWorkload:
    name: str
    N: int
    B: int
    C: int
    seed: int
    vocab: int = 152064
    ties: bool = False  # integer-valued logits: many exact ties

    @property
    def rows(self) -> int:
        return self.N * (self.B - 1)

    @property
    def bytes_read(self) -> int:
        """Algorithmic bytes of one readout: two bf16 values per candidate
        plus the winner's 8-byte id per row."""
        return self.rows * (self.C * 4 + 8)


TOPC_WORKLOADS = {
    w.name: w
    for w in [
        TopCWorkload("topc_n32_b16_c64", 32, 16, 64, 10),
        TopCWorkload("topc_n32_b16_c256", 32, 16, 256, 11),
        TopCWorkload("topc_n32_b16_c1024", 32, 16, 1024, 12),
        TopCWorkload("topc_n32_b16_c4096", 32, 16, 4096, 13),
        TopCWorkload("topc_ties_n32_b16_c256", 32, 16, 256, 14, ties=True),
    ]
}


def generate_topc(w: TopCWorkload):
    """Top-C inputs shaped like a real candidate list.

    Recipe (``SeedSequence(seed).spawn(2)``: a logits stream and an id
    stream): for every row, a full vocabulary of base logits is drawn,
    N(0, 4^2) in float32 (or integers uniform on [-3, 3] for the tie
    workload); the C largest become the candidates -- their ids, in
    descending order of base logit, form cand, and their values base_c.  The
    refiner bias on the candidates is N(0, 1^2) (integers on [-3, 3] for the
    tie workload).  Anchors are uniform on [0, vocab).  Returns
    ``(base_c, bias_c, cand, blk)`` with blk's draft slots at -1.
    """
    s_val, s_ids = np.random.SeedSequence(w.seed).spawn(2)
    g = np.random.Generator(np.random.PCG64(s_val))
    gi = np.random.Generator(np.random.PCG64(s_ids))
    rows, C, V = w.rows, w.C, w.vocab
    base_c = np.empty((rows, C), dtype=np.float32)
    cand = np.empty((rows, C), dtype=np.int64)
    for r in range(rows):
        if w.ties:
            full = g.integers(-3, 4, size=V).astype(np.float32)
        else:
            full = g.standard_normal(V, dtype=np.float32) * np.float32(4.0)
        top = np.argpartition(-full, C - 1)[:C]
        top = top[np.argsort(-full[top], kind="stable")]
        cand[r] = top
        base_c[r] = full[top]
    if w.ties:
        bias_c = g.integers(-3, 4, size=(rows, C)).astype(np.float32)
    else:
        bias_c = g.standard_normal((rows, C), dtype=np.float32)
    blk = np.full((w.N, w.B), -1, dtype=np.int64)
    blk[:, 0] = gi.integers(0, V, size=w.N)
    return f32_to_bf16_bits(base_c), f32_to_bf16_bits(bias_c), cand, blk


# ---------------------------------------------------------------------------
# Readout with the bias computed in place: base [rows, V], the refiner
# latent x [rows, R] and the head weight w [V, R], all bf16.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class GemmWorkload:
    name: str
    N: int
    B: int
    V: int
    R: int
    seed: int
    dyadic: bool  # x, w on the grid k/8, |k| <= 8: every fp32 partial sum is exact
    base_mean: float = 0.0  # mean of base; negative for log-probability-like logits

    @property
    def rows(self) -> int:
        return self.N * (self.B - 1)

    @property
    def bytes_read(self) -> int:
        """Algorithmic HBM bytes of one call: base (2 B per logit) and the
        head weight (2 B per element, read once); x is 2*rows*R."""
        return self.rows * self.V * 2 + self.V * self.R * 2 + self.rows * self.R * 2

    @property
    def flops(self) -> int:
        return 2 * self.rows * self.V * self.R


GEMM_WORKLOADS = {
    w.name: w
    for w in [
        GemmWorkload("gemm_tiny_n2_b4_v1000_r64", 2, 4, 1000, 64, 20, True),
        GemmWorkload("gemm_small_n8_b8_v32000_r256", 8, 8, 32000, 256, 21, True),
        GemmWorkload("gemm_dyadic_n32_b16_v152064_r256", 32, 16, 152064, 256, 22, True),
        GemmWorkload("gemm_normal_n32_b16_v152064_r256", 32, 16, 152064, 256, 23, False),
        GemmWorkload("gemm_normal_n1_b16_v152064_r256", 1, 16, 152064, 256, 24, False),
        # every logit negative (base ~ N(-20, 4^2)): log-probability-like rows
        GemmWorkload("gemm_negative_n32_b16_v152064_r256", 32, 16, 152064, 256, 25, False,
                     base_mean=-20.0),
    ]
}

GEMM_BENCH_WORKLOAD = "gemm_normal_n32_b16_v152064_r256"


def generate_gemm(w: GemmWorkload, rows_limit: Optional[int] = None):
    """Inputs of the readout with in-place bias.

    Recipe (``SeedSequence(seed).spawn(4)``: base, x, w and id streams):
    base ~ N(base_mean, 4^2) in float32 rounded to bf16, [rows, V]; for the dyadic
    workloads x and w are integers uniform on [-8, 8] divided by 8 (exact in
    bf16; every product is a multiple of 1/64 of magnitude <= 1, so any fp32
    partial sum over R <= 4096 terms is exact and the bias is order-free);
    otherwise x ~ N(0, 1) and w ~ N(0, 1/R) (the bias is then ~N(0, 1)).
    Anchors uniform on [0, V).  Returns ``(base, x, w, blk)`` as uint16 bf16
    patterns ([rows, V], [rows, R], [V, R]) and int64 blk with draft slots
    at -1.  ``rows_limit`` draws only the first rows of base and x.
    """
    s_base, s_x, s_w, s_ids = np.random.SeedSequence(w.seed).spawn(4)
    keep = w.rows if rows_limit is None else min(w.rows, rows_limit)
    gb = np.random.Generator(np.random.PCG64(s_base))
    base = gb.standard_normal((keep, w.V), dtype=np.float32) * np.float32(4.0)
    if w.base_mean:
        base = base + np.float32(w.base_mean)
    gx = np.random.Generator(np.random.PCG64(s_x))
    gw = np.random.Generator(np.random.PCG64(s_w))
    if w.dyadic:
        x = gx.integers(-8, 9, size=(keep, w.R)).astype(np.float32) / np.float32(8.0)
        wt = gw.integers(-8, 9, size=(w.V, w.R)).astype(np.float32) / np.float32(8.0)
    else:
        x = gx.standard_normal((keep, w.R), dtype=np.float32)
        wt = gw.standard_normal((w.V, w.R), dtype=np.float32) * np.float32(1.0 / np.sqrt(w.R))
    gi = np.random.Generator(np.random.PCG64(s_ids))
    blk = np.full((w.N, w.B), -1, dtype=np.int64)
    blk[:, 0] = gi.integers(0, w.V, size=w.N)
    return f32_to_bf16_bits(base), f32_to_bf16_bits(x), f32_to_bf16_bits(wt), blk


# ---------------------------------------------------------------------------
# Latent stage of one pass: per block the previous slot's token ids, the
# hidden cache, and the synthetic weights of the embedding, the projection
# W_lat, the folded causal mixer and the SwiGLU MLP.
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class LatentWorkload:
    name: str
    N: int
    B: int
    R: int
    H: int
    V: int
    seed: int
    # "causal": mixer = I + L on and below the diagonal (the folded form
    #           L * tril + I), zero above;
    # "full":   mixer = I + L everywhere (checks that every slot is summed);
    # "exact":  dyadic values and wg = wu = 0, so every fp32 sum is exact,
    #           the MLP adds exactly 0 and the output is bf16(u) with many
    #           exact ties;
    # "mlp_dyadic": wlat = 0 and mixer = I, so u = xh, with xh, wg, wu on
    #           coarse dyadic grids: x, u, g and v are exact in fp32 and only
    #           the SwiGLU, m and the down projection round.
    kind: str = "causal"

    @property
    def rows(self) -> int:
        """Latent rows written: slots 1..B-1 of every block."""
        return self.N * (self.B - 1)

    @property
    def weight_bytes(self) -> int:
        """W_lat, the mixer and the three MLP matrices, bf16."""
        return 2 * (self.R * self.R + self.B * self.B * self.R + 3 * self.H * self.R)

    @property
    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes of one pass: the weights once, per block the
        ids (8 B per slot plus am1), the hidden cache and the gathered
        embedding rows (2 B per channel per slot), and the bf16 output."""
        per_block = 8 * (self.B + 1) + 2 * self.B * self.R * 2 + 2 * (self.B - 1) * self.R
        return self.weight_bytes + self.N * per_block

    @property
    def flops(self) -> int:
        """Multiply-adds times two: the projection for every slot, the mixer,
        and the MLP (gate, up, down) for the slots that are read out."""
        proj = self.N * self.B * self.R * self.R
        mix = self.N * self.B * self.B * self.R
        mlp = self.rows * 3 * self.H * self.R
        return 2 * (proj + mix + mlp)


LATENT_WORKLOADS = {
    w.name: w
    for w in [
        LatentWorkload("latent_tiny_n2_b4_r64_h128_v1000", 2, 4, 64, 128, 1000, 30, "full"),
        LatentWorkload("latent_small_n8_b8_r128_h256_v32000", 8, 8, 128, 256, 32000, 31),
        LatentWorkload("latent_ragged_n5_b12_r256_h512_v1000", 5, 12, 256, 512, 1000, 32),
        LatentWorkload("latent_b32_n3_r128_h256_v1000", 3, 32, 128, 256, 1000, 33),
        LatentWorkload("latent_n1_b16_r256_h512_v152064", 1, 16, 256, 512, 152064, 34),
        LatentWorkload("latent_n64_b16_r256_h512_v152064", 64, 16, 256, 512, 152064, 35),
        LatentWorkload("latent_n32_b16_r256_h512_v152064", 32, 16, 256, 512, 152064, 39),
        LatentWorkload("latent_n256_b16_r256_h512_v152064", 256, 16, 256, 512, 152064, 36),
        LatentWorkload("latent_exact_n64_b16_r256_h512_v152064", 64, 16, 256, 512, 152064,
                       37, "exact"),
        LatentWorkload("latent_mlp_dyadic_n64_b16_r256_h512_v152064", 64, 16, 256, 512,
                       152064, 38, "mlp_dyadic"),
    ]
}

LATENT_BENCH_WORKLOAD = "latent_n256_b16_r256_h512_v152064"

# One whole pass: the latent stage feeding the readout with in-place bias
# (the latent rows are the readout matmul's x; blk is read and written in
# place), as (latent workload, readout workload) of the same N, B, R and V.
PASS_WORKLOADS = {
    "pass_n32_b16_r256_h512_v152064": ("latent_n32_b16_r256_h512_v152064",
                                       "gemm_normal_n32_b16_v152064_r256"),
    "pass_n1_b16_r256_h512_v152064": ("latent_n1_b16_r256_h512_v152064",
                                      "gemm_normal_n1_b16_v152064_r256"),
}
PASS_BENCH_WORKLOAD = "pass_n32_b16_r256_h512_v152064"


def generate_latent(w: LatentWorkload):
    """Inputs of one latent pass, as a dict of numpy arrays.

    Recipe (``SeedSequence(seed).spawn(4)``: id, cache, embedding and
    layer-weight streams):
      ids    blk [N, B] and am1 [N], uniform on [0, V) (int64);
      cache  xh [N, B, R] ~ N(0, 1);
      embed  w1 [V, R] ~ N(0, 1), then wlat [R, R] ~ N(0, 1/R);
      layer  L [B, B, R] ~ N(0, 1/(4B)), then wg, wu [H, R] ~ N(0, 1/R) and
             wd [R, H] ~ N(0, 1/H); the mixer is I + L, with L zeroed above
             the diagonal for "causal".
    For "exact": xh = 1 + k/128 with k uniform on [-64, 127]; w1 = k/16 and
    wlat = k/16 with |k| <= 4 and <= 2; L = k/4 with |k| <= 2 below the
    diagonal (zero on and above it); wg = wu = 0; wd ~ N(0, 1/H).  Every
    projection sum is then a multiple of 2^-8, every mixer sum a multiple of
    2^-10, all far inside fp32's 24 bits.
    For "mlp_dyadic": xh = k/8 with |k| <= 16, wlat = 0, mixer = I,
    wg = wu = k/64 with |k| <= 8, wd ~ N(0, 1/H) (w1 as usual): every gate and
    up product is a multiple of 2^-9 of magnitude <= 1/4, so with R <= 1024
    every partial sum is a multiple of 2^-9 below 2^8, exact in fp32.
    Float values become bf16 with round-to-nearest-even (torch, on the CPU).
    Weight layouts are out-major (one row per output unit).
    """
    N, B, R, H, V = w.N, w.B, w.R, w.H, w.V
    s_ids, s_xh, s_emb, s_layer = np.random.SeedSequence(w.seed).spawn(4)
    gi = np.random.Generator(np.random.PCG64(s_ids))
    blk = gi.integers(0, V, size=(N, B)).astype(np.int64)
    am1 = gi.integers(0, V, size=N).astype(np.int64)
    gx = np.random.Generator(np.random.PCG64(s_xh))
    ge = np.random.Generator(np.random.PCG64(s_emb))
    gl = np.random.Generator(np.random.PCG64(s_layer))
    below = np.tril(np.ones((B, B), dtype=np.float32), -1)[:, :, None]
    eye = np.eye(B, dtype=np.float32)[:, :, None]
    if w.kind == "exact":
        xh = 1.0 + gx.integers(-64, 128, size=(N, B, R)).astype(np.float32) / np.float32(128)
        w1 = ge.integers(-4, 5, size=(V, R)).astype(np.float32) / np.float32(16)
        wlat = ge.integers(-2, 3, size=(R, R)).astype(np.float32) / np.float32(16)
        L = gl.integers(-2, 3, size=(B, B, R)).astype(np.float32) / np.float32(4)
        mixl = eye + L * below
        wg = np.zeros((H, R), dtype=np.float32)
        wu = np.zeros((H, R), dtype=np.float32)
        wd = gl.standard_normal((R, H), dtype=np.float32) / np.float32(np.sqrt(H))
    elif w.kind == "mlp_dyadic":
        xh = gx.integers(-16, 17, size=(N, B, R)).astype(np.float32) / np.float32(8)
        w1 = ge.standard_normal((V, R), dtype=np.float32)
        wlat = np.zeros((R, R), dtype=np.float32)
        mixl = np.broadcast_to(eye, (B, B, R)).copy()
        wg = gl.integers(-8, 9, size=(H, R)).astype(np.float32) / np.float32(64)
        wu = gl.integers(-8, 9, size=(H, R)).astype(np.float32) / np.float32(64)
        wd = gl.standard_normal((R, H), dtype=np.float32) / np.float32(np.sqrt(H))
    else:
        xh = gx.standard_normal((N, B, R), dtype=np.float32)
        w1 = ge.standard_normal((V, R), dtype=np.float32)
        wlat = ge.standard_normal((R, R), dtype=np.float32) / np.float32(np.sqrt(R))
        L = gl.standard_normal((B, B, R), dtype=np.float32) / np.float32(np.sqrt(4 * B))
        if w.kind == "causal":
            L = L * (below + eye)
        elif w.kind != "full":
            raise ValueError("unknown latent workload kind %r" % w.kind)
        mixl = eye + L
        wg = gl.standard_normal((H, R), dtype=np.float32) / np.float32(np.sqrt(R))
        wu = gl.standard_normal((H, R), dtype=np.float32) / np.float32(np.sqrt(R))
        wd = gl.standard_normal((R, H), dtype=np.float32) / np.float32(np.sqrt(H))
    return {
        "blk": blk, "am1": am1,
        "xh": f32_to_bf16_bits(xh), "w1": f32_to_bf16_bits(w1),
        "wlat": f32_to_bf16_bits(wlat), "mixl": f32_to_bf16_bits(mixl),
        "wg": f32_to_bf16_bits(wg), "wu": f32_to_bf16_bits(wu), "wd": f32_to_bf16_bits(wd),
    }
