// latent.hip -- the latent stage of one Jacobi pass on gfx950 (wave64, MFMA).
//
// What it computes (XPress kernels page, module description and
// "_xpress_latent_kernel"): for every block n and slot b of a block of B,
//
//   prev[b] = am1[n] for b = 0, blk[n, b-1] otherwise
//   x[b, :] = xh[n, b, :] + w1[prev[b], :] @ wlat^T           fp32
//   u[b, r] = sum_j mixl[b, j, r] * x[j, r]                    fp32
//   g = bf16(u) @ wg^T,  v = bf16(u) @ wu^T                    fp32
//   m = bf16(g * sigmoid(g) * v)
//   out[n, b-1, :] = bf16(u + m @ wd^T)                        b = 1 .. B-1
//
// with bf16 inputs and weights stored out-major (one row per output unit).
//
// Design.  The page fuses the whole stage into one program per block, so one
// compute unit streams all ~1 MB of weights for its block; at small N that is
// a latency chain through a single CU.  Here the stage is three MFMA kernels
// in stream order, each spreading its weight slice over many workgroups:
//
//   mix   per (whole blocks of x-rows, 32 channels): the gathered embeddings
//         times W_lat on v_mfma_f32_32x32x16_bf16, summed with the hidden
//         cache in LDS, then the folded mixer per channel from an LDS copy of
//         its slice of mixl.  Writes u (fp32) and bf16(u) for the slots that
//         are read out.
//   gate  per (rows, 32 hidden units): bf16(u) times wg and wu;
//         m = bf16(silu(g) * v).
//   down  per (rows, 32 channels): m times wd plus the residual u, rounded
//         to bf16 into the output.
//
// Each kernel comes in two shapes.  The direct kernels give a workgroup's
// four waves 32 * slabs rows and split the contraction over 4 / slabs waves
// (slabs = 1, 2 or 4; partial sums meet in LDS), loading operands straight
// into registers: the most slabs that still give every compute unit a
// workgroup.  From 2048 rows on, the staged kernels take 128 rows per
// workgroup (one 32-row slab per wave) and copy the operands into LDS in
// coalesced 64-wide contraction chunks, up to four chunks in flight.
//
// The kernel boundaries are the cross-workgroup syncs: u and m go through a
// small workspace (L2 / MALL resident).  Each grid is 1-D over (row tile,
// column tile), and workgroup i runs on XCD i % 8.  With 8 or more row tiles
// the column tiles of one row tile share an XCD, so the activation rows they
// all read (gathered embeddings, bf16(u), m) come into that XCD's L2 once;
// measured at N = 256, B = 16 this takes the pass from 27.9 to 24.4 us (the
// activations are then several times the weights).  With fewer row tiles the
// row tiles of one column tile share an XCD and its weight slice instead.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, 64 lanes): lane l supplies
// A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32], e = 0..7;
// accumulator register r of lane l holds D[8 * (r / 4) + 4 * (l / 32) + r % 4]
// [l % 32].  With both weight matrices out-major, every operand is 8
// consecutive k values: one 16-byte load per lane per step.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "host_common.h"
#include "xpress_argmax.h"

namespace {

using namespace xpress;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;      // rows and columns of one MFMA tile
constexpr int kWaves = 4;      // waves of a workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 4;      // MFMA k-steps whose operands are loaded together
constexpr int kMaxB = 32;
constexpr int kPad = kTile + 1;  // LDS row stride of a 32-column fp32 tile

__device__ __forceinline__ u32x4 load16(const uint16_t* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// bf16 element e (0 .. 7) of eight packed in a 16-byte vector, widened
__device__ __forceinline__ float bf16_at(const u32x4& v, int e)
{
    const uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Workgroup b's (row tile, column tile).  With xmap the column tiles of one
// row tile share an XCD (workgroup b runs on XCD b % 8), so the activation
// rows they all read are fetched into that XCD's L2 once; otherwise the row
// tiles of one column tile do, sharing its weight slice.  Workgroups past the
// last row tile (xmap pads the row tiles to a multiple of 8) return at once.
__device__ __forceinline__ bool tile_of(uint32_t b, uint32_t col_tiles, uint32_t row_tiles,
                                        uint32_t xmap, uint32_t& rt, uint32_t& ct)
{
    if (xmap) {
        const uint32_t xcd = b & 7u, local = b >> 3;
        rt = (local / col_tiles) * 8u + xcd;
        ct = local % col_tiles;
    } else {
        ct = b % col_tiles;
        rt = b / col_tiles;
    }
    return rt < row_tiles;
}

// Operands of kChunk MFMA k-steps: A (8 k-values of this lane's row) and NB
// B operands sharing it (8 k-values of this lane's column of each weight).
template <int NB>
struct Chunk {
    u32x4 a[kChunk];
    u32x4 b[NB][kChunk];
};

// ap / bp point at k = 0 of this lane's row (A) and columns (B), already
// offset by 8 * (lane / 32); amask zeroes A (a zero embedding row).
template <int NB>
__device__ __forceinline__ void load_chunk(Chunk<NB>& c, const uint16_t* ap,
                                           const uint16_t* const (&bp)[NB], int k, uint32_t amask)
{
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
        c.a[s] = load16(ap + k + 16 * s) & amask;
#pragma unroll
        for (int m = 0; m < NB; ++m) c.b[m][s] = load16(bp[m] + k + 16 * s);
    }
}

template <int NB>
__device__ __forceinline__ void mma_chunk(f32x16 (&acc)[NB], const Chunk<NB>& c)
{
#pragma unroll
    for (int s = 0; s < kChunk; ++s) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, c.a[s]), __builtin_bit_cast(bf16x8, c.b[m][s]),
                acc[m], 0, 0, 0);
        }
    }
}

// acc[m] += A[32 x K] * B_m[K x 32] over k = k0 .. k0 + 16 * steps, in
// chunks of kChunk steps whose loads are issued one chunk ahead (two register
// buffers), then the remaining single steps.
template <int NB>
__device__ __forceinline__ void mma_k(f32x16 (&acc)[NB], const uint16_t* ap,
                                      const uint16_t* const (&bp)[NB], int k0, int steps,
                                      uint32_t amask)
{
    const int nfull = steps / kChunk;
    Chunk<NB> c0, c1;
    int c = 0;
    if (nfull > 0) load_chunk(c0, ap, bp, k0, amask);
    for (; c + 2 <= nfull; c += 2) {
        load_chunk(c1, ap, bp, k0 + 16 * kChunk * (c + 1), amask);
        mma_chunk(acc, c0);
        if (c + 2 < nfull) load_chunk(c0, ap, bp, k0 + 16 * kChunk * (c + 2), amask);
        mma_chunk(acc, c1);
    }
    if (c < nfull) mma_chunk(acc, c0);
    for (int s = nfull * kChunk; s < steps; ++s) {
        const u32x4 av = load16(ap + k0 + 16 * s) & amask;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, av),
                __builtin_bit_cast(bf16x8, load16(bp[m] + k0 + 16 * s)), acc[m], 0, 0, 0);
        }
    }
}

// Row (within the 32-row tile) held by accumulator register r of this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Store this wave's accumulator tile into part[32][kPad] (fp32).
__device__ __forceinline__ void store_tile(float* part, const f32x16& acc, int lane)
{
#pragma unroll
    for (int r = 0; r < 16; ++r) part[acc_row(r, lane) * kPad + (lane & 31)] = acc[r];
}

// The folded mixer of a tile: for the nb blocks whose x-rows (B per block,
// 32 channels, fp32, row stride kPad) sit in xs, u[b] = sum_j mixl[b, j] * x[j]
// for the slots b = 1 .. B-1 read out, with mixs the [B*B][32] bf16 slice of
// mixl.  A thread takes one (slot, channel) and CH blocks at a time as
// independent accumulation chains.
template <int CH>
__device__ __forceinline__ void mix_chains(const float* xs, const uint16_t* mixs, uint32_t nb,
                                           uint32_t B, uint32_t n0, uint32_t c0, uint32_t R,
                                           float* u_out, uint16_t* ub_out, int tid)
{
    const uint32_t bm1 = B - 1;
    for (uint32_t t = tid; t < bm1 * kTile; t += kThreads) {
        const uint32_t c = t & 31, b = 1 + (t >> 5);
        const uint16_t* mrow = mixs + (size_t)b * B * kTile + c;
        for (uint32_t lb0 = 0; lb0 < nb; lb0 += CH) {
            const float* xq[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                const uint32_t lb = lb0 + q < nb ? lb0 + q : nb - 1;
                xq[q] = xs + lb * B * kPad + c;
            }
            float acc[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q) acc[q] = 0.0f;
#pragma unroll 4
            for (uint32_t j = 0; j < B; ++j) {
                const float mv = from_bf16(mrow[j * kTile]);
#pragma unroll
                for (int q = 0; q < CH; ++q) acc[q] = fmaf(mv, xq[q][j * kPad], acc[q]);
            }
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                if (lb0 + q < nb) {
                    const size_t idx = ((size_t)(n0 + lb0 + q) * bm1 + (b - 1)) * R + c0 + c;
                    u_out[idx] = acc[q];
                    ub_out[idx] = to_bf16(acc[q]);
                }
            }
        }
    }
}

__device__ __forceinline__ void mix_tile(const float* xs, const uint16_t* mixs, uint32_t nb,
                                         uint32_t B, uint32_t n0, uint32_t c0, uint32_t R,
                                         float* u_out, uint16_t* ub_out, int tid)
{
    if (nb >= 4) {
        mix_chains<8>(xs, mixs, nb, B, n0, c0, R, u_out, ub_out, tid);
    } else {
        mix_chains<1>(xs, mixs, nb, B, n0, c0, R, u_out, ub_out, tid);
    }
}

// The folded mixer for tiles of many blocks (the staged kernel, B <= 16),
// from a transposed fp32 copy of the mixer slice: mixt[((b - 1) * 32 + c) *
// kMixT + j] = mixl[b, j, c0 + c], zero for j >= B.  A thread takes one
// (block, channel): the block's x values for that channel go into
// registers once, and each slot's sixteen weights come in four 16-byte LDS
// reads (the rows are padded to 20 floats so that sixteen consecutive
// channels' reads fall on different banks).  The sums are formed in the
// same order as mix_chains (j ascending from +0; the padded j add exactly
// zero), so the two give the same bits.
constexpr uint32_t kMixT = 20;

__device__ __forceinline__ void mix_tile_t(const float* xs, const float* mixt, uint32_t nb,
                                           uint32_t B, uint32_t n0, uint32_t c0, uint32_t R,
                                           float* u_out, uint16_t* ub_out, int tid)
{
    const uint32_t bm1 = B - 1;
    for (uint32_t t = tid; t < nb * kTile; t += kThreads) {
        const uint32_t lb = t >> 5, c = t & 31;
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = (uint32_t)j < B ? xs[(lb * B + j) * kPad + c] : 0.0f;
        float* urow = u_out + ((size_t)(n0 + lb) * bm1) * R + c0 + c;
        uint16_t* ubrow = ub_out + ((size_t)(n0 + lb) * bm1) * R + c0 + c;
#pragma unroll 3
        for (uint32_t b = 1; b < B; ++b) {
            const float* mr = mixt + ((b - 1) * kTile + c) * kMixT;
            float m[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4*>(mr + 4 * q);
                m[4 * q] = v.x;
                m[4 * q + 1] = v.y;
                m[4 * q + 2] = v.z;
                m[4 * q + 3] = v.w;
            }
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc = fmaf(m[j], x[j], acc);
            urow[(size_t)(b - 1) * R] = acc;
            ubrow[(size_t)(b - 1) * R] = to_bf16(acc);
        }
    }
}

struct MixArgs {
    const int64_t* blk;
    const int64_t* am1;
    const uint16_t* xh;
    const uint16_t* w1;
    const uint16_t* wlat;
    const uint16_t* mixl;
    float* u;        // [N * (B - 1), R]
    uint16_t* ub;    // [N * (B - 1), R]
    int64_t V;
    uint32_t N, B, R, bpt, col_tiles;
    uint32_t row_tiles, xmap;
};

// One workgroup per (bpt whole blocks -- at most 32 * WR x-rows -- and 32
// channels).  Wave w takes the 32-row slab w % WR and the K range w / WR of
// WK equal parts.
template <int WR, int WK>
__global__ void __launch_bounds__(kThreads) latent_mix_kernel(MixArgs a)
{
    static_assert(WR * WK == kWaves, "four waves");
    constexpr int kRows = WR * kTile;
    __shared__ float part[WK][kRows * kPad];
    __shared__ uint16_t xhs[kRows * kTile];
    extern __shared__ u32x4 mixs_dyn[];  // [B * B][32] bf16 slice of mixl
    const uint16_t* mixs = reinterpret_cast<const uint16_t*>(mixs_dyn);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const int wr = wave % WR, wk = wave / WR;
    uint32_t rt, ct;
    if (!tile_of(blockIdx.x, a.col_tiles, a.row_tiles, a.xmap, rt, ct)) return;
    const uint32_t c0 = ct * kTile;
    const uint32_t B = a.B, R = a.R;
    const uint32_t n0 = rt * a.bpt;
    const uint32_t nb = (a.N - n0 < a.bpt) ? (a.N - n0) : a.bpt;
    const uint32_t rows = nb * B;  // valid x-rows of the tile

    // the mixer slice [B*B rows of 32 channels] and the cache tile to LDS
    const uint32_t mix_chunks = B * B * 4;  // 16-byte chunks
    for (uint32_t q = tid; q < mix_chunks; q += kThreads) {
        mixs_dyn[q] = load16(a.mixl + (size_t)(q >> 2) * R + c0 + 8 * (q & 3));
    }
    for (uint32_t q = tid; q < (uint32_t)kRows * 4; q += kThreads) {
        const uint32_t i = q >> 2, p = q & 3;
        const uint32_t ic = i < rows ? i : 0;
        const u32x4 v = load16(a.xh + ((size_t)n0 * B + ic) * R + c0 + 8 * p);
        *reinterpret_cast<u32x4*>(xhs + i * kTile + 8 * p) = v & (i < rows ? ~0u : 0u);
    }

    // A row of this lane: the embedding of the previous slot's token
    const uint32_t i = wr * kTile + (lane & 31);
    const uint32_t ic = i < rows ? i : 0;
    const uint32_t n = n0 + ic / B, slot = ic % B;
    const int64_t tok = (slot == 0) ? a.am1[n] : a.blk[(size_t)n * B + slot - 1];
    // an id outside [0, V) (and a padding row) reads as a zero embedding row
    const bool tok_ok = i < rows && tok >= 0 && tok < a.V;
    const uint16_t* ap = a.w1 + (size_t)(tok_ok ? tok : 0) * R + 8 * half;
    const uint16_t* bp[1] = {a.wlat + (size_t)(c0 + (lane & 31)) * R + 8 * half};
    const int steps = (int)(R / 16) / WK;
    f32x16 acc[1] = {};
    mma_k<1>(acc, ap, bp, wk * steps * 16, steps, tok_ok ? ~0u : 0u);
    store_tile(&part[wk][wr * kTile * kPad], acc[0], lane);
    __syncthreads();

    // x = cache + the K-partials, kept in part[0]
    for (int e = tid; e < kRows * kTile; e += kThreads) {
        const int r = e >> 5, c = e & 31;
        const int o = r * kPad + c;
        float x;
        if constexpr (WK == 4) {
            x = (part[0][o] + part[1][o]) + (part[2][o] + part[3][o]);
        } else if constexpr (WK == 2) {
            x = part[0][o] + part[1][o];
        } else {
            x = part[0][o];
        }
        part[0][o] = x + from_bf16(xhs[r * kTile + c]);
    }
    __syncthreads();

    mix_tile(&part[0][0], mixs, nb, B, n0, c0, R, a.u, a.ub, tid);
}

struct GateArgs {
    const uint16_t* ub;  // [rows, R]
    const uint16_t* wg;  // [H, R]
    const uint16_t* wu;  // [H, R]
    uint16_t* m;         // [rows, H]
    uint32_t rows, R, H, col_tiles;
    uint32_t row_tiles, xmap;
};

// g * sigmoid(g) * v in fp32: the accurate exp, then the hardware reciprocal
// (about 1 ulp) instead of a correctly rounded division.
__device__ __forceinline__ float swiglu(float g, float v)
{
    return g * __builtin_amdgcn_rcpf(1.0f + expf(-g)) * v;
}

// bf16(swiglu) of a wave's 16 accumulator values, stored to m for the rows
// that exist.  All sixteen are formed first, outside any branch, so that
// their exponentials interleave; only a slab that reaches past the last row
// takes the per-element check.  row0: the slab's first row.
__device__ __forceinline__ void store_m_tile(uint16_t* m, uint32_t ldm, uint32_t col,
                                             const f32x16& g, const f32x16& v, uint32_t row0,
                                             uint32_t rows, int lane)
{
    uint16_t mv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) mv[r] = to_bf16(swiglu(g[r], v[r]));
    if (row0 + kTile <= rows) {
#pragma unroll
        for (int r = 0; r < 16; ++r) m[(size_t)(row0 + acc_row(r, lane)) * ldm + col] = mv[r];
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t rr = row0 + acc_row(r, lane);
            if (rr < rows) m[(size_t)rr * ldm + col] = mv[r];
        }
    }
}

// One workgroup per (32 * WR rows, 32 hidden units); g and v share A.
template <int WR, int WK>
__global__ void __launch_bounds__(kThreads) latent_gate_kernel(GateArgs a)
{
    static_assert(WR * WK == kWaves, "four waves");
    constexpr int kRows = WR * kTile;
    __shared__ float part[2][WK > 1 ? WK : 1][WK > 1 ? kRows * kPad : 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const int wr = wave % WR, wk = wave / WR;
    uint32_t rt, ht;
    if (!tile_of(blockIdx.x, a.col_tiles, a.row_tiles, a.xmap, rt, ht)) return;
    const uint32_t h0 = ht * kTile, i0 = rt * kRows;
    const uint32_t row = i0 + wr * kTile + (lane & 31);
    const uint32_t rowc = row < a.rows ? row : a.rows - 1;  // padding rows: any valid row
    const uint16_t* ap = a.ub + (size_t)rowc * a.R + 8 * half;
    const uint16_t* bp[2] = {a.wg + (size_t)(h0 + (lane & 31)) * a.R + 8 * half,
                             a.wu + (size_t)(h0 + (lane & 31)) * a.R + 8 * half};
    const int steps = (int)(a.R / 16) / WK;
    f32x16 acc[2] = {};
    mma_k<2>(acc, ap, bp, wk * steps * 16, steps, ~0u);
    if constexpr (WK == 1) {
        store_m_tile(a.m, a.H, h0 + (lane & 31), acc[0], acc[1], i0 + wr * kTile, a.rows, lane);
    } else {
        store_tile(&part[0][wk][wr * kTile * kPad], acc[0], lane);
        store_tile(&part[1][wk][wr * kTile * kPad], acc[1], lane);
        __syncthreads();
        // every element's value first, outside any branch (their
        // exponentials interleave), then the stores for the rows that exist
        constexpr int kPer = kRows * kTile / kThreads;
        uint16_t mv[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = tid + q * kThreads;
            const int o = (e >> 5) * kPad + (e & 31);
            float gs, vs;
            if constexpr (WK == 4) {
                gs = (part[0][0][o] + part[0][1][o]) + (part[0][2][o] + part[0][3][o]);
                vs = (part[1][0][o] + part[1][1][o]) + (part[1][2][o] + part[1][3][o]);
            } else {
                gs = part[0][0][o] + part[0][1][o];
                vs = part[1][0][o] + part[1][1][o];
            }
            mv[q] = to_bf16(swiglu(gs, vs));
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = tid + q * kThreads;
            const int r = e >> 5, c = e & 31;
            if (i0 + r < a.rows) a.m[(size_t)(i0 + r) * a.H + h0 + c] = mv[q];
        }
    }
}

struct DownArgs {
    const uint16_t* m;   // [rows, H]
    const uint16_t* wd;  // [R, H]
    const float* u;      // [rows, R]
    uint16_t* out;       // [rows, R]
    uint32_t rows, R, H, col_tiles;
    uint32_t row_tiles, xmap;
};

// One workgroup per (32 * WR rows, 32 channels).
template <int WR, int WK>
__global__ void __launch_bounds__(kThreads) latent_down_kernel(DownArgs a)
{
    static_assert(WR * WK == kWaves, "four waves");
    constexpr int kRows = WR * kTile;
    __shared__ float part[WK > 1 ? WK : 1][WK > 1 ? kRows * kPad : 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const int wr = wave % WR, wk = wave / WR;
    uint32_t rt, ct;
    if (!tile_of(blockIdx.x, a.col_tiles, a.row_tiles, a.xmap, rt, ct)) return;
    const uint32_t c0 = ct * kTile, i0 = rt * kRows;
    const uint32_t row = i0 + wr * kTile + (lane & 31);
    const uint32_t rowc = row < a.rows ? row : a.rows - 1;
    const uint16_t* ap = a.m + (size_t)rowc * a.H + 8 * half;
    const uint16_t* bp[1] = {a.wd + (size_t)(c0 + (lane & 31)) * a.H + 8 * half};
    const int steps = (int)(a.H / 16) / WK;
    if constexpr (WK == 1) {
        // the residual, fetched ahead of the products
        float res[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t rr = i0 + wr * kTile + acc_row(r, lane);
            res[r] = a.u[(size_t)(rr < a.rows ? rr : a.rows - 1) * a.R + c0 + (lane & 31)];
        }
        f32x16 acc[1] = {};
        mma_k<1>(acc, ap, bp, 0, steps, ~0u);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t rr = i0 + wr * kTile + acc_row(r, lane);
            if (rr < a.rows) a.out[(size_t)rr * a.R + c0 + (lane & 31)] = to_bf16(res[r] + acc[0][r]);
        }
    } else {
        constexpr int kPer = kRows * kTile / kThreads;  // elements per thread
        float res[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = tid + q * kThreads;
            const uint32_t rr = i0 + (e >> 5);
            res[q] = a.u[(size_t)(rr < a.rows ? rr : a.rows - 1) * a.R + c0 + (e & 31)];
        }
        f32x16 acc[1] = {};
        mma_k<1>(acc, ap, bp, wk * steps * 16, steps, ~0u);
        store_tile(&part[wk][wr * kTile * kPad], acc[0], lane);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e = tid + q * kThreads;
            const int r = e >> 5, c = e & 31;
            if (i0 + r >= a.rows) continue;
            const int o = r * kPad + c;
            float mm;
            if constexpr (WK == 4) {
                mm = (part[0][o] + part[1][o]) + (part[2][o] + part[3][o]);
            } else {
                mm = part[0][o] + part[1][o];
            }
            a.out[(size_t)(i0 + r) * a.R + c0 + c] = to_bf16(res[q] + mm);
        }
    }
}

// ---------------------------------------------------------------------------
// LDS-staged variants for many rows.  A workgroup computes 128 rows (one
// 32-row slab per wave) of one or more 32-column tiles.  The contraction is
// walked in chunks of 64; the A and B rows of a chunk are copied straight
// from global memory into LDS by the 16-byte load-to-LDS instruction (eight
// lanes per 128-byte row segment, so every load instruction reads eight whole
// cache lines), four chunks in flight at once, and the matrix cores read
// their operands back with 16-byte LDS loads.  Within an LDS row the 16-byte
// columns are permuted by XOR with ((row >> 1) & 7): a row is 128 bytes, so
// rows two apart share banks, and keying on row >> 1 puts the 16 rows one
// pass of an operand load touches on 16 different bank groups (row & 7 left
// them two to a group).
// ---------------------------------------------------------------------------
constexpr int kKC = 64;           // contraction elements per chunk
constexpr int kRing = 4;          // chunks in flight
constexpr int kSlabRows = 128;    // A rows of a staged workgroup

// Rows [32 j + 8 w, +8) of a chunk are loaded by wave w's j-th instruction;
// lane l reads row 32 j + 8 w + l / 8, logical 16-byte column
// (l % 8) ^ ((row >> 1) & 7), and lands in LDS at row-major position
// (row, l % 8).
template <int ROWS>
struct DmaRows {
    static constexpr int kN = ROWS / 32;  // load instructions per wave per chunk
    const uint16_t* src[kN];              // this lane's row, at its swizzled column
};

template <int ROWS>
__device__ __forceinline__ void dma_chunk(const DmaRows<ROWS>& d, uint16_t* lds_slot, int k0,
                                          int wave)
{
#pragma unroll
    for (int j = 0; j < DmaRows<ROWS>::kN; ++j) {
        dma16(d.src[j] + k0, lds_addr(lds_slot + (32 * j + 8 * wave) * kKC));
    }
}

// MFMA operand: logical row r, k = 16 s + 8 (lane / 32) of a staged chunk.
__device__ __forceinline__ bf16x8 lds_operand(const uint16_t* lds_slot, int r0, int s, int lane)
{
    const int r = r0 + (lane & 31);
    const int q = (2 * s + (lane >> 5)) ^ ((r >> 1) & 7);
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4*>(lds_slot + r * kKC + 8 * q));
}

template <int ROWS>
__device__ __forceinline__ void dma_setup(DmaRows<ROWS>& d, const uint16_t* const* row_base,
                                          int lane, int wave)
{
    // the row 32 j + 8 wave + lane / 8 has (row >> 1) & 7 = (4 wave + lane / 16) & 7
    const int sw = (4 * wave + (lane >> 4)) & 7;
#pragma unroll
    for (int j = 0; j < DmaRows<ROWS>::kN; ++j) {
        d.src[j] = row_base[j] + 8 * ((lane & 7) ^ sw);
    }
}

// Wait until this wave's loads of chunk c have landed, given `ahead` later
// chunks already issued (0 .. kRing-1), each PER load instructions.
template <int PER>
__device__ __forceinline__ void wait_chunk(int ahead)
{
    switch (ahead) {
        case 3: wait_vmcnt<3 * PER>(); break;
        case 2: wait_vmcnt<2 * PER>(); break;
        case 1: wait_vmcnt<1 * PER>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// acc[t] += A[wave slab] * B[tile t] over the contraction (nc chunks).
// zero_row: bit q set when A row (lane / 8) + 8 * wave + 32 q must read as
// zeros (an invalid embedding id); those LDS rows are cleared after landing.
template <int ROWS_A, int ROWS_B, int NT>
__device__ __forceinline__ void staged_mma(f32x16 (&acc)[NT], const DmaRows<ROWS_A>& da,
                                           const DmaRows<ROWS_B>& db,
                                           uint16_t (*lds_a)[ROWS_A * kKC],
                                           uint16_t (*lds_b)[ROWS_B * kKC], int nc, int tid,
                                           uint32_t zero_row)
{
    constexpr int kPer = DmaRows<ROWS_A>::kN + DmaRows<ROWS_B>::kN;
    const int wave = tid >> 6, lane = tid & 63;
    const int first = nc < kRing ? nc : kRing;
    for (int c = 0; c < first; ++c) {
        dma_chunk(da, lds_a[c], c * kKC, wave);
        dma_chunk(db, lds_b[c], c * kKC, wave);
    }
    for (int c = 0; c < nc; ++c) {
        const int slot = c % kRing;
        const int issued = (c + kRing < nc ? c + kRing : nc);  // chunks issued so far
        wait_chunk<kPer>(issued - 1 - c);
        if (zero_row) {
#pragma unroll
            for (int q = 0; q < DmaRows<ROWS_A>::kN; ++q) {
                if (zero_row & (1u << q)) {
                    *reinterpret_cast<u32x4*>(lds_a[slot] + (32 * q + 8 * wave + (lane >> 3)) * kKC +
                                              8 * (lane & 7)) = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kKC / 16; ++s) {
            const bf16x8 av = lds_operand(lds_a[slot], kTile * wave, s, lane);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    av, lds_operand(lds_b[slot], kTile * t, s, lane), acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
        if (c + kRing < nc) {
            dma_chunk(da, lds_a[slot], (c + kRing) * kKC, wave);
            dma_chunk(db, lds_b[slot], (c + kRing) * kKC, wave);
        }
    }
}

// gate, staged: 128 rows x 32*NH hidden units; B holds NH tiles of wg, then
// the NH matching tiles of wu.
template <int NH>
__global__ void __launch_bounds__(kThreads) latent_gate_staged(GateArgs a)
{
    constexpr int kB = 2 * kTile * NH;
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[kRing][kSlabRows * kKC];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[kRing][kB * kKC];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const uint32_t col_tiles = a.H / (kTile * NH);
    uint32_t rt, ht;
    if (!tile_of(blockIdx.x, col_tiles, a.row_tiles, a.xmap, rt, ht)) return;
    const uint32_t h0 = ht * kTile * NH, i0 = rt * kSlabRows;
    const uint16_t* abase[DmaRows<kSlabRows>::kN];
#pragma unroll
    for (int j = 0; j < DmaRows<kSlabRows>::kN; ++j) {
        const uint32_t row = i0 + 32 * j + 8 * wave + (lane >> 3);
        abase[j] = a.ub + (size_t)(row < a.rows ? row : 0) * a.R;  // padding rows: any row
    }
    const uint16_t* bbase[DmaRows<kB>::kN];
#pragma unroll
    for (int j = 0; j < DmaRows<kB>::kN; ++j) {
        const uint32_t br = 32 * j + 8 * wave + (lane >> 3);
        const uint32_t hr = h0 + br % (kTile * NH);
        bbase[j] = (br < (uint32_t)(kTile * NH) ? a.wg : a.wu) + (size_t)hr * a.R;
    }
    DmaRows<kSlabRows> da;
    DmaRows<kB> db;
    dma_setup(da, abase, lane, wave);
    dma_setup(db, bbase, lane, wave);
    f32x16 acc[2 * NH] = {};
    staged_mma<kSlabRows, kB, 2 * NH>(acc, da, db, lds_a, lds_b, (int)(a.R / kKC), tid, 0u);
#pragma unroll
    for (int t = 0; t < NH; ++t) {
        store_m_tile(a.m, a.H, h0 + kTile * t + (lane & 31), acc[t], acc[NH + t],
                     i0 + kTile * wave, a.rows, lane);
    }
}

// down, staged: 128 rows x 32 channels, plus the residual.
__global__ void __launch_bounds__(kThreads) latent_down_staged(DownArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[kRing][kSlabRows * kKC];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[kRing][kTile * kKC];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t rt, ct;
    if (!tile_of(blockIdx.x, a.col_tiles, a.row_tiles, a.xmap, rt, ct)) return;
    const uint32_t c0 = ct * kTile, i0 = rt * kSlabRows;
    // the residual first: these loads are older than the chunk loads the
    // contraction counts
    float res[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t rr = i0 + kTile * wave + acc_row(r, lane);
        res[r] = a.u[(size_t)(rr < a.rows ? rr : 0) * a.R + c0 + (lane & 31)];
    }
    const uint16_t* abase[DmaRows<kSlabRows>::kN];
#pragma unroll
    for (int j = 0; j < DmaRows<kSlabRows>::kN; ++j) {
        const uint32_t row = i0 + 32 * j + 8 * wave + (lane >> 3);
        abase[j] = a.m + (size_t)(row < a.rows ? row : 0) * a.H;
    }
    const uint16_t* bbase[1] = {a.wd + (size_t)(c0 + 8 * wave + (lane >> 3)) * a.H};
    DmaRows<kSlabRows> da;
    DmaRows<kTile> db;
    dma_setup(da, abase, lane, wave);
    dma_setup(db, bbase, lane, wave);
    f32x16 acc[1] = {};
    staged_mma<kSlabRows, kTile, 1>(acc, da, db, lds_a, lds_b, (int)(a.H / kKC), tid, 0u);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t rr = i0 + kTile * wave + acc_row(r, lane);
        if (rr < a.rows) a.out[(size_t)rr * a.R + c0 + (lane & 31)] = to_bf16(res[r] + acc[0][r]);
    }
}

// mix, staged: bpt = 128 / B whole blocks (their x-rows gathered from w1)
// x 32 channels, then the folded mixer from LDS.
__global__ void __launch_bounds__(kThreads) latent_mix_staged(MixArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[kRing][kSlabRows * kKC];
    __shared__ __attribute__((aligned(16))) uint16_t lds_b[kRing][kTile * kKC];
    extern __shared__ u32x4 mixs_dyn[];  // [B * B][32] bf16 slice of mixl
    const uint16_t* mixs = reinterpret_cast<const uint16_t*>(mixs_dyn);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    uint32_t rt, ct;
    if (!tile_of(blockIdx.x, a.col_tiles, a.row_tiles, a.xmap, rt, ct)) return;
    const uint32_t c0 = ct * kTile;
    const uint32_t B = a.B, R = a.R;
    const uint32_t n0 = rt * a.bpt;
    const uint32_t nb = (a.N - n0 < a.bpt) ? (a.N - n0) : a.bpt;
    const uint32_t rows = nb * B;

    // Every load here goes out at once, older than the chunk loads the
    // contraction counts: the token ids (they gate the embedding copies),
    // the mixer slice and the cache rows.  Only the token ids are waited for
    // before the chunk copies go out; the slice is stored to LDS after the
    // contraction (its loads, older than the copies, have landed by the
    // first chunk's wait), so the copies do not wait for it.
    constexpr int kN = DmaRows<kSlabRows>::kN;
    int64_t tok[kN];
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        const uint32_t i = 32 * j + 8 * wave + (lane >> 3);
        const uint32_t ic = i < rows ? i : 0;
        const uint32_t n = n0 + ic / B, slot = ic % B;
        const int64_t* tp = (slot == 0) ? a.am1 + n : a.blk + (size_t)n * B + slot - 1;
        tok[j] = *tp;
    }
    // the token loads stay ahead of the loads below (waiting for them then
    // leaves the slice and cache loads in flight)
    asm volatile("" ::: "memory");
    constexpr int kMixPer = kMaxB * kMaxB * 4 / kThreads;
    static_assert(kMixPer * kThreads == kMaxB * kMaxB * 4, "mixer slice split over threads");
    const uint32_t mix_chunks = B * B * 4;
    // unconditional loads (chunks past the slice repeat its last one and are
    // not stored): a predicated load with a default value makes the compiler
    // wait for it on the spot
    u32x4 mreg[kMixPer];
#pragma unroll
    for (int q = 0; q < kMixPer; ++q) {
        uint32_t c = tid + q * kThreads;
        c = c < mix_chunks ? c : mix_chunks - 1u;
        mreg[q] = load16(a.mixl + (size_t)(c >> 2) * R + c0 + 8 * (c & 3));
    }
    float xh[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t i = kTile * wave + acc_row(r, lane);
        xh[r] = from_bf16(a.xh[((size_t)n0 * B + (i < rows ? i : 0)) * R + c0 + (lane & 31)]);
    }
    const uint16_t* abase[kN];
    uint32_t zero_row = 0;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        const uint32_t i = 32 * j + 8 * wave + (lane >> 3);
        const bool ok = tok[j] >= 0 && tok[j] < a.V;
        abase[j] = a.w1 + (size_t)(ok ? tok[j] : 0) * R;
        // an id outside [0, V) reads as a zero embedding row (padding rows
        // beyond the tile's blocks are never read back)
        if (i < rows && !ok) zero_row |= 1u << j;
    }
    const uint16_t* bbase[1] = {a.wlat + (size_t)(c0 + 8 * wave + (lane >> 3)) * R};
    DmaRows<kSlabRows> da;
    DmaRows<kTile> db;
    dma_setup(da, abase, lane, wave);
    dma_setup(db, bbase, lane, wave);
    f32x16 acc[1] = {};
    staged_mma<kSlabRows, kTile, 1>(acc, da, db, lds_a, lds_b, (int)(R / kKC), tid, zero_row);
    // the mixer slice, read by the mixer after the barrier below: for B <= 16
    // transposed to fp32 (mix_tile_t), else as loaded (mix_tile)
    const bool transposed = B <= 16;
    float* mixt = reinterpret_cast<float*>(mixs_dyn);
    if (transposed) {
#pragma unroll
        for (int q = 0; q < kMixPer; ++q) {
            const uint32_t c = tid + q * kThreads;
            if (c < mix_chunks) {
                const uint32_t bj = c >> 2, b = bj / B, j = bj - b * B, c8 = (c & 3) * 8;
                if (b >= 1) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        mixt[((b - 1) * kTile + c8 + e) * kMixT + j] = bf16_at(mreg[q], e);
                    }
                }
            }
        }
        for (uint32_t i = tid; i < (B - 1) * kTile; i += kThreads) {
            for (uint32_t j = B; j < 16; ++j) mixt[i * kMixT + j] = 0.0f;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kMixPer; ++q) {
            const uint32_t c = tid + q * kThreads;
            if (c < mix_chunks) mixs_dyn[c] = mreg[q];
        }
    }
    // x = cache + projection, into LDS over the A staging area (free after
    // the contraction's last barrier)
    static_assert(kSlabRows * kPad * sizeof(float) <= sizeof(lds_a), "x tile fits the ring");
    float* xs = reinterpret_cast<float*>(&lds_a[0][0]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        xs[(kTile * wave + acc_row(r, lane)) * kPad + (lane & 31)] = acc[0][r] + xh[r];
    }
    __syncthreads();
    if (transposed) {
        mix_tile_t(xs, mixt, nb, B, n0, c0, R, a.u, a.ub, tid);
    } else {
        mix_tile(xs, mixs, nb, B, n0, c0, R, a.u, a.ub, tid);
    }
}

// Workgroup shape per kernel: 1, 2 or 4 row slabs of the direct kernels, 8
// for the LDS-staged kernel, 0 = chosen from the shape.
constexpr int kStaged = 8;
constexpr uint64_t kStagedFromRows = 2048;  // measured: direct wins at 1024 rows
struct LatentTiles {
    int mix = 0, gate = 0, down = 0;
};
std::mutex g_tiles_mu;
LatentTiles g_tiles;

// The largest slab count that still gives every compute unit a workgroup.
int auto_slabs(uint64_t wgs_at_one_slab, int cus)
{
    if (wgs_at_one_slab >= 4ull * (uint64_t)cus) return 4;
    if (wgs_at_one_slab >= 2ull * (uint64_t)cus) return 2;
    return 1;
}

// Workspace carve-up: u (fp32), bf16(u) and m, each 256-byte aligned.
struct LatentScratch {
    size_t u_off, ub_off, m_off, bytes;
};

LatentScratch scratch_layout(int64_t rows, int64_t R, int64_t H)
{
    auto up = [](size_t x) { return (x + 255u) & ~(size_t)255u; };
    LatentScratch s;
    s.u_off = 0;
    s.ub_off = up((size_t)rows * R * 4u);
    s.m_off = s.ub_off + up((size_t)rows * R * 2u);
    s.bytes = s.m_off + up((size_t)rows * H * 2u);
    return s;
}

int check_sizes(int64_t N, int64_t B, int64_t R, int64_t H, int64_t V)
{
    if (N < 0 || B < 2 || B > kMaxB || V < 1) return XPRESS_EINVAL;
    if (R < 64 || R > 1024 || R % 64 != 0) return XPRESS_EINVAL;
    if (H < 64 || H > 8192 || H % 64 != 0) return XPRESS_EINVAL;
    if (N > 0x7FFFFFFFll / B) return XPRESS_EINVAL;
    return XPRESS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int xpress_latent_reserve(int64_t N, int64_t B, int64_t R, int64_t H, hipStream_t stream)
{
    int rc = check_sizes(N, B, R, H, 1);
    if (rc != XPRESS_OK) return rc;
    const int64_t rows = N * (B - 1);
    if (rows == 0) return XPRESS_OK;
    const LatentScratch s = scratch_layout(rows, R, H);
    uint64_t* table = nullptr;
    return workspace_table(stream, (int64_t)(s.bytes / 8u), &table);
}

int xpress_latent_pass(const int64_t* blk, const int64_t* am1, const uint16_t* xh,
                       const uint16_t* w1, const uint16_t* wlat, const uint16_t* mixl,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       uint16_t* lat_out, int64_t N, int64_t B, int64_t R, int64_t H,
                       int64_t V, hipStream_t stream)
{
    int rc = check_sizes(N, B, R, H, V);
    if (rc != XPRESS_OK) return rc;
    if (N == 0) return XPRESS_OK;
    const void* in16[] = {xh, w1, wlat, mixl, wg, wu, wd};
    for (const void* p : in16) {
        if (p == nullptr || !aligned(p, 16)) return XPRESS_EINVAL;
    }
    if (blk == nullptr || am1 == nullptr || lat_out == nullptr) return XPRESS_EINVAL;
    if (!aligned(blk, 8) || !aligned(am1, 8) || !aligned(lat_out, 2)) return XPRESS_EINVAL;
    const int64_t rows = N * (B - 1);
    const size_t out_bytes = (size_t)rows * R * 2u;
    const struct {
        const void* p;
        size_t n;
    } ins[] = {{blk, (size_t)N * B * 8u},       {am1, (size_t)N * 8u},
               {xh, (size_t)N * B * R * 2u},    {w1, (size_t)V * R * 2u},
               {wlat, (size_t)R * R * 2u},      {mixl, (size_t)B * B * R * 2u},
               {wg, (size_t)H * R * 2u},        {wu, (size_t)H * R * 2u},
               {wd, (size_t)R * H * 2u}};
    for (const auto& in : ins) {
        if (ranges_overlap(lat_out, out_bytes, in.p, in.n)) return XPRESS_EINVAL;
    }

    const LatentScratch s = scratch_layout(rows, R, H);
    uint64_t* table = nullptr;
    rc = workspace_table(stream, (int64_t)(s.bytes / 8u), &table);
    if (rc != XPRESS_OK) return rc;
    char* base = reinterpret_cast<char*>(table);
    float* u = reinterpret_cast<float*>(base + s.u_off);
    uint16_t* ub = reinterpret_cast<uint16_t*>(base + s.ub_off);
    uint16_t* m = reinterpret_cast<uint16_t*>(base + s.m_off);

    int cus = device_cus();
    if (cus < 1) cus = 256;
    LatentTiles t;
    {
        std::lock_guard<std::mutex> lk(g_tiles_mu);
        t = g_tiles;
    }

    // mix: bpt = (32 * WR) / B whole blocks per workgroup (128 / B staged)
    const uint64_t ctiles = (uint64_t)(R / kTile);
    const uint64_t xrows = (uint64_t)N * B;  // staged from kStagedFromRows x-rows
    int wr_mix = t.mix;
    if (!wr_mix) {
        wr_mix = xrows >= kStagedFromRows
                     ? kStaged
                     : auto_slabs((uint64_t)((N + kTile / B - 1) / (kTile / B)) * ctiles, cus);
    }
    MixArgs ma;
    ma.blk = blk;
    ma.am1 = am1;
    ma.xh = xh;
    ma.w1 = w1;
    ma.wlat = wlat;
    ma.mixl = mixl;
    ma.u = u;
    ma.ub = ub;
    ma.V = V;
    ma.N = (uint32_t)N;
    ma.B = (uint32_t)B;
    ma.R = (uint32_t)R;
    ma.bpt = (uint32_t)((wr_mix == kStaged ? kSlabRows : kTile * wr_mix) / B);
    ma.col_tiles = (uint32_t)ctiles;
    // grid of one kernel: row tiles x column tiles; with at least 8 row
    // tiles, the column tiles of a row tile share an XCD (row tiles padded to
    // a multiple of 8)
    auto grid_of = [](uint64_t row_tiles, uint64_t col_tiles, uint32_t* xmap) -> uint64_t {
        *xmap = row_tiles >= 8 ? 1u : 0u;
        return (*xmap ? (row_tiles + 7) / 8 * 8 : row_tiles) * col_tiles;
    };
    const uint64_t mix_rt = (uint64_t)((N + ma.bpt - 1) / ma.bpt);
    ma.row_tiles = (uint32_t)(mix_rt < 0xFFFFFFFFull ? mix_rt : 0xFFFFFFFFull);
    const uint64_t mix_wgs = grid_of(mix_rt, ctiles, &ma.xmap);

    const uint64_t rows_u = (uint64_t)rows;
    int wr_gate = t.gate, wr_down = t.down;
    if (!wr_gate) {
        wr_gate = rows_u >= kStagedFromRows ? kStaged
                                            : auto_slabs((rows_u + kTile - 1) / kTile * (H / kTile), cus);
    }
    if (!wr_down) {
        wr_down = rows_u >= kStagedFromRows ? kStaged
                                            : auto_slabs((rows_u + kTile - 1) / kTile * ctiles, cus);
    }
    const uint64_t slabs128 = (rows_u + kSlabRows - 1) / kSlabRows;
    // staged gate: two hidden tiles per workgroup once one-tile workgroups
    // (one per CU: the staging takes most of the LDS) would need two rounds
    const int gate_nh =
        (H % 64 == 0 && slabs128 * (uint64_t)(H / 32) > (uint64_t)cus) ? 2 : 1;
    const uint64_t gate_rt = wr_gate == kStaged ? slabs128
                                                : (rows_u + kTile * wr_gate - 1) / (kTile * wr_gate);
    const uint64_t down_rt = wr_down == kStaged ? slabs128
                                                : (rows_u + kTile * wr_down - 1) / (kTile * wr_down);
    uint32_t gate_xmap = 0, down_xmap = 0;
    const uint64_t gate_wgs = grid_of(gate_rt,
                                      wr_gate == kStaged ? (uint64_t)(H / (kTile * gate_nh))
                                                         : (uint64_t)(H / kTile),
                                      &gate_xmap);
    const uint64_t down_wgs = grid_of(down_rt, ctiles, &down_xmap);
    if (mix_wgs > 0x7FFFFFFFull || gate_wgs > 0x7FFFFFFFull || down_wgs > 0x7FFFFFFFull) {
        return XPRESS_EINVAL;
    }

    // the staged kernel keeps a transposed fp32 copy of the slice for B <= 16
    const size_t mix_lds = (wr_mix == kStaged && B <= 16) ? (size_t)(B - 1) * kTile * kMixT * 4u
                                                          : (size_t)B * B * kTile * 2u;
    const void* mix_fn = wr_mix == kStaged ? reinterpret_cast<const void*>(&latent_mix_staged)
                       : wr_mix == 4 ? reinterpret_cast<const void*>(&latent_mix_kernel<4, 1>)
                       : wr_mix == 2 ? reinterpret_cast<const void*>(&latent_mix_kernel<2, 2>)
                                     : reinterpret_cast<const void*>(&latent_mix_kernel<1, 4>);
    if (mix_lds > 16384u) {
        // the mixer slice of a large block size takes most of the LDS (up to
        // 64 KiB at B = 32, beside at most 46 KiB of static LDS)
        hipError_t ea = hipFuncSetAttribute(mix_fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)mix_lds);
        if (ea != hipSuccess) return hip_fail(ea);
    }
    const dim3 blk3(kThreads);
    const dim3 mix_grid((uint32_t)mix_wgs);
    if (wr_mix == kStaged) {
        hipLaunchKernelGGL(latent_mix_staged, mix_grid, blk3, mix_lds, stream, ma);
    } else if (wr_mix == 4) {
        hipLaunchKernelGGL((latent_mix_kernel<4, 1>), mix_grid, blk3, mix_lds, stream, ma);
    } else if (wr_mix == 2) {
        hipLaunchKernelGGL((latent_mix_kernel<2, 2>), mix_grid, blk3, mix_lds, stream, ma);
    } else {
        hipLaunchKernelGGL((latent_mix_kernel<1, 4>), mix_grid, blk3, mix_lds, stream, ma);
    }

    GateArgs ga;
    ga.ub = ub;
    ga.wg = wg;
    ga.wu = wu;
    ga.m = m;
    ga.rows = (uint32_t)rows;
    ga.R = (uint32_t)R;
    ga.H = (uint32_t)H;
    ga.col_tiles = (uint32_t)(H / kTile);
    ga.row_tiles = (uint32_t)gate_rt;
    ga.xmap = gate_xmap;
    const dim3 gate_grid((uint32_t)gate_wgs);
    if (wr_gate == kStaged && gate_nh == 2) {
        hipLaunchKernelGGL((latent_gate_staged<2>), gate_grid, blk3, 0, stream, ga);
    } else if (wr_gate == kStaged) {
        hipLaunchKernelGGL((latent_gate_staged<1>), gate_grid, blk3, 0, stream, ga);
    } else if (wr_gate == 4) {
        hipLaunchKernelGGL((latent_gate_kernel<4, 1>), gate_grid, blk3, 0, stream, ga);
    } else if (wr_gate == 2) {
        hipLaunchKernelGGL((latent_gate_kernel<2, 2>), gate_grid, blk3, 0, stream, ga);
    } else {
        hipLaunchKernelGGL((latent_gate_kernel<1, 4>), gate_grid, blk3, 0, stream, ga);
    }

    DownArgs da;
    da.m = m;
    da.wd = wd;
    da.u = u;
    da.out = lat_out;
    da.rows = (uint32_t)rows;
    da.R = (uint32_t)R;
    da.H = (uint32_t)H;
    da.col_tiles = (uint32_t)ctiles;
    da.row_tiles = (uint32_t)down_rt;
    da.xmap = down_xmap;
    const dim3 down_grid((uint32_t)down_wgs);
    if (wr_down == kStaged) {
        hipLaunchKernelGGL(latent_down_staged, down_grid, blk3, 0, stream, da);
    } else if (wr_down == 4) {
        hipLaunchKernelGGL((latent_down_kernel<4, 1>), down_grid, blk3, 0, stream, da);
    } else if (wr_down == 2) {
        hipLaunchKernelGGL((latent_down_kernel<2, 2>), down_grid, blk3, 0, stream, da);
    } else {
        hipLaunchKernelGGL((latent_down_kernel<1, 4>), down_grid, blk3, 0, stream, da);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}

int xpress_latent_set_tiles(int mix, int gate, int down)
{
    for (int v : {mix, gate, down}) {
        if (v != 0 && v != 1 && v != 2 && v != 4 && v != kStaged) return XPRESS_EINVAL;
    }
    std::lock_guard<std::mutex> lk(g_tiles_mu);
    g_tiles.mix = mix;
    g_tiles.gate = gate;
    g_tiles.down = down;
    return XPRESS_OK;
}

}  // extern "C"
