// readout_gemm.hip -- readout with the refiner bias computed in place, for
// MI355X (gfx950).
//
// One Jacobi pass (XPress kernels page, module description) forms
//     logits[r, v] = base[r, v] + (x @ W2)[r, v]
// with a readout matmul whose bf16 result the fused add + argmax then
// consumes as its bias.  Here that matmul is fused into the readout: the
// bias tile comes out of the matrix cores, is rounded to bf16 exactly as the
// matmul's bf16 output would be, added to base and rounded again, and only
// the running first maximum of each row leaves the registers.  Neither the
// [rows, V] bias nor the [rows, V] logits is ever written:
//     bias[r, v]    = bf16( sum_k x[r, k] * w[v, k] )   (fp32 accumulation)
//     s[r, v]       = bf16( base[r, v] + bias[r, v] )
//     blk[n, 1 + b] = first argmax_v s[r, v],   r = n*(B-1) + b
// x is [rows, R] and w is [V, R] (the head weight, one row per id), both bf16.
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//   * the vocabulary runs along the MFMA's M dimension (A operand = a 32-id
//     slice of w), the draft rows along N (B operand = x^T): each lane's 16
//     accumulators are then 4 runs of 4 consecutive ids of ONE draft row,
//     which is what the epilogue's running maximum wants;
//   * a wave owns 32 draft rows; their x rows (R bf16 each) stay in
//     registers as the B operands for the whole launch;
//   * a workgroup of kWaves waves covers 32*kWaves rows and a contiguous range
//     of 64-id tiles; each tile of w is staged through registers into a
//     padded, double-buffered LDS tile shared by the waves, the next tile's
//     loads in flight while the current one is multiplied;
//   * the workgroups that cover the row groups of one vocabulary range are
//     placed on one XCD (workgroup b runs on XCD b mod 8), so each w tile is
//     fetched from HBM once and served from that XCD's L2 afterwards;
//   * per (row, range) the packed (value, ~id) key goes to a key table and the
//     library's second pass reduces each row's keys into blk.
// Numerics: the fp32 accumulation order of the MFMA is the hardware's; where
// every partial sum is exact (dyadic inputs) the bias equals the bf16 of the
// exact dot product bit for bit.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "xpress_argmax.h"
#include "device_common.h"
#include "host_common.h"

namespace {

using namespace xpress;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileV = 32;   // vocabulary ids per tile: one 32-id MFMA slice
constexpr int kWaves = 8;    // waves per workgroup
constexpr int kGroups = 2;   // 32-row groups per wave: they share every A operand read

struct GemmArgs {
    const uint16_t* base;
    const uint16_t* x;
    const uint16_t* w;
    uint64_t* table;       // [rows, ranges] packed keys
    int64_t stride_base;   // elements
    uint32_t rows;
    uint32_t V;
    uint32_t tiles;        // ceil(V / kTileV)
    uint32_t ranges;       // vocabulary ranges (a multiple of 8)
    uint32_t row_wgs;      // workgroups per range (row groups / kWaves)
};

// Two fp32 values rounded to bf16 (round-to-nearest-even), packed lo | hi.
__device__ __forceinline__ uint32_t round_pack2(float lo, float hi)
{
    f32x2 s;
    s.x = lo;
    s.y = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(s, bf16x2));
}

template <int R>
__global__ __launch_bounds__(kWaves * 64) void gemm_readout_kernel(GemmArgs a)
{
    constexpr int KC = R / 16;                  // MFMA steps over k
    constexpr int ROWB = R * 2 + 16;            // bytes per LDS tile row (16 B pad)
    constexpr int CHUNKS = kTileV * R / 8;      // 16-byte chunks per w tile
    constexpr int THREADS = kWaves * 64;
    constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
    constexpr int WROWS = 32 * kGroups;         // rows per wave
    constexpr int BLOADS = WROWS * kTileV * 2 / 1024;  // base copies per wave per tile
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][kTileV * ROWB];
    // base of one full tile for every row of the workgroup, two buffers
    __shared__ __attribute__((aligned(16))) uint16_t base_lds[2][kWaves * WROWS * kTileV];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t khalf = lane >> 5;
    const uint32_t b = blockIdx.x;
    const uint32_t xcd = b & 7u;
    const uint32_t local = b >> 3;
    const uint32_t range = (local / a.row_wgs) * 8u + xcd;
    const uint32_t rw = local % a.row_wgs;
    const uint32_t t0 = (uint32_t)((uint64_t)range * a.tiles / a.ranges);
    const uint32_t t1 = (uint32_t)((uint64_t)(range + 1u) * a.tiles / a.ranges);

    // this wave's rows: kGroups groups of 32; the lane's row in group g is
    // g * 32 + l % 32
    const uint32_t wrow0 = (rw * kWaves + wave) * WROWS;
    uint32_t row[kGroups];
    bool row_ok[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        row[g] = wrow0 + 32u * g + (lane & 31u);
        row_ok[g] = row[g] < a.rows;
    }

    // B operands: the lane's draft rows of x, 8 of the 16 k of every step
    bf16x8 bx[kGroups][KC];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row_ok[g]) {
                v = *reinterpret_cast<const u32x4*>(a.x + (uint64_t)row[g] * R + 16 * c + 8 * khalf);
            }
            bx[g][c] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // staging of one w tile: chunk id -> (tile row, 16-byte column)
    u32x4 stage[PER_THREAD];
    auto load_tile = [&](uint32_t t) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const uint32_t id = threadIdx.x + i * THREADS;
            const uint32_t trow = id / (R / 8);
            const uint32_t tcol = id % (R / 8);
            const uint32_t v = t * kTileV + trow;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (id < (uint32_t)CHUNKS && v < a.V) {
                val = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(a.w + (uint64_t)v * R) + tcol);
            }
            stage[i] = val;
        }
    };
    auto store_tile = [&](uint32_t buf) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const uint32_t id = threadIdx.x + i * THREADS;
            const uint32_t trow = id / (R / 8);
            const uint32_t tcol = id % (R / 8);
            if (id < (uint32_t)CHUNKS) {
                *reinterpret_cast<u32x4*>(&lds[buf][trow * ROWB + tcol * 16]) = stage[i];
            }
        }
    };

    // Running first maximum of each of this lane's rows.  It starts at the
    // lane's first id (below V whenever the range has a tile) with value -inf
    // and only a strictly larger value replaces it, so a lane whose values
    // are all -inf still reports its first id.  Lanes of rows past the last
    // row compute on zeros and never publish.
    const uint32_t first_id = t0 * kTileV + 4u * khalf;
    float best[kGroups];
    uint32_t bidx[kGroups];
    const uint16_t* brow[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        best[g] = -__builtin_inff();
        bidx[g] = (t0 < t1 && first_id < a.V) ? first_id : kNoIndex;
        // invalid rows read row 0 (always in bounds) and never update
        brow[g] = a.base + (int64_t)(row_ok[g] ? row[g] : 0u) * a.stride_base;
    }

    // tiles below full_end are full; a ragged vocabulary's last tile is not
    const uint32_t full_end = (t0 < t1 && t1 * kTileV > a.V) ? t1 - 1u : t1;

    // base of full tiles goes straight into LDS: each wave copies its own
    // rows (instruction j: rows 16j .. 16j+15 of the wave's, lane l row
    // 16j + l/4, logical 16-byte column (l % 4) ^ (row % 4)), so a load
    // instruction reads sixteen 64-byte row segments, and the wave only
    // waits for its own copies before its epilogue reads them back
    const uint16_t* bsrc[BLOADS];
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) {
        const uint32_t rl = 16u * j + (lane >> 2);
        const uint32_t r = wrow0 + rl;
        bsrc[j] = a.base + (int64_t)(r < a.rows ? r : 0u) * a.stride_base +
                  8u * ((lane & 3u) ^ (rl & 3u));
    }
    auto dma_base = [&](uint32_t t, uint32_t buf) {
#pragma unroll
        for (int j = 0; j < BLOADS; ++j) {
            dma16(bsrc[j] + (uint64_t)t * kTileV,
                  lds_addr(&base_lds[buf][(wave * WROWS + 16u * j) * kTileV]));
        }
    };

    if (t0 < t1) {
        if (t0 < full_end) dma_base(t0, t0 & 1u);
        load_tile(t0);
        store_tile(0);
    }
    __syncthreads();

    // One tile: the next tile's base (into LDS) and w (into registers) go out
    // first and stay in flight; the MFMAs run on the current LDS w tile; the
    // epilogue waits for this tile's base, copied one tile earlier; then the
    // next w tile goes into the other LDS buffer.
    auto tile = [&](uint32_t t, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const uint32_t cur = (t - t0) & 1u;
        const bool more = t + 1u < t1;
        const bool next_full = t + 1u < full_end;
        const uint32_t tv = t * kTileV;
        if (next_full) dma_base(t + 1u, (t + 1u) & 1u);
        if (more) load_tile(t + 1u);
        u32x2 bv[kGroups][4];
        if constexpr (!FULL) {
            // each id at min(id, V - 1): in bounds, masked out past V
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t v = tv + 8u * q + 4u * khalf;
                    uint32_t e[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) e[jj] = brow[g][(v + jj < a.V) ? v + jj : a.V - 1u];
                    bv[g][q].x = e[0] | (e[1] << 16);
                    bv[g][q].y = e[2] | (e[3] << 16);
                }
            }
        }

        // one A operand read feeds the kGroups independent accumulator chains
        f32x16 acc[kGroups];
#pragma unroll
        for (int g = 0; g < kGroups; ++g) acc[g] = f32x16{};
        const unsigned char* arow = &lds[cur][(lane & 31u) * ROWB + 16u * khalf];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const bf16x8 a0 =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(arow + 32 * c));
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bx[g][c], acc[g], 0, 0, 0);
            }
        }

        if constexpr (FULL) {
            // this tile's base landed once only the loads issued above remain
            if (next_full && more) {
                wait_vmcnt<BLOADS + PER_THREAD>();
            } else if (next_full) {
                wait_vmcnt<BLOADS>();
            } else if (more) {
                wait_vmcnt<PER_THREAD>();
            } else {
                wait_vmcnt<0>();
            }
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const uint32_t lrow = wave * WROWS + 32u * g + (lane & 31u);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t pc = (uint32_t)q ^ (lrow & 3u);
                    bv[g][q] = *reinterpret_cast<const u32x2*>(
                        &base_lds[t & 1u][lrow * kTileV + pc * 8u + 4u * khalf]);
                }
            }
        }

        // epilogue: bias rounded to bf16, added to base, rounded; ascending ids
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t v = tv + 8u * q + 4u * khalf;
                const uint32_t s01 =
                    add_round2(bv[g][q].x, round_pack2(acc[g][4 * q], acc[g][4 * q + 1]));
                const uint32_t s23 =
                    add_round2(bv[g][q].y, round_pack2(acc[g][4 * q + 2], acc[g][4 * q + 3]));
                const float sv[4] = {bf16_lo(s01), bf16_hi(s01), bf16_lo(s23), bf16_hi(s23)};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // ids past V exist only in a ragged last tile
                    const bool take =
                        FULL ? (sv[jj] > best[g]) : ((v + jj < a.V) && (sv[jj] > best[g]));
                    best[g] = take ? sv[jj] : best[g];
                    bidx[g] = take ? v + jj : bidx[g];
                }
            }
        }

        if (more) store_tile(cur ^ 1u);
        __syncthreads();
    };

    if (t0 < t1) {
        uint32_t t = t0;
        for (; t < full_end; ++t) tile(t, std::true_type{});
        if (t < t1) tile(t, std::false_type{});
    }

    // lanes l and l + 32 hold two halves of the same row's ids
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        const float ov = __shfl_xor(best[g], 32);
        const uint32_t oi = __shfl_xor(bidx[g], 32);
        merge(best[g], bidx[g], ov, oi);
        if (khalf == 0u && row_ok[g]) {
            a.table[(uint64_t)row[g] * a.ranges + range] = make_key(best[g], bidx[g]);
        }
    }
}

template <int R>
hipError_t launch_gemm(const GemmArgs& a, uint32_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL(gemm_readout_kernel<R>, dim3(grid), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

extern "C" int xpress_readout_gemm_argmax_to_blk(const uint16_t* base, const uint16_t* x,
                                                 const uint16_t* w, int64_t* blk, int64_t N,
                                                 int64_t B, int64_t V, int64_t R,
                                                 int64_t stride_base_r, hipStream_t stream)
{
    if (N < 0 || B < 1 || V < 1 || V > 0x7FFFFFFFll || stride_base_r < V) return XPRESS_EINVAL;
    if (R != 64 && R != 128 && R != 256) return XPRESS_EINVAL;
    if (B - 1 > 0 && N > INT64_MAX / (B - 1)) return XPRESS_EINVAL;
    const int64_t rows = N * (B - 1);
    if (rows == 0) return XPRESS_OK;
    if (rows > 0x7FFFFFFFll || N > INT64_MAX / B) return XPRESS_EINVAL;
    if (!base || !x || !w || !blk) return XPRESS_EINVAL;
    if (!is_aligned16(base) || !is_aligned16(x) || !is_aligned16(w) || stride_base_r % 8 != 0) {
        return XPRESS_EINVAL;
    }
    if ((rows - 1) > (INT64_MAX / 8 - V) / stride_base_r || V > INT64_MAX / 8 / R) {
        return XPRESS_EINVAL;
    }
    const size_t blk_bytes = (size_t)(N * B) * 8u;
    if (ranges_overlap(blk, blk_bytes, base, (size_t)((rows - 1) * stride_base_r + V) * 2u) ||
        ranges_overlap(blk, blk_bytes, x, (size_t)(rows * R) * 2u) ||
        ranges_overlap(blk, blk_bytes, w, (size_t)(V * R) * 2u)) {
        return XPRESS_EINVAL;
    }

    GemmArgs a;
    a.base = base;
    a.x = x;
    a.w = w;
    a.stride_base = stride_base_r;
    a.rows = (uint32_t)rows;
    a.V = (uint32_t)V;
    a.tiles = (uint32_t)((V + kTileV - 1) / kTileV);
    const int64_t groups = (rows + 31) / 32;
    a.row_wgs = (uint32_t)((groups + kWaves * kGroups - 1) / (kWaves * kGroups));
    // about one workgroup per CU (a workgroup fills its CU's LDS and two
    // waves per SIMD); ranges a multiple of 8 (one per XCD slot)
    int64_t ranges = (int64_t)device_cus() / a.row_wgs;
    ranges = ranges / 8 * 8;
    if (ranges < 8) ranges = 8;
    const int64_t max_ranges = ((int64_t)a.tiles + 7) / 8 * 8;
    if (ranges > max_ranges) ranges = max_ranges;
    if ((int64_t)a.row_wgs * ranges > 0x7FFFFFFFll) return XPRESS_EINVAL;
    a.ranges = (uint32_t)ranges;

    int rc = workspace_table(stream, rows * ranges, &a.table);
    if (rc != XPRESS_OK) return rc;

    const uint32_t grid = a.row_wgs * a.ranges;
    hipError_t e;
    switch (R) {
        case 64: e = launch_gemm<64>(a, grid, stream); break;
        case 128: e = launch_gemm<128>(a, grid, stream); break;
        default: e = launch_gemm<256>(a, grid, stream); break;
    }
    if (e != hipSuccess) return hip_fail(e);
    e = launch_reduce_table(a.table, blk, nullptr, a.rows, (uint32_t)(B - 1), a.V, a.ranges,
                            stream);
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}
