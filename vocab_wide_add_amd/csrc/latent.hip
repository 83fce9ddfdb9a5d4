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
//   mix   per (32 x-rows, 32 channels): the gathered embeddings times W_lat on
//         v_mfma_f32_32x32x16_bf16 with K split over 4 waves, the partials
//         summed in LDS with the hidden cache, then the folded mixer per
//         channel from an LDS copy of its slice of mixl.  Writes u (fp32) and
//         bf16(u) for the slots that are read out.
//   gate  per (32 rows, 32 hidden units): bf16(u) times wg and wu, K split
//         over 4 waves; m = bf16(silu(g) * v).
//   down  per (32 rows, 32 channels): m times wd, K split over 4 waves, plus
//         the residual u, rounded to bf16 into the output.
//
// The kernel boundaries are the cross-workgroup syncs: u and m go through a
// small workspace (L2 / MALL resident).  Each grid is 1-D with the weight
// tile index fastest, so workgroups sharing a weight slice land on the same
// XCD (workgroup i runs on XCD i % 8) and share its L2.
//
// MFMA operand layout (v_mfma_f32_32x32x16_bf16, 64 lanes): lane l supplies
// A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32], e = 0..7;
// accumulator register r of lane l holds D[8 * (r / 4) + 4 * (l / 32) + r % 4]
// [l % 32].  With both weight matrices out-major, every operand is 8
// consecutive k values: one 16-byte load per lane per step.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "device_common.h"
#include "host_common.h"
#include "xpress_argmax.h"

namespace {

using namespace xpress;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 32;      // rows and columns of one MFMA tile
constexpr int kWaves = 4;      // waves of a workgroup; they split K
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 4;      // MFMA k-steps whose operands are loaded at once
constexpr int kMaxB = 32;
constexpr int kPad = kTile + 1;  // LDS row stride of a 32 x 32 fp32 tile

__device__ __forceinline__ bf16x8 load8(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero8()
{
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ uint16_t to_bf16(float x)
{
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// acc += A[32 x K] * B[K x 32] over this wave's K range [k_begin, k_begin +
// k_len), k_len a multiple of 16.  a_row / b_row point at the row (of A) and
// the column (of B, stored as a row of the out-major weight) this lane
// supplies, or a_row is null for a padding row (zeros).
__device__ __forceinline__ void mfma_range(f32x16& acc, const uint16_t* a_row,
                                           const uint16_t* b_row, int k_begin, int k_len,
                                           int half)
{
    for (int k0 = 0; k0 < k_len; k0 += 16 * kChunk) {
        bf16x8 a[kChunk], b[kChunk];
#pragma unroll
        for (int s = 0; s < kChunk; ++s) {
            const int k = k_begin + k0 + 16 * s + 8 * half;
            const bool live = k0 + 16 * s < k_len;
            a[s] = (live && a_row) ? load8(a_row + k) : zero8();
            b[s] = live ? load8(b_row + k) : zero8();
        }
#pragma unroll
        for (int s = 0; s < kChunk; ++s) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc, 0, 0, 0);
        }
    }
}

// Store this wave's accumulator tile into part[32][kPad] (fp32).
__device__ __forceinline__ void store_tile(float* part, const f32x16& acc, int lane)
{
    const int col = lane & 31;
    const int row0 = 4 * (lane >> 5);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        part[(8 * (r >> 2) + row0 + (r & 3)) * kPad + col] = acc[r];
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
};

// One workgroup per (tile of bpt whole blocks = bpt * B x-rows, 32 channels).
__global__ void __launch_bounds__(kThreads) latent_mix_kernel(MixArgs a)
{
    __shared__ float part[kWaves][kTile * kPad];
    __shared__ uint16_t xhs[kTile * kTile];
    extern __shared__ u32x4 mixs_dyn[];  // [B * B][32] bf16 slice of mixl
    const uint16_t* mixs = reinterpret_cast<const uint16_t*>(mixs_dyn);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const uint32_t ct = blockIdx.x % a.col_tiles;
    const uint32_t rt = blockIdx.x / a.col_tiles;
    const uint32_t c0 = ct * kTile;
    const uint32_t B = a.B, R = a.R;
    const uint32_t n0 = rt * a.bpt;
    const uint32_t nb = (a.N - n0 < a.bpt) ? (a.N - n0) : a.bpt;
    const uint32_t rows = nb * B;  // valid x-rows of the tile

    // the mixer slice [B*B rows of 32 channels] and the cache tile to LDS
    const uint32_t mix_chunks = B * B * 4;  // 16-byte chunks
    for (uint32_t q = tid; q < mix_chunks; q += kThreads) {
        const uint32_t row = q >> 2, part16 = q & 3;
        mixs_dyn[q] = *reinterpret_cast<const u32x4*>(a.mixl + (size_t)row * R + c0 + 8 * part16);
    }
    if (tid < kTile * 4) {
        const uint32_t i = tid >> 2, part16 = tid & 3;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (i < rows) {
            v = *reinterpret_cast<const u32x4*>(a.xh + ((size_t)n0 * B + i) * R + c0 + 8 * part16);
        }
        *reinterpret_cast<u32x4*>(xhs + i * kTile + 8 * part16) = v;
    }

    // x-row this lane supplies to A: the embedding of the previous token
    const uint32_t i = lane & 31;
    const uint16_t* a_row = nullptr;
    if (i < rows) {
        const uint32_t lb = i / B, slot = i % B;
        const uint32_t n = n0 + lb;
        const int64_t tok = (slot == 0) ? a.am1[n] : a.blk[(size_t)n * B + slot - 1];
        // an id outside [0, V) reads as a zero embedding row
        if (tok >= 0 && tok < a.V) a_row = a.w1 + (size_t)tok * R;
    }
    const uint16_t* b_row = a.wlat + (size_t)(c0 + i) * R;
    const int k_len = (int)(R / kWaves);
    f32x16 acc = {};
    mfma_range(acc, a_row, b_row, wave * k_len, k_len, half);
    store_tile(part[wave], acc, lane);
    __syncthreads();

    // x = cache + sum of the 4 K-partials, kept in part[0]
    for (int e = tid; e < kTile * kTile; e += kThreads) {
        const int r = e >> 5, c = e & 31;
        const int o = r * kPad + c;
        const float x = ((part[0][o] + part[1][o]) + (part[2][o] + part[3][o])) +
                        from_bf16(xhs[r * kTile + c]);
        part[0][o] = x;
    }
    __syncthreads();

    // folded mixer for the slots read out: u[b] = sum_j mixl[b, j] * x[j]
    const uint32_t bm1 = B - 1;
    const uint32_t outs = nb * bm1 * kTile;
    for (uint32_t e = tid; e < outs; e += kThreads) {
        const uint32_t c = e & 31, q = e >> 5;
        const uint32_t lb = q / bm1, b = 1 + q % bm1;
        const float* xcol = &part[0][lb * B * kPad + c];
        const uint16_t* mrow = mixs + (size_t)b * B * kTile + c;
        float u = 0.0f;
        for (uint32_t j = 0; j < B; ++j) {
            u = fmaf(from_bf16(mrow[j * kTile]), xcol[j * kPad], u);
        }
        const size_t row_out = (size_t)(n0 + lb) * bm1 + (b - 1);
        a.u[row_out * R + c0 + c] = u;
        a.ub[row_out * R + c0 + c] = to_bf16(u);
    }
}

struct GateArgs {
    const uint16_t* ub;  // [rows, R]
    const uint16_t* wg;  // [H, R]
    const uint16_t* wu;  // [H, R]
    uint16_t* m;         // [rows, H]
    uint32_t rows, R, H, col_tiles;
};

// One workgroup per (32 rows, 32 hidden units).
__global__ void __launch_bounds__(kThreads) latent_gate_kernel(GateArgs a)
{
    __shared__ float part[2][kWaves][kTile * kPad];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const uint32_t ht = blockIdx.x % a.col_tiles;
    const uint32_t rt = blockIdx.x / a.col_tiles;
    const uint32_t h0 = ht * kTile, i0 = rt * kTile;
    const uint32_t i = lane & 31;
    const uint16_t* a_row = (i0 + i < a.rows) ? a.ub + (size_t)(i0 + i) * a.R : nullptr;
    const int k_len = (int)(a.R / kWaves);
    f32x16 g = {}, v = {};
    mfma_range(g, a_row, a.wg + (size_t)(h0 + i) * a.R, wave * k_len, k_len, half);
    mfma_range(v, a_row, a.wu + (size_t)(h0 + i) * a.R, wave * k_len, k_len, half);
    store_tile(part[0][wave], g, lane);
    store_tile(part[1][wave], v, lane);
    __syncthreads();
    for (int e = tid; e < kTile * kTile; e += kThreads) {
        const int r = e >> 5, c = e & 31;
        if (i0 + r >= a.rows) continue;
        const int o = r * kPad + c;
        const float gs = (part[0][0][o] + part[0][1][o]) + (part[0][2][o] + part[0][3][o]);
        const float vs = (part[1][0][o] + part[1][1][o]) + (part[1][2][o] + part[1][3][o]);
        const float f = gs / (1.0f + expf(-gs)) * vs;
        a.m[(size_t)(i0 + r) * a.H + h0 + c] = to_bf16(f);
    }
}

struct DownArgs {
    const uint16_t* m;   // [rows, H]
    const uint16_t* wd;  // [R, H]
    const float* u;      // [rows, R]
    uint16_t* out;       // [rows, R]
    uint32_t rows, R, H, col_tiles;
};

// One workgroup per (32 rows, 32 channels).
__global__ void __launch_bounds__(kThreads) latent_down_kernel(DownArgs a)
{
    __shared__ float part[kWaves][kTile * kPad];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
    const uint32_t ct = blockIdx.x % a.col_tiles;
    const uint32_t rt = blockIdx.x / a.col_tiles;
    const uint32_t c0 = ct * kTile, i0 = rt * kTile;
    const uint32_t i = lane & 31;
    const uint16_t* a_row = (i0 + i < a.rows) ? a.m + (size_t)(i0 + i) * a.H : nullptr;
    const int k_len = (int)(a.H / kWaves);
    f32x16 acc = {};
    mfma_range(acc, a_row, a.wd + (size_t)(c0 + i) * a.H, wave * k_len, k_len, half);
    store_tile(part[wave], acc, lane);
    __syncthreads();
    for (int e = tid; e < kTile * kTile; e += kThreads) {
        const int r = e >> 5, c = e & 31;
        if (i0 + r >= a.rows) continue;
        const int o = r * kPad + c;
        const size_t idx = (size_t)(i0 + r) * a.R + c0 + c;
        const float mm = (part[0][o] + part[1][o]) + (part[2][o] + part[3][o]);
        a.out[idx] = to_bf16(a.u[idx] + mm);
    }
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
    ma.bpt = (uint32_t)(kTile / B);
    ma.col_tiles = (uint32_t)(R / kTile);
    const uint64_t mix_tiles = (uint64_t)((N + ma.bpt - 1) / ma.bpt) * ma.col_tiles;
    const uint64_t row_tiles = (uint64_t)((rows + kTile - 1) / kTile);
    const uint64_t gate_wgs = row_tiles * (uint64_t)(H / kTile);
    const uint64_t down_wgs = row_tiles * (uint64_t)(R / kTile);
    if (mix_tiles > 0x7FFFFFFFull || gate_wgs > 0x7FFFFFFFull || down_wgs > 0x7FFFFFFFull) {
        return XPRESS_EINVAL;
    }
    const size_t mix_lds = (size_t)B * B * kTile * 2u;
    if (mix_lds > 32768u) {
        // the mixer slice of a large block size takes most of the LDS (up to
        // 64 KiB at B = 32, beside 18.5 KiB of static LDS)
        hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(&latent_mix_kernel),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)mix_lds);
        if (ea != hipSuccess) return hip_fail(ea);
    }
    hipLaunchKernelGGL(latent_mix_kernel, dim3((uint32_t)mix_tiles), dim3(kThreads), mix_lds,
                       stream, ma);

    GateArgs ga;
    ga.ub = ub;
    ga.wg = wg;
    ga.wu = wu;
    ga.m = m;
    ga.rows = (uint32_t)rows;
    ga.R = (uint32_t)R;
    ga.H = (uint32_t)H;
    ga.col_tiles = (uint32_t)(H / kTile);
    hipLaunchKernelGGL(latent_gate_kernel, dim3((uint32_t)gate_wgs), dim3(kThreads), 0, stream,
                       ga);

    DownArgs da;
    da.m = m;
    da.wd = wd;
    da.u = u;
    da.out = lat_out;
    da.rows = (uint32_t)rows;
    da.R = (uint32_t)R;
    da.H = (uint32_t)H;
    da.col_tiles = (uint32_t)(R / kTile);
    hipLaunchKernelGGL(latent_down_kernel, dim3((uint32_t)down_wgs), dim3(kThreads), 0, stream,
                       da);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}

}  // extern "C"
