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
//   * a wave owns 64 draft rows (two 32-row groups whose matrix instructions
//     share every A-operand read); their x rows stay in registers as the B
//     operands for the whole launch;
//   * a workgroup of 8 waves covers 512 rows (above 128 rows; 2 waves up to
//     128 rows, 1 wave up to 64) and a contiguous range of 32-id tiles; w
//     tiles and each wave's base tiles are copied straight into LDS by the
//     16-byte load-to-LDS instruction, two tiles ahead in rings of three
//     (three ahead in a ring of four for one wave), and each wave waits only
//     on its own copies (explicit counts) before the one barrier per tile;
//   * all waves run the same phase together (matrix instructions, then the
//     epilogue): measured on this part, a SIMD's two waves retire matrix
//     instructions faster together than one alone, and vector instructions
//     likewise, while the two kinds from different waves slow each other;
//   * the workgroups that cover the row groups of one vocabulary range are
//     placed on one XCD (workgroup b runs on XCD b mod 8), so each w tile is
//     fetched from HBM once and served from that XCD's L2 afterwards;
//   * in the 2- and 8-wave shapes the epilogue keeps a tile's first maximum
//     in one integer max per logit: a widened bf16 sum has 16 zero low bits,
//     which take a tag that falls with the id's position in the tile, so
//     among equal values the earlier id has the larger bit pattern; the
//     running (value, id) is updated once per tile.  For positive values the
//     bit patterns order as the values do (+inf included), so this is exact
//     wherever a lane's maximum over its range is positive; a workgroup in
//     which some lane's maximum is not (zero, negative, -inf) runs its range
//     again with the per-logit compare-and-select epilogue, which is exact
//     for every value and is the one-wave shape's only epilogue;
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
constexpr int kWavesMax = 8; // waves per workgroup above 128 rows (512 rows each)
constexpr int kGroups = 2;   // 32-row groups per wave: they share every A operand read
constexpr int kAhead = 4;    // A-operand registers: reads run three steps ahead

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
    uint32_t row_wgs;      // workgroups per range
    uint32_t reverse;      // nonzero: workgroups mapped last to first
};

// The row of a 32-row group whose B operand (x) or A operand (w) lane l
// carries.
__device__ __forceinline__ uint32_t arow_x(uint32_t lane) { return lane & 31u; }

// s_waitcnt lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

// Two fp32 values rounded to bf16 (round-to-nearest-even), packed lo | hi.
__device__ __forceinline__ uint32_t round_pack2(float lo, float hi)
{
    f32x2 s;
    s.x = lo;
    s.y = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(s, bf16x2));
}

// Order-preserving map of two packed bf16 patterns: each half, sign and
// magnitude, becomes the 16-bit two's complement integer +magnitude or
// -magnitude, so that as signed integers the halves order as the values do,
// with -0 and +0 both 0 (equal, as the values compare) and a NaN with the
// sign set below -inf.
__device__ __forceinline__ uint32_t ord_pair(uint32_t p)
{
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const s16x2 sign = __builtin_bit_cast(s16x2, p) >> (s16x2){15, 15};  // 0 or -1
    const s16x2 mag = __builtin_bit_cast(s16x2, p & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, (s16x2)((mag ^ sign) - sign));
}

// Inverse of ord_pair on the high half of a word whose low half is zero:
// the bf16 pattern of the value in the high half (-0 comes back as +0).
__device__ __forceinline__ uint32_t unord_hi(uint32_t w)
{
    const int32_t o = (int32_t)w >> 16;  // sign-extended 16-bit integer
    const uint32_t h = o < 0 ? (0x8000u | (uint32_t)(-o)) : (uint32_t)o;
    return h << 16;
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (the
// instruction takes an immediate): a chain of compares down from N; n above
// N waits for all.
template <int N>
__device__ __forceinline__ void wait_vmcnt_dyn(int n)
{
    if constexpr (N <= 0) {
        wait_vmcnt<0>();
    } else {
        if (n == N) {
            wait_vmcnt<N>();
        } else {
            wait_vmcnt_dyn<N - 1>(n);
        }
    }
}

// KW waves per workgroup (64 rows each): 8 with one workgroup per CU, or 1
// or 2 (64 or 128 rows) with two per CU, so that few rows do not pay for 512.
// RING tiles of w and base sit in LDS; copies run RING - 1 tiles ahead.
template <int R, int KW, int RING>
__global__ __launch_bounds__(KW * 64) void gemm_readout_kernel(GemmArgs a)
{
    constexpr int kWaves = KW;
    constexpr int kRing = RING;
    constexpr int AHEAD = RING - 1;
    constexpr int KC = R / 16;                  // MFMA steps over k
    constexpr int ROWB = R * 2;                 // bytes per w row in LDS
    constexpr int CPR = R / 8;                  // 16-byte chunks per w row
    constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;  // chunk swizzle mask
    constexpr int WBYTES = kTileV * ROWB;       // one w tile
    constexpr int TW = WBYTES / 1024;           // load-to-LDS copies per w tile
    constexpr int WPW = TW >= kWaves ? TW / kWaves : 1;  // copies per issuing wave
    constexpr int WROWS = 32 * kGroups;         // rows per wave
    constexpr int BLOADS = WROWS * kTileV * 2 / 1024;  // base copies per wave per tile
    static_assert(WPW * kWaves == TW || (TW < kWaves && WPW == 1 && kWaves % TW == 0),
                  "w copies split over waves");
    static_assert(BLOADS * 1024 == WROWS * kTileV * 2, "base copies cover the wave's rows");
    constexpr int BBYTES = kWaves * WROWS * kTileV * 2;  // one base tile, all waves
    constexpr int XBYTES = 32 * R * 2;          // x of one 32-row group
    static_assert(WBYTES + kWaves * XBYTES <= kRing * (WBYTES + BBYTES),
                  "x staging fits beside w buffer 0");
    // One LDS block: the w ring (kRing tiles; row i of a tile, one id, at
    // i * ROWB, its 16-byte chunk j at position j ^ (i & SWZ), so the 16 rows
    // one matrix-operand read touches sit in 16 different bank groups), then
    // the base ring (one full tile for each wave's rows).  At start, the
    // bytes past w buffer 0 hold each wave's x in turn (same swizzle).
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kRing * (WBYTES + BBYTES)];
    auto w_buf = [&](int buf) -> unsigned char* { return lds + buf * WBYTES; };
    auto base_buf = [&](int buf) -> uint16_t* {
        return reinterpret_cast<uint16_t*>(lds + kRing * WBYTES + buf * BBYTES);
    };

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t khalf = lane >> 5;
    // (reversed, the grid's last workgroup takes the first pair; the grid is
    // a multiple of 8, so a range's workgroups still share an XCD)
    const uint32_t b = a.reverse ? gridDim.x - 1u - blockIdx.x : blockIdx.x;
    const uint32_t xcd = b & 7u;
    const uint32_t local = b >> 3;
    const uint32_t range = (local / a.row_wgs) * 8u + xcd;
    const uint32_t rw = local % a.row_wgs;
    const uint32_t t0 = (uint32_t)((uint64_t)range * a.tiles / a.ranges);
    // The first tile as the copies see it.  Before the exact rerun it is
    // passed through an empty asm statement, so the rerun's copy addresses
    // are computed afresh instead of being kept in registers (the compiler
    // would otherwise hold the prologue's 64-bit addresses across the whole
    // range for it).
    uint32_t t0c = t0;
    const uint32_t t1 = (uint32_t)((uint64_t)(range + 1u) * a.tiles / a.ranges);
    const int T = (int)(t1 - t0);
    // tiles below Tfull are full; a ragged vocabulary's last tile is not
    // (an opaque scalar: the compiler would otherwise keep the comparison
    // with T as a per-lane flag across the whole range)
    int Tfull = (T > 0 && t1 * kTileV > a.V) ? T - 1 : T;
    asm volatile("" : "+s"(Tfull));

    // this wave's rows: kGroups groups of 32; the lane's row in group g is
    // g * 32 + l % 32.  The slab a wave takes rotates with the workgroup's
    // slot on its XCD, so the compute units of one XCD, which all load every
    // x row at start, do not all ask for the same rows at the same time.
    const uint32_t slab = (wave + local) % (uint32_t)kWaves;
    const uint32_t wrow0 = (rw * kWaves + slab) * WROWS;
    uint32_t row[kGroups];
    bool row_ok[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        row[g] = wrow0 + 32u * g + (lane & 31u);
        row_ok[g] = row[g] < a.rows;
    }

    // --- copies into LDS -------------------------------------------------
    // Source addresses are formed at each copy (a few integer operations per
    // copy) rather than kept in registers, which the x operands fill.
    // base: each wave copies its own rows (instruction j: rows 16j .. 16j+15
    // of the wave's, lane l row 16j + l/4, logical 16-byte column
    // (l % 4) ^ ((row / 4) % 4)); only that wave reads them back.  A row is
    // 64 bytes, so rows 4 apart share LDS banks: keying the swizzle on
    // row / 4 spreads the 32 rows of one epilogue read over all 16 bank
    // groups (two rows each) where row % 4 left 8 rows on each of 4.  Rows
    // past the last read the last row and are never used.
    const uint32_t b_lrow = lane >> 2;
    const uint32_t b_col = 8u * ((lane & 3u) ^ ((b_lrow >> 2) & 3u));
    auto dma_base = [&](uint32_t t, int buf) {
#pragma unroll
        for (int j = 0; j < BLOADS; ++j) {
            uint32_t r = wrow0 + 16u * j + b_lrow;
            r = r < a.rows ? r : a.rows - 1u;
            dma16(a.base + (uint64_t)r * (uint64_t)a.stride_base + b_col + (uint64_t)t * kTileV,
                  lds_addr(base_buf(buf) + (wave * WROWS + 16u * j) * kTileV));
        }
    };
    // w: copy m of a tile fills LDS bytes [1024 m, 1024 m + 1024) with 64
    // chunks (tile row q / CPR, position q % CPR for q = 64 m + lane); wave
    // w issues copies (w * WPW + k) mod TW (at R = 64 the last four waves
    // repeat the first four's, so that every wave issues the same count)
    auto dma_w = [&](uint32_t t, int buf) {
#pragma unroll
        for (int k = 0; k < WPW; ++k) {
            const uint32_t m = (wave * WPW + k) % (uint32_t)TW;
            const uint32_t q = 64u * m + lane;
            const uint32_t i = q / CPR;
            const uint32_t p = q % CPR;
            uint32_t v = t * kTileV + i;
            v = v < a.V ? v : a.V - 1u;        // ids past V: any row, masked later
            dma16(a.w + (uint64_t)v * R + 8u * (p ^ (i & (uint32_t)SWZ)),
                  lds_addr(reinterpret_cast<const uint16_t*>(w_buf(buf) + 1024u * m)));
        }
    };

    // Copy schedule: during tile j every wave copies base tile j + AHEAD (if
    // full; at the start of the tile) and its share of w tile j + AHEAD
    // (between the two row groups' epilogues), into the ring buffer tile j - 1
    // has just left; the copies of tiles 0 .. AHEAD - 1 go out before the
    // loop.  n_copies(j) counts the wave's copies during tile j, base before
    // w; the wait at the end of tile j (everything but the copies of the
    // AHEAD - 1 latest tiles) lands tile j + 1 for the barrier.
    auto n_copies = [&](int j) -> int {
        const int tt = j + AHEAD;
        if (tt < 0 || tt >= T) return 0;
        return (tt < Tfull ? BLOADS : 0) + WPW;
    };
    auto issue_base = [&](int j) {
        const int tt = j + AHEAD;
        if (tt >= 0 && tt < Tfull) dma_base(t0c + (uint32_t)tt, tt % kRing);
    };
    auto issue_w = [&](int j) {
        const int tt = j + AHEAD;
        if (tt >= 0 && tt < T) dma_w(t0c + (uint32_t)tt, tt % kRing);
    };
    constexpr int kMaxCount = (AHEAD - 1) * (BLOADS + WPW);
    static_assert(kMaxCount < 64, "wait counts fit vmcnt");
    auto issue = [&](int j) {
        issue_base(j);
        issue_w(j);
    };
    // Prologue.  x is read into registers through LDS: each wave copies one
    // 32-row group at a time (16-byte load-to-LDS, whole rows, so every copy
    // reads contiguous memory; direct loads in the matrix layout would touch
    // 32 rows per instruction and cost many more requests) into its own
    // region past w buffer 0, then reads the B operands back.  w tile 0 is
    // copied meanwhile; base tile 0 and tiles 1 .. AHEAD - 1 follow once
    // every wave is done with its region, in the order the loop's wait
    // counts assume.
    issue_w(-AHEAD);
    unsigned char* xstage = w_buf(1) + wave * XBYTES;
    // a wave whose second row group lies wholly past the last row skips it
    // (wave-uniform), here and in every tile
    const bool g1 = wrow0 + 32u < a.rows;
    bf16x8 bx[kGroups][KC];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        if (g == 1 && !g1) break;
        // copy m: 64 chunks, row r = q / CPR of the group, position q % CPR
        // holds logical chunk (q % CPR) ^ (r & SWZ), for q = 64 m + lane;
        // rows past the last read the last row and never publish
#pragma unroll
        for (int m = 0; m < XBYTES / 1024; ++m) {
            const uint32_t q = 64u * m + lane;
            const uint32_t r = q / CPR;
            const uint32_t p = q % CPR;
            uint32_t srow = wrow0 + 32u * g + r;
            srow = srow < a.rows ? srow : a.rows - 1u;
            dma16(a.x + (uint64_t)srow * R + 8u * (p ^ (r & (uint32_t)SWZ)),
                  lds_addr(reinterpret_cast<const uint16_t*>(xstage + 1024u * m)));
        }
        wait_vmcnt<0>();
        const unsigned char* xrow = xstage + arow_x(lane) * ROWB;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const uint32_t pos = (2u * c) ^ (khalf ^ (arow_x(lane) & (uint32_t)SWZ));
            bx[g][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xrow + 16u * pos));
        }
        // the reads land before the region is copied over again
        wait_lgkmcnt0();
    }
    __syncthreads();
    issue_base(-AHEAD);
    int later = 0;
    for (int j = 1 - AHEAD; j < 0; ++j) {
        issue(j);
        later += n_copies(j);
    }
    // base tile 0 has landed once only the later tiles' copies remain (w
    // tile 0 landed with x)
    wait_vmcnt_dyn<kMaxCount>(later);

    // Running first maximum of each of this lane's rows, ids held relative
    // to t0 * kTileV + 4 khalf (tile-uniform candidates, no per-lane id
    // registers).  It starts at the lane's first id (below V whenever the
    // range has a tile) with value -inf and only a strictly larger value
    // replaces it, so a lane whose values are all -inf still reports its
    // first id.  Lanes of rows past the last row never publish.
    const uint32_t first_id = t0 * kTileV + 4u * khalf;
    float best[kGroups];
    uint32_t bidx[kGroups];
    auto reset_best = [&]() {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            best[g] = -__builtin_inff();
            bidx[g] = (T > 0 && first_id < a.V) ? 0u : kNoIndex;
        }
    };
    reset_best();

    f32x16 acc[kGroups];
    // Base of group g's rows in tile i, four consecutive ids per entry: from
    // LDS for a full tile, straight from memory for the ragged last tile
    // (each id at min(id, V - 1); rows past the last read row 0 and never
    // publish).
    auto load_bv = [&](int g, int i, uint32_t tv, auto full_tag, u32x2 (&bv)[4]) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        if constexpr (FULL) {
            const uint32_t lrow = wave * WROWS + 32u * g + (lane & 31u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t pc = (uint32_t)q ^ ((lrow >> 2) & 3u);
                bv[q] = *reinterpret_cast<const u32x2*>(
                    base_buf(i % kRing) + lrow * kTileV + pc * 8u + 4u * khalf);
            }
        } else {
            const uint16_t* brow = a.base + (int64_t)(row_ok[g] ? row[g] : 0u) * a.stride_base;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t v = tv + 8u * q + 4u * khalf;
                uint32_t e[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) e[jj] = brow[(v + jj < a.V) ? v + jj : a.V - 1u];
                bv[q].x = e[0] | (e[1] << 16);
                bv[q].y = e[2] | (e[3] << 16);
            }
        }
    };

    const uint32_t arow = lane & 31u;
    const uint32_t aswz = (khalf ^ (arow & (uint32_t)SWZ));
    __syncthreads();
    // Epilogue modes.  EXACT: compare and select per logit, exact for every
    // value.  TAGGED: the sum's bf16 bits in the high half of a word and
    // 31 - (position in the tile) in the low half (positions 8q + jj; the
    // lane's 4 khalf is in first_id), one signed integer max per logit: the
    // tile's largest value and, among equal ones, its first position --
    // exact where the lane's maximum is positive and not NaN.  ORD: the same
    // after the order-preserving map of the bf16 halves, exact for every
    // value but NaN.
    constexpr int kExact = 0, kTaggedRaw = 1, kTaggedOrd = 2;
    bool ord_mode = false;
    // Running best in the tagged modes: the high half of the (mapped) sum's
    // word, tag cleared, as an int32; below every candidate at the start.
    auto reset_best_mode = [&](auto mode_tag) __attribute__((always_inline)) {
        reset_best();
        if constexpr (decltype(mode_tag)::value == kTaggedOrd) {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) best[g] = __int_as_float(INT32_MIN);
        }
    };
    // The epilogue of row group g on tile i (accumulators in acc[g]).
    auto epi_group = [&](int g, int i, uint32_t tv, auto full_tag, auto mode_tag) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_tag)::value;
        constexpr int MODE = decltype(mode_tag)::value;
        u32x2 bv[4];
        load_bv(g, i, tv, full_tag, bv);
        if constexpr (MODE == kExact) {
            // Within the tile a candidate's id is its position in the tile,
            // an immediate operand of the select (a wave-uniform id would
            // have to be copied into a vector register for every candidate:
            // a select reads at most one scalar operand, and the condition is
            // one); the running id is held relative to the tile meanwhile
            // (wrapping arithmetic) and restored after the tile.
            float tb = best[g];
            uint32_t tp = bidx[g] - (uint32_t)(kTileV * i);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t s01 =
                    add_round2(bv[q].x, round_pack2(acc[g][4 * q], acc[g][4 * q + 1]));
                const uint32_t s23 =
                    add_round2(bv[q].y, round_pack2(acc[g][4 * q + 2], acc[g][4 * q + 3]));
                const float sv[4] = {bf16_lo(s01), bf16_hi(s01), bf16_lo(s23), bf16_hi(s23)};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // ids past V exist only in a ragged last tile
                    const bool take =
                        FULL ? (sv[jj] > tb)
                             : ((tv + 8u * q + 4u * khalf + jj < a.V) && (sv[jj] > tb));
                    tb = take ? sv[jj] : tb;
                    tp = take ? (uint32_t)(8 * q + jj) : tp;
                }
            }
            best[g] = tb;
            bidx[g] = tp + (uint32_t)(kTileV * i);
        } else {
            // The tile's maximum meets the running one with its tag cleared,
            // so an equal value from a later tile does not replace it.
            int32_t m = INT32_MIN;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t s01 = add_round2(bv[q].x, round_pack2(acc[g][4 * q], acc[g][4 * q + 1]));
                uint32_t s23 =
                    add_round2(bv[q].y, round_pack2(acc[g][4 * q + 2], acc[g][4 * q + 3]));
                if constexpr (MODE == kTaggedOrd) {
                    s01 = ord_pair(s01);
                    s23 = ord_pair(s23);
                }
                const int32_t tagged[4] = {
                    (int32_t)((s01 << 16) | (uint32_t)(31 - 8 * q)),
                    (int32_t)((s01 & 0xFFFF0000u) | (uint32_t)(30 - 8 * q)),
                    (int32_t)((s23 << 16) | (uint32_t)(29 - 8 * q)),
                    (int32_t)((s23 & 0xFFFF0000u) | (uint32_t)(28 - 8 * q))};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // ids past V exist only in a ragged last tile
                    const int32_t c =
                        FULL ? tagged[jj]
                             : ((tv + 8u * q + 4u * khalf + jj < a.V) ? tagged[jj] : INT32_MIN);
                    m = m > c ? m : c;
                }
            }
            const int32_t mv = (int32_t)((uint32_t)m & 0xFFFF0000u);
            const int32_t tb = __float_as_int(best[g]);
            const bool take = mv > tb;
            best[g] = take ? __int_as_float(mv) : best[g];
            bidx[g] = take ? (uint32_t)(kTileV * i) + (31u - ((uint32_t)m & 0xFFFFu)) : bidx[g];
        }
    };

    // One tile: copies two tiles ahead; the matrix instructions on w tile i
    // (one A-operand read feeds both row groups); the epilogue (bias rounded
    // to bf16, added to base, rounded, compared); then the wait that lands
    // tile i + 1 and the barrier.  All waves run the same phase together: on
    // this part a SIMD's two waves issue matrix instructions faster together
    // than one alone, and vector instructions likewise, while the two kinds
    // from different waves slow each other down.  Full tiles run in the loop;
    // a ragged last tile runs after it, where x is no longer live, so its
    // clamped loads do not compete with x for registers.
    auto step = [&](int i, auto full_tag, auto steady_tag, auto ng_tag, auto mode_tag) __attribute__((always_inline)) {
        constexpr int NG = decltype(ng_tag)::value;  // row groups in use
        // steady: tile i + AHEAD exists and is full, so the copies and the
        // wait count are the fixed ones and the body has no branches
        constexpr bool STEADY = decltype(steady_tag)::value;
        const uint32_t tv = (t0 + (uint32_t)i) * kTileV;
        // base copies now, w copies between the two groups' epilogues: each
        // wave's copies go to the address unit in two smaller bursts
        if constexpr (STEADY) {
            dma_base(t0c + (uint32_t)(i + AHEAD), (i + AHEAD) % kRing);
        } else {
            issue_base(i);
        }
        const unsigned char* wrow = w_buf(i % kRing) + arow * ROWB;
        // logical chunk 2c + khalf of the lane's w row sits at position
        // (2c + khalf) ^ (row & SWZ)
        auto a_op = [&](int c) {
            const uint32_t pos = (2u * c) ^ aswz;
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wrow + 16u * pos));
        };
        // A operands read kAhead steps ahead into rotating registers; one read
        // feeds both row groups' matrix instructions; a scheduling barrier
        // after each step keeps that order.
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = f32x16{};
        bf16x8 ar[kAhead];
#pragma unroll
        for (int c = 0; c < kAhead - 1 && c < KC; ++c) ar[c] = a_op(c);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            if (c + kAhead - 1 < KC) ar[(c + kAhead - 1) % kAhead] = a_op(c + kAhead - 1);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                acc[g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[c % kAhead], bx[g][c], acc[g],
                                                                 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // The epilogue starts after the last matrix instruction: the vector
        // work is not spread between them (on this part vector and matrix
        // instructions interleaved in one wave slow each other beyond a few
        // per step).
        if constexpr (NG == 2) {
            asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
        } else {
            asm volatile("" : "+v"(acc[0]));
        }
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            if (g == 1) {
                if constexpr (STEADY) {
                    dma_w(t0c + (uint32_t)(i + AHEAD), (i + AHEAD) % kRing);
                } else {
                    issue_w(i);
                }
            }
            if (g >= NG) break;
            epi_group(g, i, tv, full_tag, mode_tag);
        }
        // tile i + 1 went out during tile i + 1 - AHEAD; only the copies of
        // the tiles after that may remain
        if constexpr (STEADY) {
            wait_vmcnt<kMaxCount>();
        } else {
            if (i + 1 < T) {
                int later = 0;
                for (int j = i + 2 - AHEAD; j <= i; ++j) later += n_copies(j);
                wait_vmcnt_dyn<kMaxCount>(later);
            }
        }
        __syncthreads();
    };
    // Tiles i0 .. T - 1 in one epilogue mode.
    auto run_from = [&](int i0, auto ng_tag, auto mode_tag) __attribute__((always_inline)) {
        int i = i0;
        for (; i + AHEAD < Tfull; ++i)
            step(i, std::true_type{}, std::true_type{}, ng_tag, mode_tag);
        for (; i < Tfull; ++i) step(i, std::true_type{}, std::false_type{}, ng_tag, mode_tag);
        if (Tfull < T && T - 1 >= i0)
            step(T - 1, std::false_type{}, std::false_type{}, ng_tag, mode_tag);
    };
    // Tile 0 alone, in whichever of the loop's shapes it has.
    auto step0 = [&](auto ng_tag, auto mode_tag) __attribute__((always_inline)) {
        if (AHEAD < Tfull) {
            step(0, std::true_type{}, std::true_type{}, ng_tag, mode_tag);
        } else if (0 < Tfull) {
            step(0, std::true_type{}, std::false_type{}, ng_tag, mode_tag);
        } else {
            step(0, std::false_type{}, std::false_type{}, ng_tag, mode_tag);
        }
    };
    // The 2- and 8-wave shapes take a tagged epilogue (measured: 61.0 ->
    // 57.7 us at 480 rows, 29.1 -> 28.6 us at 120 rows): after tile 0 the
    // workgroup votes on whether every lane's maximum so far is positive.
    // If so the raw-bit tags are exact for the whole range (a lane's maximum
    // only grows); if not -- negative logits, e.g. log-probabilities -- tile
    // 0's epilogue runs again in the order-preserving mode from the
    // accumulators and the base tile still in place (no copy of tile 0 + 2
    // AHEAD has been issued into its buffer yet) and the rest of the range
    // follows in that mode.  The one-wave shape, which is bound by streaming
    // w, keeps the compare-and-select epilogue alone (the tagged loops made
    // it slower: 342 instead of 292 registers, 18.6 -> 29.4 us at 15 rows).
    constexpr bool kTagged = (KW >= 2);
    auto run_tagged = [&](auto ng_tag) __attribute__((always_inline)) {
        if (T <= 0) return;
        step0(ng_tag, std::integral_constant<int, kTaggedRaw>{});
        bool nonpos = false;
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
            nonpos |= row_ok[g] && bidx[g] != kNoIndex && __float_as_int(best[g]) <= 0;
        // (a range of one ragged tile has no later tiles to switch for: the
        // check after the range covers it)
        if (__syncthreads_or(nonpos) && 0 < Tfull) {
            ord_mode = true;
            reset_best_mode(std::integral_constant<int, kTaggedOrd>{});
            const uint32_t tv0 = t0 * kTileV;
#pragma unroll
            for (int g = 0; g < decltype(ng_tag)::value; ++g)
                epi_group(g, 0, tv0, std::true_type{}, std::integral_constant<int, kTaggedOrd>{});
            run_from(1, ng_tag, std::integral_constant<int, kTaggedOrd>{});
        } else {
            run_from(1, ng_tag, std::integral_constant<int, kTaggedRaw>{});
        }
    };
    if constexpr (kTagged) {
        if (g1) {
            run_tagged(std::integral_constant<int, 2>{});
        } else {
            run_tagged(std::integral_constant<int, 1>{});
        }
    } else {
        if (g1) {
            run_from(0, std::integral_constant<int, 2>{}, std::integral_constant<int, kExact>{});
        } else {
            run_from(0, std::integral_constant<int, 1>{}, std::integral_constant<int, kExact>{});
        }
    }
    // Back to plain bf16 bit patterns in the high half (the low half is zero).
    if (ord_mode) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) best[g] = __uint_as_float(unord_hi(__float_as_uint(best[g])));
    }
    // The tagged maxima are exact except where a lane's maximum is not
    // positive in the raw mode, or is a NaN: one with the sign clear lies
    // above +inf in either mode (the compare-and-select epilogue never takes
    // a NaN); one with the sign set is negative in the raw mode and lies
    // below -inf in the order-preserving one, so it can only be a lane's
    // maximum where every other value is also such a NaN.  If any live lane's
    // maximum is one of these, the whole workgroup covers its range once
    // more with the exact epilogue: the copies of tiles 0 .. AHEAD - 1 go out
    // again in the loop's order (x is still in registers) and every wave
    // passes the same barriers.  Every copy of the first run has landed and
    // been read before its last barrier.
    if constexpr (kTagged) {
        bool redo = false;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const uint32_t mag = __float_as_uint(best[g]) & 0x7FFFFFFFu;
            const bool bad = ord_mode ? (mag > 0x7F800000u)
                                      : (__float_as_int(best[g]) <= 0 ||
                                         __float_as_int(best[g]) > 0x7F800000);
            redo |= row_ok[g] && bidx[g] != kNoIndex && bad;
        }
        if (__syncthreads_or(redo)) {
            reset_best();
            asm volatile("" : "+s"(t0c));
            issue_w(-AHEAD);
            issue_base(-AHEAD);
            int later2 = 0;
            for (int j = 1 - AHEAD; j < 0; ++j) {
                issue(j);
                later2 += n_copies(j);
            }
            wait_vmcnt_dyn<kMaxCount>(later2);
            __syncthreads();
            // recomputed rather than held across the range
            uint32_t w0 = wrow0;
            asm volatile("" : "+s"(w0));
            if (w0 + 32u < a.rows) {
                run_from(0, std::integral_constant<int, 2>{}, std::integral_constant<int, kExact>{});
            } else {
                run_from(0, std::integral_constant<int, 1>{}, std::integral_constant<int, kExact>{});
            }
        }
    }

#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
        // lanes l and l + 32 hold two halves of the same row's ids
        float bv = best[g];
        uint32_t bi = bidx[g] == kNoIndex ? kNoIndex : bidx[g] + first_id;
        const float ov = __shfl_xor(bv, 32);
        const uint32_t oi = __shfl_xor(bi, 32);
        merge(bv, bi, ov, oi);
        if (khalf == 0u && row_ok[g]) {
            a.table[(uint64_t)row[g] * a.ranges + range] = make_key(bv, bi);
        }
    }
}

template <int R>
hipError_t launch_gemm(const GemmArgs& a, int waves, uint32_t grid, hipStream_t stream)
{
    // one wave: a ring of four (60 to 80 KiB at R = 256, two workgroups per
    // CU) so copies run three tiles ahead of a wave that computes a tile in a
    // fraction of the memory latency; otherwise three
    switch (waves) {
        case 1: hipLaunchKernelGGL((gemm_readout_kernel<R, 1, 4>), dim3(grid), dim3(64), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((gemm_readout_kernel<R, 2, 3>), dim3(grid), dim3(128), 0, stream, a); break;
        default:
            hipLaunchKernelGGL((gemm_readout_kernel<R, kWavesMax, 3>), dim3(grid), dim3(kWavesMax * 64),
                               0, stream, a);
            break;
    }
    return hipGetLastError();
}

// Launch shape for `rows` draft rows over V ids.  Up to 64 rows: one wave
// per workgroup, up to 128: two (two workgroups per CU either way, LDS
// allowing); beyond: eight waves (512 rows), one workgroup per CU, and as
// many workgroups per range as the rows need.  The vocabulary is cut into a
// multiple of 8 ranges (one per XCD slot) of whole 32-id tiles.  Returns
// false when the grid would not fit 31 bits.
struct GemmPlan {
    int waves;
    uint32_t tiles;
    uint32_t row_wgs;
    uint32_t ranges;
};

bool gemm_plan(int64_t rows, int64_t V, GemmPlan* p)
{
    p->tiles = (uint32_t)((V + kTileV - 1) / kTileV);
    p->waves = rows <= 64 ? 1 : rows <= 128 ? 2 : kWavesMax;
    const int per_cu = p->waves == kWavesMax ? 1 : 2;
    const int64_t rows_per_wg = (int64_t)p->waves * 32 * kGroups;
    const int64_t row_wgs = (rows + rows_per_wg - 1) / rows_per_wg;
    int64_t ranges = (int64_t)device_cus() * per_cu / row_wgs;
    ranges = ranges / 8 * 8;
    if (ranges < 8) ranges = 8;
    const int64_t max_ranges = ((int64_t)p->tiles + 7) / 8 * 8;
    if (ranges > max_ranges) ranges = max_ranges;
    if (row_wgs * ranges > 0x7FFFFFFFll) return false;
    p->row_wgs = (uint32_t)row_wgs;
    p->ranges = (uint32_t)ranges;
    return true;
}

}  // namespace

extern "C" int xpress_describe_gemm_plan(int64_t N, int64_t B, int64_t V, int* waves,
                                         int* ranges, int* row_wgs, int* tiles)
{
    if (N < 0 || B < 1 || V < 1 || V > 0x7FFFFFFFll) return XPRESS_EINVAL;
    if (B - 1 > 0 && N > 0x7FFFFFFFll / (B - 1)) return XPRESS_EINVAL;
    const int64_t rows = N * (B - 1);
    GemmPlan p;
    if (!gemm_plan(rows > 0 ? rows : 1, V, &p)) return XPRESS_EINVAL;
    if (waves) *waves = p.waves;
    if (ranges) *ranges = (int)p.ranges;
    if (row_wgs) *row_wgs = (int)p.row_wgs;
    if (tiles) *tiles = (int)p.tiles;
    return XPRESS_OK;
}

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

    GemmPlan p;
    if (!gemm_plan(rows, V, &p)) return XPRESS_EINVAL;
    GemmArgs a;
    a.base = base;
    a.x = x;
    a.w = w;
    a.stride_base = stride_base_r;
    a.rows = (uint32_t)rows;
    a.V = (uint32_t)V;
    a.tiles = p.tiles;
    a.row_wgs = p.row_wgs;
    a.ranges = p.ranges;
    a.reverse = reverse_order() ? 1u : 0u;

    int rc = workspace_table(stream, rows * (int64_t)p.ranges, &a.table);
    if (rc != XPRESS_OK) return rc;

    const uint32_t grid = a.row_wgs * a.ranges;
    hipError_t e;
    switch (R) {
        case 64: e = launch_gemm<64>(a, p.waves, grid, stream); break;
        case 128: e = launch_gemm<128>(a, p.waves, grid, stream); break;
        default: e = launch_gemm<256>(a, p.waves, grid, stream); break;
    }
    if (e != hipSuccess) return hip_fail(e);
    e = launch_reduce_table(a.table, blk, nullptr, a.rows, (uint32_t)(B - 1), a.V, a.ranges,
                            stream);
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}
