// xpress_argmax.hip -- fused add + argmax readout for MI355X (gfx950).
//
// The operation is the readout stage of one XPress Jacobi pass (XPress
// kernels page, "fused_add_argmax_to_blk" and its two stage kernels): for
// every draft row r = n*(B-1) + b,
//     blk[n, 1 + b] = lowest v maximising bf16(base[r, v] + bias[r, v]),
// with the [rows, V] sum never stored and slot 0 of each block untouched.
//
// Design (gfx950, wave64).  The work is a pure stream over 4 bytes per
// element with ~8 VALU operations per element, so it is HBM-bound and has no
// contraction in it -- no MFMA.  What matters is keeping enough 16-byte loads
// in flight on every CU:
//   * a row is split into `splits` contiguous vector ranges, one workgroup
//     each; every lane streams 16-byte (8 x bf16) non-temporal loads of base
//     and bias, UNROLL vectors of each in flight before any arithmetic;
//   * element step: widen both bf16 to fp32 (a shift or a mask), one fp32
//     add, one v_cvt_pk_bf16_f32 per pair (round-to-nearest-even, fp32
//     denormals kept by the default kernel mode), widen back;
//   * the lane keeps a running (max, vector id) per position 0..7 of the
//     16-byte vector, replaced only on a strictly larger value -- vectors are
//     visited in ascending order, so each position keeps its first maximum;
//   * the 8 positions, then the 64 lanes (DPP quad_perm / row mirrors,
//     ds_swizzle across 16, readlane across 32), then the waves (LDS) are
//     merged in (value desc, index asc) order, which is the total order whose
//     maximum is the first maximum;
//   * the workgroups of a row meet in one of three ways (see
//     xpress_set_plan in the header): a single workgroup per row; one
//     64-bit word per row holding the best packed key and an arrival count,
//     updated by agent-scope compare-and-swap, whose last arriver writes blk
//     and clears the word; or a key table plus a second small kernel.  The
//     balanced plan cuts the flattened rows into equal ranges and folds the
//     rows it splits through the same compare-and-swap word.
// The pages' own design (a [rows, chunks] fp32 + int64 scratch and a second
// kernel per row) is the two-pass variant here, with one u64 key per chunk.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "xpress_argmax.h"
#include "device_common.h"
#include "host_common.h"

namespace {

using namespace xpress;

// ---------------------------------------------------------------------------
// Streaming parts.
// ---------------------------------------------------------------------------

// Vector path: vectors [q0, q1) of one row (a vector = 8 consecutive bf16 at
// a 16-byte aligned address), strided over the T threads.  Returns the
// thread's (value, index) candidate.
template <int T, int UNROLL>
__device__ __forceinline__ void scan_vectors(const u32x4* __restrict__ pa,
                                             const u32x4* __restrict__ pb,
                                             uint32_t q0, uint32_t q1,
                                             float& out_v, uint32_t& out_i)
{
    float best[8];
    uint32_t bq[8];
    const uint32_t qfirst = q0 + threadIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        best[j] = -__builtin_inff();
        bq[j] = qfirst;
    }

    auto consume = [&](const u32x4& va, const u32x4& vb, uint32_t q) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t p = add_round2(va[w], vb[w]);
            float s0 = bf16_lo(p);
            float s1 = bf16_hi(p);
            bool t0 = s0 > best[2 * w];
            best[2 * w] = t0 ? s0 : best[2 * w];
            bq[2 * w] = t0 ? q : bq[2 * w];
            bool t1 = s1 > best[2 * w + 1];
            best[2 * w + 1] = t1 ? s1 : best[2 * w + 1];
            bq[2 * w + 1] = t1 ? q : bq[2 * w + 1];
        }
    };

    uint32_t q = qfirst;
    for (; q + (UNROLL - 1) * T < q1; q += UNROLL * T) {
        u32x4 va[UNROLL], vb[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            va[u] = __builtin_nontemporal_load(pa + q + u * T);
            vb[u] = __builtin_nontemporal_load(pb + q + u * T);
        }
        // keep every load of the batch ahead of the first use of any of them
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            consume(va[u], vb[u], q + u * T);
        }
    }
    for (; q < q1; q += T) {
        u32x4 va = __builtin_nontemporal_load(pa + q);
        u32x4 vb = __builtin_nontemporal_load(pb + q);
        consume(va, vb, q);
    }

    float v = -__builtin_inff();
    uint32_t i = kNoIndex;
    if (qfirst < q1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            merge(v, i, best[j], bq[j] * 8u + (uint32_t)j);
        }
    }
    out_v = v;
    out_i = i;
}

// Scalar path: elements [e0, e1) of one row, strided over the T threads.
template <int T>
__device__ __forceinline__ void scan_scalars(const uint16_t* __restrict__ a,
                                             const uint16_t* __restrict__ b,
                                             uint32_t e0, uint32_t e1,
                                             float& out_v, uint32_t& out_i)
{
    float best = -__builtin_inff();
    uint32_t bi = kNoIndex;
    uint32_t e = e0 + threadIdx.x;
    if (e < e1) {
        bi = e;
    }
    for (; e < e1; e += T) {
        float s = add_round1(a[e], b[e]);
        bool t = s > best;
        best = t ? s : best;
        bi = t ? e : bi;
    }
    out_v = best;
    out_i = bi;
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

struct RowArgs {
    const uint16_t* base;
    const uint16_t* bias;
    int64_t* blk;
    int64_t stride_base;  // elements
    int64_t stride_bias;  // elements
    uint32_t rows;
    uint32_t bm1;         // B - 1
    uint32_t V;
    uint32_t splits;      // workgroups per row
    uint64_t* keys;       // ATOMIC: [rows] key-and-count words;
                          // TWO_PASS: [rows, splits] key table
    const int64_t* cand;  // top-C readout: [rows, V] candidate ids, else null
    uint32_t reverse;     // nonzero: units (ranges) visited last to first
};

enum Combine { kSingle = XPRESS_COMBINE_SINGLE, kAtomic = XPRESS_COMBINE_ATOMIC,
               kTwoPass = XPRESS_COMBINE_TWO_PASS, kBalanced = XPRESS_COMBINE_BALANCED };

// Row r = n*(B-1) + b writes slot 1 + b of block n.  The full-vocabulary
// readout writes the winning position (a vocabulary id); the top-C readout
// writes the winning candidate's id, cand[r, position].
__device__ __forceinline__ void write_blk(const RowArgs& a, uint32_t row, int64_t idx)
{
    const uint32_t n = row / a.bm1;
    const uint32_t b = row - n * a.bm1;
    const int64_t tok = a.cand ? a.cand[(int64_t)row * a.V + idx] : idx;
    a.blk[(int64_t)n * (a.bm1 + 1) + 1 + b] = tok;
}

// Fold one workgroup's candidate key into its row's 64-bit word, which holds
// (best key so far) << 16 | the number of workgroups that have folded in.
// Every access to the word is an atomic operation on that one location, so
// the updates are totally ordered and each compare-and-swap sees every
// earlier one: the workgroup that finds the count at arrivals - 1 holds the
// row's final key in its own new value.  It writes blk and clears the word
// for the next call.  No fence is needed: nothing else is published between
// workgroups.  arrivals <= 65535.
__device__ __forceinline__ void fold_key(const RowArgs& a, uint32_t row, uint64_t key,
                                         uint32_t arrivals)
{
    uint64_t* word = &a.keys[row];
    uint64_t old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t desired;
    do {
        const uint64_t best = old >> 16;
        desired = ((key > best ? key : best) << 16) | ((old + 1u) & 0xFFFFu);
    } while (!__hip_atomic_compare_exchange_weak(word, &old, desired, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if ((old & 0xFFFFu) == arrivals - 1u) {
        __hip_atomic_store(word, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        write_blk(a, row, key_index(desired >> 16));
    }
}

// One workgroup per (row, split) unit; the grid strides over units so any
// number of rows fits in one launch.
template <int T, int UNROLL, bool VEC, int COMBINE>
__global__ __launch_bounds__(T) void readout_kernel(RowArgs a)
{
    const uint32_t units = a.rows * a.splits;
    for (uint32_t k = blockIdx.x; k < units; k += gridDim.x) {
        const uint32_t unit = a.reverse ? units - 1u - k : k;
        const uint32_t row = unit / a.splits;
        const uint32_t split = unit - row * a.splits;
        const uint16_t* rb = a.base + (int64_t)row * a.stride_base;
        const uint16_t* ri = a.bias + (int64_t)row * a.stride_bias;

        float v;
        uint32_t i;
        if constexpr (VEC) {
            const uint32_t nvec = a.V / 8u;
            const uint32_t q0 = (uint32_t)(((uint64_t)split * nvec) / a.splits);
            const uint32_t q1 = (uint32_t)(((uint64_t)(split + 1) * nvec) / a.splits);
            scan_vectors<T, UNROLL>(reinterpret_cast<const u32x4*>(rb),
                                    reinterpret_cast<const u32x4*>(ri), q0, q1, v, i);
            // the last V % 8 elements belong to the row's last split
            const uint32_t tail0 = nvec * 8u;
            if (split == a.splits - 1 && tail0 + threadIdx.x < a.V) {
                const uint32_t e = tail0 + threadIdx.x;
                merge(v, i, add_round1(rb[e], ri[e]), e);
            }
        } else {
            const uint32_t e0 = (uint32_t)(((uint64_t)split * a.V) / a.splits);
            const uint32_t e1 = (uint32_t)(((uint64_t)(split + 1) * a.V) / a.splits);
            scan_scalars<T>(rb, ri, e0, e1, v, i);
        }

        block_argmax<T>(v, i);

        if (threadIdx.x == 0) {
            if constexpr (COMBINE == kSingle) {
                write_blk(a, row, (int64_t)i);
            } else if constexpr (COMBINE == kTwoPass) {
                a.keys[(uint64_t)row * a.splits + split] = make_key(v, i);
            } else {
                fold_key(a, row, make_key(v, i), a.splits);
            }
        }
    }
}

// Balanced plan: the full 16-byte vectors of all rows, in row-major order,
// are cut into gridDim.x equal contiguous ranges, one per workgroup, with the
// grid sized to a whole number of workgroups per CU.  Every CU then streams
// the same number of bytes, so none idles while others finish (one workgroup
// per row leaves the CUs that received fewer rows idle at the end).  A
// workgroup meets each row its range touches; a row wholly inside one range
// is written directly, a row shared by several ranges is folded through its
// key-and-count word, expecting as many arrivals as ranges touch it.
// Requires V >= 8, 16-byte aligned rows, and at least one vector per range.
__device__ __forceinline__ uint32_t range_of(uint64_t x, uint64_t q, uint64_t g)
{
    // the range [floor(k*q/g), floor((k+1)*q/g)) that holds vector x
    return (uint32_t)(((x + 1u) * g - 1u) / q);
}

template <int T, int UNROLL>
__global__ __launch_bounds__(T) void readout_balanced_kernel(RowArgs a)
{
    const uint64_t nvec = a.V / 8u;
    const uint64_t q = (uint64_t)a.rows * nvec;
    const uint64_t g = gridDim.x;
    const uint64_t bid = a.reverse ? g - 1u - blockIdx.x : blockIdx.x;
    const uint64_t x1 = (bid + 1u) * q / g;
    uint64_t x = bid * q / g;
    while (x < x1) {
        const uint32_t row = (uint32_t)(x / nvec);
        const uint64_t row0 = (uint64_t)row * nvec;
        const uint64_t seg_end = (x1 < row0 + nvec) ? x1 : row0 + nvec;
        const uint32_t q0 = (uint32_t)(x - row0);
        const uint32_t q1 = (uint32_t)(seg_end - row0);
        const uint16_t* rb = a.base + (int64_t)row * a.stride_base;
        const uint16_t* ri = a.bias + (int64_t)row * a.stride_bias;

        float v;
        uint32_t i;
        scan_vectors<T, UNROLL>(reinterpret_cast<const u32x4*>(rb),
                                reinterpret_cast<const u32x4*>(ri), q0, q1, v, i);
        // the last V % 8 elements go with the row's last vector
        const uint32_t tail0 = (uint32_t)nvec * 8u;
        if (q1 == (uint32_t)nvec && tail0 + threadIdx.x < a.V) {
            const uint32_t e = tail0 + threadIdx.x;
            merge(v, i, add_round1(rb[e], ri[e]), e);
        }

        block_argmax<T>(v, i);

        if (threadIdx.x == 0) {
            const uint32_t first = range_of(row0, q, g);
            const uint32_t last = range_of(row0 + nvec - 1u, q, g);
            if (first == last) {
                write_blk(a, row, (int64_t)i);
            } else {
                fold_key(a, row, make_key(v, i), last - first + 1u);
            }
        }
        x = seg_end;
    }
}

// Top-C readout for candidate lists that fit one wave's reach: one wave per
// row, four rows per 256-thread workgroup.  Each lane keeps its best
// candidate's (value, position, id); the ids are streamed with the logits,
// so after the wave's (value, position) reduction the lane that holds the
// winning position writes its id -- no second, dependent memory round trip
// for the gather.  A lane replaces its incumbent only on a strictly larger
// value (or, when it has none yet, on any value but NaN), visiting its
// positions in ascending order, so it keeps its first maximum and never
// holds a NaN.  A row whose sums are all NaN (no lane holds a candidate)
// writes its first candidate's id, as a row of -inf sums does.
template <bool VEC>
__global__ __launch_bounds__(256) void topc_wave_kernel(const uint16_t* __restrict__ base_c,
                                                        const uint16_t* __restrict__ bias_c,
                                                        const int64_t* __restrict__ cand,
                                                        int64_t* __restrict__ blk,
                                                        uint32_t rows, uint32_t bm1,
                                                        uint32_t C)
{
    const uint32_t lane = threadIdx.x & 63u;
    for (uint32_t row = blockIdx.x * 4u + threadIdx.x / 64u; row < rows;
         row += gridDim.x * 4u) {
        const uint16_t* a = base_c + (uint64_t)row * C;
        const uint16_t* b = bias_c + (uint64_t)row * C;
        const int64_t* cd = cand + (uint64_t)row * C;
        float best = -__builtin_inff();
        uint32_t bi = kNoIndex;
        int64_t bid = 0;
        auto take = [&](float sv, uint32_t c, int64_t id) {
            const bool t = (sv > best) | ((bi == kNoIndex) & (sv == sv));
            best = t ? sv : best;
            bi = t ? c : bi;
            bid = t ? id : bid;
        };
        uint32_t tail0 = 0;
        if constexpr (VEC) {
            const uint32_t nvec = C / 8u;
            const u32x4* pa = reinterpret_cast<const u32x4*>(a);
            const u32x4* pb = reinterpret_cast<const u32x4*>(b);
            const u32x4* pc = reinterpret_cast<const u32x4*>(cd);
            for (uint32_t q = lane; q < nvec; q += 64u) {
                const u32x4 va = __builtin_nontemporal_load(pa + q);
                const u32x4 vb = __builtin_nontemporal_load(pb + q);
                u32x4 ids[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) ids[k] = __builtin_nontemporal_load(pc + 4 * q + k);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t pr = add_round2(va[w], vb[w]);
                    const int64_t id0 = (int64_t)(((uint64_t)ids[w][1] << 32) | ids[w][0]);
                    const int64_t id1 = (int64_t)(((uint64_t)ids[w][3] << 32) | ids[w][2]);
                    take(bf16_lo(pr), q * 8u + 2u * w, id0);
                    take(bf16_hi(pr), q * 8u + 2u * w + 1u, id1);
                }
            }
            tail0 = nvec * 8u;
        }
        for (uint32_t c = tail0 + lane; c < C; c += 64u) {
            take(add_round1(a[c], b[c]), c, cd[c]);
        }
        float v = best;
        uint32_t i = bi;
        wave_argmax(v, i);
        const uint32_t n = row / bm1;
        int64_t* slot = blk + (int64_t)n * (bm1 + 1) + 1 + (row - n * bm1);
        if (i == kNoIndex) {
            if (lane == 0u) *slot = cd[0];
        } else if (bi == i) {
            *slot = bid;
        }
    }
}

// Keys a lane of the second pass loads before comparing any.
constexpr int kReduceBatch = 8;

// Second pass of the two-pass combine: one wave per row reads the row's
// `splits` keys with consecutive lanes on consecutive keys, keeps the largest
// (a larger key is a larger value or, on equal values, a smaller index),
// reduces over the wave and writes blk from lane 0.  Loads are unconditional
// (clamped to the row's last key) and masked afterwards, so that a batch of
// them is in flight together: a predicated load would be waited on alone.
__global__ __launch_bounds__(256) void reduce_keys_kernel(RowArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t last = a.splits - 1u;
    for (uint32_t row = blockIdx.x * 4u + (threadIdx.x >> 6); row < a.rows;
         row += gridDim.x * 4u) {
        const uint64_t* k = a.keys + (uint64_t)row * a.splits;
        unsigned long long best = 0;
        if (a.splits <= 64u) {
            // at most one key per lane
            const unsigned long long v = k[lane < a.splits ? lane : last];
            best = lane < a.splits ? v : 0ull;
        } else {
            // batches of up to 64 * kReduceBatch keys: one memory latency per
            // batch rather than one per 64 keys
            for (uint32_t s0 = 0; s0 < a.splits; s0 += 64u * kReduceBatch) {
                unsigned long long v[kReduceBatch];
#pragma unroll
                for (int u = 0; u < kReduceBatch; ++u) {
                    const uint32_t s = s0 + 64u * u + lane;
                    v[u] = k[s < a.splits ? s : last];
                }
#pragma unroll
                for (int u = 0; u < kReduceBatch; ++u) {
                    const bool in = s0 + 64u * u + lane < a.splits;
                    best = in && v[u] > best ? v[u] : best;
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const unsigned long long o = __shfl_xor(best, off);
            best = o > best ? o : best;
        }
        if (lane == 0u) write_blk(a, row, key_index(best));
    }
}

// The element step over a table of pairs: out[i*65536 + b] = bf16(a_i + b).
__global__ __launch_bounds__(256) void round_table_kernel(const uint16_t* __restrict__ a_vals,
                                                          uint32_t n_a,
                                                          uint32_t* __restrict__ out)
{
    // each thread makes one packed pair (b, b + 1) for one a
    const uint64_t total = (uint64_t)n_a * 32768u;
    for (uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x; t < total;
         t += (uint64_t)gridDim.x * 256u) {
        const uint32_t ia = (uint32_t)(t >> 15);
        const uint32_t b0 = (uint32_t)(t & 32767u) * 2u;
        const uint32_t av = a_vals[ia];
        out[t] = add_round2(av | (av << 16), b0 | ((b0 + 1u) << 16));
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------


struct Plan {
    int combine;
    int splits;   // workgroups per row; for kBalanced, workgroups per CU
    int threads;
    bool vec;
    int launches;
    uint32_t grid;  // kBalanced: total workgroups
    bool reverse;   // units visited last to first (debug)
};

std::mutex g_plan_mu;
std::atomic<int> g_reverse_order{0};
int g_override_combine = XPRESS_COMBINE_AUTO;
int g_override_splits = 0;
int g_override_threads = 0;

// Vectors of each stream in flight per thread before the first use.  Measured
// at 480 x 152064 on MI355X: 2 and 3 within noise of each other, 1 and 4-8
// slower at 1024 threads.
constexpr int kUnroll = 2;

// Below this many rows the default plan splits rows over workgroups, aiming
// at about kSplitTargetUnits workgroups in all.
constexpr int64_t kSplitBelowRows = 128;
constexpr int64_t kSplitTargetUnits = 512;

// Workgroups per CU of the balanced plan.
constexpr int64_t kBalancedPerCu = 2;

// Largest candidate count the top-C readout handles with one wave per row;
// larger lists take the streaming readout.  Measured on MI355X, 480 rows,
// per step inside a HIP graph: one wave per row 2.3 / 2.2 / 2.8 / 3.2 /
// 4.4 us at C = 64 / 128 / 256 / 512 / 1024, the streaming readout 2.8 /
// 2.8 / 3.1 / 3.1 / 3.3 us.
constexpr int64_t kTopcWaveMaxC = 256;


// Workgroup size of the default plan.  Measured on MI355X with one
// workgroup per row (interleaved medians): at 480 rows x 152064, 256 threads
// 44.8 us vs 45.5 us for 512 or 1024; at 3840 rows, 1024 threads ~2% ahead
// of 256; below 128 rows (split plans) 1024.  Capped so that every thread
// still gets at least two unrolled rounds of loads in a row of V elements.
int auto_threads(int64_t rows, int64_t V, bool vec)
{
    const int64_t units = vec ? V / 8 : V;
    int t = (rows >= kSplitBelowRows && rows < 1024) ? 256 : 1024;
    while (t > 64 && units < (int64_t)t * kUnroll * 2) t /= 2;
    return t;
}

Plan make_plan(const uint16_t* base, const uint16_t* bias, int64_t rows, int64_t V,
               int64_t sb, int64_t sbi)
{
    Plan p;
    p.vec = is_aligned16(base) && is_aligned16(bias) && (sb % 8 == 0) && (sbi % 8 == 0);
    int oc, os, ot;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        oc = g_override_combine;
        os = g_override_splits;
        ot = g_override_threads;
    }
    p.threads = ot ? ot : auto_threads(rows, V, p.vec);
    // Measured on MI355X: one workgroup per row streams within ~3% of a
    // plain read kernel once there are a few hundred rows, and stays the
    // fastest down to tens of rows (the second launch of the two-pass
    // combine costs ~2 us; the compare-and-swap folds of the atomic combine
    // queue up on each row's word: 47.8 us with 2 splits and 70.4 us with 8
    // at 480 x 152064, against 44.8 us unsplit).  Only a handful of very wide
    // rows leave most CUs idle; those are split and combined in two passes.
    const int64_t per_split = (int64_t)p.threads * kUnroll * 2 * (p.vec ? 8 : 1);
    int64_t max_splits = V / per_split;
    if (max_splits < 1) max_splits = 1;
    int64_t s = 1;
    int combine = kSingle;
    if (rows < kSplitBelowRows && max_splits > 1) {
        s = (kSplitTargetUnits + rows - 1) / rows;
        if (s > max_splits) s = max_splits;
        if (s > 1) combine = kTwoPass;
        else s = 1;
    }
    if (oc != XPRESS_COMBINE_AUTO) {
        combine = oc;
        if (os > 0) s = os;
        else if (combine != kSingle && s == 1) s = max_splits < 8 ? max_splits : 8;
    } else if (os > 0) {
        s = os;
        if (s > 1 && combine == kSingle) combine = kTwoPass;
    }
    if (s > 65535) s = 65535;
    // (row, split) units are counted in 32 bits on the device
    if (s > 1 && rows * s > 0x7FFFFFFFll) s = 0x7FFFFFFFll / rows;
    if (s < 1) s = 1;
    if (combine == kSingle) s = 1;
    p.grid = 0;
    if (combine == kBalanced) {
        // s = workgroups per CU; every range must hold at least one vector,
        // and the range arithmetic stays in 64 bits
        const int64_t per_cu = (os > 0) ? os : kBalancedPerCu;
        const int64_t g = (int64_t)device_cus() * (per_cu < 1 ? 1 : (per_cu > 64 ? 64 : per_cu));
        const int64_t q = rows * (V / 8);
        // (x + 1) * g must not overflow 64 bits for x < q
        if (!p.vec || V < 8 || q < g || q > ((int64_t)1 << 62) / g) {
            combine = kSingle;
            s = 1;
        } else {
            s = g / device_cus();
            p.grid = (uint32_t)g;
        }
    }
    p.combine = combine;
    p.splits = (int)s;
    p.launches = (p.combine == kTwoPass) ? 2 : 1;
    p.reverse = reverse_order();
    return p;
}

// Per (device, stream) workspace.  The atomic region ([rows] u64
// key-and-count words) is zero when idle: allocated zeroed, and every call's
// last arriver clears the word it used.  The table region is overwritten
// whole by every two-pass call.  A region that has to grow is replaced by a
// larger one (at least twice the old size, so the sizes form a geometric
// series) and the old one is retired, not freed: work already queued, and
// HIP graphs captured earlier, may still use it.  Retired regions are freed
// by xpress_release, and their total stays below the live region's size.
struct Workspace {
    uint64_t* keys = nullptr;
    int64_t rows_cap = 0;
    uint64_t* table = nullptr;
    int64_t table_cap = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::map<int, std::vector<void*>> g_retired;   // per device
std::map<int, int64_t> g_ws_bytes;             // live + retired bytes per device
int64_t g_ws_limit = 0;                        // bytes per device; 0 = no limit

int stream_capturing(hipStream_t stream, bool* capturing)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &st);
    if (e != hipSuccess) return hip_fail(e);
    *capturing = (st != hipStreamCaptureStatusNone);
    return XPRESS_OK;
}

int64_t grown_cap(int64_t need, int64_t old_cap, int64_t floor_cap)
{
    int64_t cap = need > floor_cap ? need : floor_cap;
    if (old_cap > 0 && cap < 2 * old_cap) cap = 2 * old_cap;
    return cap;
}

// Make sure the (device, stream) workspace holds `rows` atomic slots and a
// `table` entry table; grows (synchronously) when needed.  Called with
// g_ws_mu held.
int ensure_workspace_locked(int dev, hipStream_t stream, int64_t rows, int64_t table,
                            Workspace** out)
{
    Workspace& w = g_ws[std::make_pair(dev, stream)];
    const bool grow_rows = rows > w.rows_cap;
    const bool grow_table = table > w.table_cap;
    if (grow_rows || grow_table) {
        bool capturing = false;
        int rc = stream_capturing(stream, &capturing);
        if (rc != XPRESS_OK) return rc;
        if (capturing) return XPRESS_ECAPTURE;
    }
    hipError_t e;
    if (grow_rows) {
        const int64_t cap = grown_cap(rows, w.rows_cap, 4096);
        if (g_ws_limit > 0 && g_ws_bytes[dev] + cap * 8 > g_ws_limit) return XPRESS_ENOMEM;
        void* p = nullptr;
        e = hipMalloc(&p, (size_t)cap * 8u);
        if (e != hipSuccess) {
            note_hip_error(e);
            return XPRESS_ENOMEM;
        }
        // zeroed before any kernel can see it (synchronous)
        e = hipMemset(p, 0, (size_t)cap * 8u);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            (void)hipFree(p);
            return hip_fail(e);
        }
        if (w.keys) g_retired[dev].push_back(w.keys);
        w.keys = static_cast<uint64_t*>(p);
        w.rows_cap = cap;
        g_ws_bytes[dev] += cap * 8;
    }
    if (grow_table) {
        const int64_t cap = grown_cap(table, w.table_cap, 65536);
        if (g_ws_limit > 0 && g_ws_bytes[dev] + cap * 8 > g_ws_limit) return XPRESS_ENOMEM;
        void* p = nullptr;
        e = hipMalloc(&p, (size_t)cap * 8u);
        if (e != hipSuccess) {
            note_hip_error(e);
            return XPRESS_ENOMEM;
        }
        if (w.table) g_retired[dev].push_back(w.table);
        w.table = static_cast<uint64_t*>(p);
        w.table_cap = cap;
        g_ws_bytes[dev] += cap * 8;
    }
    *out = &w;
    return XPRESS_OK;
}

int ensure_workspace(hipStream_t stream, int64_t rows, int64_t table, Workspace** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    return ensure_workspace_locked(dev, stream, rows, table, out);
}

template <int T, bool VEC, int COMBINE>
hipError_t launch_readout(const RowArgs& a, hipStream_t stream)
{
    const uint64_t units = (uint64_t)a.rows * a.splits;
    const uint32_t grid = (uint32_t)(units < (1u << 22) ? units : (1u << 22));
    hipLaunchKernelGGL((readout_kernel<T, kUnroll, VEC, COMBINE>), dim3(grid), dim3(T), 0,
                       stream, a);
    return hipGetLastError();
}

template <int T, bool VEC>
hipError_t launch_by_combine(const RowArgs& a, int combine, hipStream_t stream)
{
    switch (combine) {
        case kSingle: return launch_readout<T, VEC, kSingle>(a, stream);
        case kAtomic: return launch_readout<T, VEC, kAtomic>(a, stream);
        default: return launch_readout<T, VEC, kTwoPass>(a, stream);
    }
}

template <int T>
hipError_t launch_by_vec(const RowArgs& a, const Plan& p, hipStream_t stream)
{
    return p.vec ? launch_by_combine<T, true>(a, p.combine, stream)
                 : launch_by_combine<T, false>(a, p.combine, stream);
}

template <int T>
hipError_t launch_balanced(const RowArgs& a, const Plan& p, hipStream_t stream)
{
    hipLaunchKernelGGL((readout_balanced_kernel<T, kUnroll>), dim3(p.grid), dim3(T), 0, stream,
                       a);
    return hipGetLastError();
}

hipError_t launch_plan(const RowArgs& a, const Plan& p, hipStream_t stream)
{
    if (p.combine == kBalanced) {
        switch (p.threads) {
            case 64: return launch_balanced<64>(a, p, stream);
            case 128: return launch_balanced<128>(a, p, stream);
            case 512: return launch_balanced<512>(a, p, stream);
            case 1024: return launch_balanced<1024>(a, p, stream);
            default: return launch_balanced<256>(a, p, stream);
        }
    }
    switch (p.threads) {
        case 64: return launch_by_vec<64>(a, p, stream);
        case 128: return launch_by_vec<128>(a, p, stream);
        case 512: return launch_by_vec<512>(a, p, stream);
        case 1024: return launch_by_vec<1024>(a, p, stream);
        default: return launch_by_vec<256>(a, p, stream);
    }
}


int validate(const uint16_t* base, const uint16_t* bias, const int64_t* blk, int64_t N,
             int64_t B, int64_t V, int64_t sb, int64_t sbi, const int64_t* cand,
             int64_t* rows_out)
{
    if (N < 0 || B < 1 || V < 1 || V > 0x7FFFFFFFll || sb < V || sbi < V) {
        return XPRESS_EINVAL;
    }
    if (B - 1 > 0 && N > INT64_MAX / (B - 1)) return XPRESS_EINVAL;
    const int64_t rows = N * (B - 1);
    *rows_out = rows;
    if (rows == 0) return XPRESS_OK;
    if (rows > 0x7FFFFFFFll || N > INT64_MAX / B) return XPRESS_EINVAL;
    if (!base || !bias || !blk) return XPRESS_EINVAL;
    if ((rows - 1) > (INT64_MAX / 8 - V) / sb || (rows - 1) > (INT64_MAX / 8 - V) / sbi) {
        return XPRESS_EINVAL;
    }
    const size_t base_bytes = (size_t)((rows - 1) * sb + V) * 2u;
    const size_t bias_bytes = (size_t)((rows - 1) * sbi + V) * 2u;
    const size_t blk_bytes = (size_t)(N * B) * 8u;
    if (ranges_overlap(blk, blk_bytes, base, base_bytes) ||
        ranges_overlap(blk, blk_bytes, bias, bias_bytes)) {
        return XPRESS_EINVAL;
    }
    if (cand != nullptr) {
        // candidate ids are [rows, V] contiguous, like the logits
        const size_t cand_bytes = (size_t)(rows * V) * 8u;
        if (ranges_overlap(blk, blk_bytes, cand, cand_bytes)) return XPRESS_EINVAL;
    }
    return XPRESS_OK;
}

RowArgs row_args(const uint16_t* base, const uint16_t* bias, const int64_t* cand, int64_t* blk,
                 int64_t rows, int64_t B, int64_t V, int64_t sb, int64_t sbi, const Plan& p)
{
    RowArgs a;
    a.base = base;
    a.bias = bias;
    a.blk = blk;
    a.stride_base = sb;
    a.stride_bias = sbi;
    a.rows = (uint32_t)rows;
    a.bm1 = (uint32_t)(B - 1);
    a.V = (uint32_t)V;
    a.splits = (uint32_t)p.splits;
    a.keys = nullptr;
    a.cand = cand;
    a.reverse = p.reverse ? 1u : 0u;
    return a;
}

// The plan's launches, with a.keys already pointing at its scratch.
int launch_readout_plan(const RowArgs& a, const Plan& p, hipStream_t stream)
{
    hipError_t e = launch_plan(a, p, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (p.combine == kTwoPass) {
        e = launch_reduce_table(a.keys, a.blk, a.cand, a.rows, a.bm1, a.V, a.splits, stream);
        if (e != hipSuccess) return hip_fail(e);
    }
    return XPRESS_OK;
}

// The no-allocation variant's key table: a fixed device array, one copy per
// GPU, shared by every call on that GPU.  Its address on each device is
// looked up once, with that device current.
constexpr int64_t kScratchKeys = 4096;
static __device__ __align__(256) uint64_t scratch[kScratchKeys];

std::mutex g_scratch_mu;
std::map<int, uint64_t*> g_scratch_ptr;

int scratch_table(uint64_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        it = g_scratch_ptr.emplace(dev, static_cast<uint64_t*>(ptr)).first;
    }
    *out = it->second;
    return XPRESS_OK;
}

// Plan, workspace and launches shared by both readouts.
int run_readout(const uint16_t* base, const uint16_t* bias, const int64_t* cand, int64_t* blk,
                int64_t N, int64_t B, int64_t V, int64_t sb, int64_t sbi, hipStream_t stream)
{
    int64_t rows = 0;
    int rc = validate(base, bias, blk, N, B, V, sb, sbi, cand, &rows);
    if (rc != XPRESS_OK || rows == 0) return rc;

    const Plan p = make_plan(base, bias, rows, V, sb, sbi);
    RowArgs a = row_args(base, bias, cand, blk, rows, B, V, sb, sbi, p);

    if (p.combine != kSingle) {
        Workspace* w = nullptr;
        const int64_t table = (p.combine == kTwoPass) ? rows * p.splits : 0;
        const bool words = (p.combine == kAtomic || p.combine == kBalanced);
        rc = ensure_workspace(stream, words ? rows : 0, table, &w);
        if (rc != XPRESS_OK) return rc;
        a.keys = words ? w->keys : w->table;
    }

    return launch_readout_plan(a, p, stream);
}

}  // namespace

namespace xpress {

XPRESS_INTERNAL thread_local int g_last_hip_error = 0;

void note_hip_error(hipError_t e) { g_last_hip_error = (int)e; }

int hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return XPRESS_EHIP;
}

int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        n = 256;
    }
    if (dev < 64) cached[dev] = n;
    return n;
}

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool reverse_order() { return g_reverse_order.load() != 0; }

bool ranges_overlap(const void* p0, size_t n0, const void* p1, size_t n1)
{
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p0), a1 = a0 + n0;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(p1), b1 = b0 + n1;
    return a0 < b1 && b0 < a1;
}

int workspace_table(hipStream_t stream, int64_t entries, uint64_t** table)
{
    Workspace* w = nullptr;
    const int rc = ensure_workspace(stream, 0, entries, &w);
    if (rc != XPRESS_OK) return rc;
    *table = w->table;
    return XPRESS_OK;
}

hipError_t launch_reduce_table(uint64_t* table, int64_t* blk, const int64_t* cand, uint32_t rows,
                               uint32_t bm1, uint32_t V, uint32_t splits, hipStream_t stream)
{
    RowArgs a = {};
    a.blk = blk;
    a.rows = rows;
    a.bm1 = bm1;
    a.V = V;
    a.splits = splits;
    a.keys = table;
    a.cand = cand;
    const uint32_t grid = (rows + 3u) / 4u < 65536u ? (rows + 3u) / 4u : 65536u;
    hipLaunchKernelGGL(reduce_keys_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace xpress

extern "C" {

int xpress_add_argmax_to_blk(const uint16_t* base, const uint16_t* bias, int64_t* blk,
                             int64_t N, int64_t B, int64_t V, int64_t stride_base_r,
                             int64_t stride_bias_r, hipStream_t stream)
{
    return run_readout(base, bias, nullptr, blk, N, B, V, stride_base_r, stride_bias_r,
                       stream);
}

int xpress_add_argmax_to_blk_noalloc(const uint16_t* base, const uint16_t* bias, int64_t* blk,
                                     int64_t N, int64_t B, int64_t V, int64_t stride_base_r,
                                     int64_t stride_bias_r, hipStream_t stream)
{
    int64_t rows = 0;
    int rc = validate(base, bias, blk, N, B, V, stride_base_r, stride_bias_r, nullptr, &rows);
    if (rc != XPRESS_OK || rows == 0) return rc;
    Plan p = make_plan(base, bias, rows, V, stride_base_r, stride_bias_r);
    // split rows always meet in two passes here: the table is overwritten
    // whole by every call, so nothing in the shared array has to start at
    // zero
    if (p.combine != kSingle) {
        p.combine = kTwoPass;
        p.launches = 2;
    }
    RowArgs a = row_args(base, bias, nullptr, blk, rows, B, V, stride_base_r, stride_bias_r, p);
    if (p.combine == kTwoPass) {
        if (rows * (int64_t)p.splits > kScratchKeys) return XPRESS_ESCRATCH;
        rc = scratch_table(&a.keys);
        if (rc != XPRESS_OK) return rc;
    }
    return launch_readout_plan(a, p, stream);
}

int xpress_topc_argmax_to_blk(const uint16_t* base_c, const uint16_t* bias_c,
                              const int64_t* cand, int64_t* blk, int64_t N, int64_t B,
                              int64_t C, hipStream_t stream)
{
    if (N > 0 && B > 1 && cand == nullptr) return XPRESS_EINVAL;
    int override_combine;
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        override_combine = g_override_combine;
    }
    if (override_combine != XPRESS_COMBINE_AUTO || C > kTopcWaveMaxC) {
        return run_readout(base_c, bias_c, cand, blk, N, B, C, C, C, stream);
    }
    int64_t rows = 0;
    int rc = validate(base_c, bias_c, blk, N, B, C, C, C, cand, &rows);
    if (rc != XPRESS_OK || rows == 0) return rc;
    const bool vec = is_aligned16(base_c) && is_aligned16(bias_c) && is_aligned16(cand) &&
                     (C % 8 == 0);
    const int64_t blocks = (rows + 3) / 4;
    const uint32_t grid = (uint32_t)(blocks < 65536 ? blocks : 65536);
    if (vec) {
        hipLaunchKernelGGL(topc_wave_kernel<true>, dim3(grid), dim3(256), 0, stream, base_c,
                           bias_c, cand, blk, (uint32_t)rows, (uint32_t)(B - 1), (uint32_t)C);
    } else {
        hipLaunchKernelGGL(topc_wave_kernel<false>, dim3(grid), dim3(256), 0, stream, base_c,
                           bias_c, cand, blk, (uint32_t)rows, (uint32_t)(B - 1), (uint32_t)C);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}

int xpress_reserve(int64_t N, int64_t B, int64_t V, hipStream_t stream)
{
    if (N < 0 || B < 1 || V < 1 || V > 0x7FFFFFFFll) return XPRESS_EINVAL;
    if (B - 1 > 0 && N > 0x7FFFFFFFll / (B - 1)) return XPRESS_EINVAL;
    const int64_t rows = N * (B - 1);
    if (rows == 0) return XPRESS_OK;
    // reserve for both the aligned and the unaligned plan of this shape
    const uint16_t* aligned = reinterpret_cast<const uint16_t*>(uintptr_t(256));
    const Plan pv = make_plan(aligned, aligned, rows, V, (V + 7) / 8 * 8, (V + 7) / 8 * 8);
    const Plan ps = make_plan(aligned + 1, aligned + 1, rows, V, V | 1, V | 1);
    int64_t table = 0;
    if (pv.combine == kTwoPass) table = rows * pv.splits;
    if (ps.combine == kTwoPass && rows * ps.splits > table) table = rows * ps.splits;
    Workspace* w = nullptr;
    const int rc = ensure_workspace(stream, rows, table, &w);
    if (rc != XPRESS_OK) return rc;
    // also look up the no-allocation variant's table on this device
    uint64_t* fixed = nullptr;
    return scratch_table(&fixed);
}

int xpress_release(void)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    for (auto it = g_ws.begin(); it != g_ws.end();) {
        if (it->first.first == dev) {
            if (it->second.keys) (void)hipFree(it->second.keys);
            if (it->second.table) (void)hipFree(it->second.table);
            it = g_ws.erase(it);
        } else {
            ++it;
        }
    }
    for (void* p : g_retired[dev]) (void)hipFree(p);
    g_retired[dev].clear();
    g_ws_bytes[dev] = 0;
    return XPRESS_OK;
}

int xpress_set_workspace_limit(int64_t bytes)
{
    if (bytes < 0) return XPRESS_EINVAL;
    std::lock_guard<std::mutex> lk(g_ws_mu);
    g_ws_limit = bytes;
    return XPRESS_OK;
}

int xpress_workspace_bytes(int64_t* live_and_retired)
{
    if (!live_and_retired) return XPRESS_EINVAL;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lk(g_ws_mu);
    *live_and_retired = g_ws_bytes[dev];
    return XPRESS_OK;
}

int xpress_set_plan(int combine, int splits, int block_threads)
{
    if (combine < XPRESS_COMBINE_AUTO || combine > XPRESS_COMBINE_BALANCED) return XPRESS_EINVAL;
    if (splits < 0) return XPRESS_EINVAL;
    if (block_threads != 0 && block_threads != 64 && block_threads != 128 &&
        block_threads != 256 && block_threads != 512 && block_threads != 1024) {
        return XPRESS_EINVAL;
    }
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_override_combine = combine;
    g_override_splits = splits;
    g_override_threads = block_threads;
    return XPRESS_OK;
}

int xpress_set_reverse_order(int reversed)
{
    g_reverse_order.store(reversed ? 1 : 0);
    return XPRESS_OK;
}

int xpress_describe_plan(const uint16_t* base, const uint16_t* bias, int64_t N, int64_t B,
                         int64_t V, int64_t stride_base_r, int64_t stride_bias_r,
                         int* combine, int* splits, int* block_threads, int* vector_path,
                         int* launches)
{
    if (N < 0 || B < 1 || V < 1 || V > 0x7FFFFFFFll || stride_base_r < V ||
        stride_bias_r < V) {
        return XPRESS_EINVAL;
    }
    const int64_t rows = N * (B - 1);
    const Plan p = make_plan(base, bias, rows > 0 ? rows : 1, V, stride_base_r, stride_bias_r);
    if (combine) *combine = p.combine;
    if (splits) *splits = p.splits;
    if (block_threads) *block_threads = p.threads;
    if (vector_path) *vector_path = p.vec ? 1 : 0;
    if (launches) *launches = rows > 0 ? p.launches : 0;
    return XPRESS_OK;
}

int xpress_bf16_add_round_table(const uint16_t* a_vals, int64_t n_a, uint16_t* out,
                                hipStream_t stream)
{
    if (n_a < 0 || n_a > 65536) return XPRESS_EINVAL;
    if (n_a == 0) return XPRESS_OK;
    if (!a_vals || !out || (reinterpret_cast<uintptr_t>(out) & 3u)) return XPRESS_EINVAL;
    const uint64_t total = (uint64_t)n_a * 32768u;
    const uint64_t blocks = (total + 255) / 256;
    const uint32_t grid = (uint32_t)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(round_table_kernel, dim3(grid), dim3(256), 0, stream, a_vals,
                       (uint32_t)n_a, reinterpret_cast<uint32_t*>(out));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}

int xpress_last_hip_error(void) { return xpress::g_last_hip_error; }

const char* xpress_error_string(int status)
{
    switch (status) {
        case XPRESS_OK: return "ok";
        case XPRESS_EINVAL: return "invalid argument: the sizes, strides or pointers describe no valid layout";
        case XPRESS_EHIP: return "a HIP call failed (see xpress_last_hip_error)";
        case XPRESS_ENOMEM: return "could not allocate the device workspace";
        case XPRESS_ECAPTURE: return "the workspace must grow while the stream is capturing; call xpress_reserve first";
        case XPRESS_ESCRATCH: return "the call needs more than the no-allocation variant's fixed key table (4096 keys)";
        default: return "unknown status";
    }
}

const char* xpress_version(void) { return "0.1.0"; }

}  // extern "C"
