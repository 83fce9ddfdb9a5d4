// read_probe.hip -- a plain streaming read of the readout's two inputs, for
// measuring the practical HBM read ceiling that the readout's access pattern
// can reach on this part.  Not on the readout's path: the benchmark reports
// it beside the readout so that the readout's rate can be read against what
// reading the same bytes costs.
//
// Two patterns over the same buffers:
//   * per row: one 256-thread workgroup per row, 16-byte non-temporal loads,
//     two vectors of each stream in flight per thread -- the readout's own
//     layout and launch shape at a few hundred rows, with the arithmetic
//     taken out;
//   * grid-stride: two workgroups of 256 threads per compute unit sweep the
//     flattened arrays (first row's start to last row's end) in lockstep,
//     every workgroup on the next 4 KiB of each stream -- the most
//     favourable order for the memory
//     system, which a per-row argmax cannot use without a cross-workgroup
//     reduction per row segment.
// Each thread folds what it reads into one word so that no load is dead; the
// word is stored only if it equals a constant the data would have to hit by
// chance (the store is there to keep the loads, not to report anything).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "xpress_argmax.h"
#include "device_common.h"
#include "host_common.h"

namespace {

using namespace xpress;

constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__device__ __forceinline__ uint32_t fold(const u32x4& a, const u32x4& b)
{
    return a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
}

template <int T, int U>
__global__ __launch_bounds__(T) void read_rows_kernel(const uint16_t* __restrict__ base,
                                                      const uint16_t* __restrict__ bias,
                                                      uint32_t rows, uint32_t nvec,
                                                      int64_t stride, uint32_t* sink)
{
    uint32_t acc = 0;
    for (uint32_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const u32x4* pa = reinterpret_cast<const u32x4*>(base + (int64_t)row * stride);
        const u32x4* pb = reinterpret_cast<const u32x4*>(bias + (int64_t)row * stride);
        uint32_t q = threadIdx.x;
        for (; q + (U - 1) * T < nvec; q += U * T) {
            u32x4 va[U], vb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                va[u] = __builtin_nontemporal_load(pa + q + u * T);
                vb[u] = __builtin_nontemporal_load(pb + q + u * T);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= fold(va[u], vb[u]);
        }
        for (; q < nvec; q += T) {
            acc ^= fold(__builtin_nontemporal_load(pa + q), __builtin_nontemporal_load(pb + q));
        }
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

template <int U>
__global__ __launch_bounds__(256) void read_flat_kernel(const uint16_t* __restrict__ base,
                                                        const uint16_t* __restrict__ bias,
                                                        uint64_t nvec, uint32_t* sink)
{
    const u32x4* pa = reinterpret_cast<const u32x4*>(base);
    const u32x4* pb = reinterpret_cast<const u32x4*>(bias);
    uint32_t acc = 0;
    const uint64_t step = (uint64_t)gridDim.x * 256u * U;
    for (uint64_t i = (uint64_t)blockIdx.x * 256u * U + threadIdx.x; i < nvec; i += step) {
        // every load of the batch is issued before any is used (a load
        // inside a branch would be waited for on its own)
        u32x4 va[U], vb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + (uint64_t)u * 256u;
            const bool in = j < nvec;
            va[u] = in ? __builtin_nontemporal_load(pa + j) : u32x4{0u, 0u, 0u, 0u};
            vb[u] = in ? __builtin_nontemporal_load(pb + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(va[u], vb[u]);
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

}  // namespace

extern "C" int xpress_read_probe(const uint16_t* base, const uint16_t* bias, int64_t rows,
                                 int64_t V, int64_t stride, int mode, uint32_t* sink,
                                 hipStream_t stream)
{
    if (rows < 0 || V < 8 || V % 8 != 0 || stride < V || stride % 8 != 0 || rows > 0x7FFFFFFFll ||
        V > 0x7FFFFFFFll || (mode != XPRESS_READ_ROWS && mode != XPRESS_READ_FLAT)) {
        return XPRESS_EINVAL;
    }
    if (rows == 0) return XPRESS_OK;
    if (!base || !bias || !sink || !is_aligned16(base) || !is_aligned16(bias)) return XPRESS_EINVAL;
    if (mode == XPRESS_READ_ROWS) {
        const uint32_t grid = (uint32_t)(rows < (1 << 22) ? rows : (1 << 22));
        hipLaunchKernelGGL((read_rows_kernel<256, 2>), dim3(grid), dim3(256), 0, stream, base,
                           bias, (uint32_t)rows, (uint32_t)(V / 8), stride, sink);
    } else {
        // from the first row's start to the last row's end, padding between
        // rows included
        const uint64_t nvec = ((uint64_t)(rows - 1) * (uint64_t)stride + (uint64_t)V) / 8u;
        hipLaunchKernelGGL((read_flat_kernel<2>), dim3(2 * device_cus()), dim3(256), 0, stream,
                           base, bias, nvec, sink);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    return XPRESS_OK;
}
