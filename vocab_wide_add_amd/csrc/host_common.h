// host_common.h -- host-side helpers shared by the translation units of
// libxpress_argmax.  Internal: hidden from the library's exported symbols.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#define XPRESS_INTERNAL __attribute__((visibility("hidden")))

namespace xpress {

// Records e as the thread's last HIP error and returns XPRESS_EHIP.
XPRESS_INTERNAL int hip_fail(hipError_t e);

// Records e as the thread's last HIP error (without choosing a status).
XPRESS_INTERNAL void note_hip_error(hipError_t e);

// Compute units of the current device (cached per device).
XPRESS_INTERNAL int device_cus();

XPRESS_INTERNAL bool is_aligned16(const void* p);

// Whether launches should visit their work units in reverse order (the
// debug setting of xpress_set_reverse_order).
XPRESS_INTERNAL bool reverse_order();

XPRESS_INTERNAL bool ranges_overlap(const void* p0, size_t n0, const void* p1, size_t n1);

// The (device, stream) workspace's key table, grown to at least `entries`
// u64 slots.  Returns XPRESS_OK, XPRESS_ECAPTURE, XPRESS_ENOMEM or XPRESS_EHIP.
XPRESS_INTERNAL int workspace_table(hipStream_t stream, int64_t entries, uint64_t** table);

// Second pass of a split readout: for every row the largest of its `splits`
// packed keys in table[row * splits ...] names the winner, and blk[n, 1 + b]
// receives its index, or cand[row * V + index] when cand is not null (the
// top-C readout's candidate ids, V candidates per row).
XPRESS_INTERNAL hipError_t launch_reduce_table(uint64_t* table, int64_t* blk,
                                               const int64_t* cand, uint32_t rows,
                                               uint32_t bm1, uint32_t V, uint32_t splits,
                                               hipStream_t stream);

}  // namespace xpress
