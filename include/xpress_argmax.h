/*
 * xpress_argmax.h -- C ABI of the MI355X (gfx950) fused add + argmax readout.
 *
 * The operation (XPress kernels page, "fused_add_argmax_to_blk" and its stage
 * kernels "_xpress_add_argmax_partial_kernel" /
 * "_xpress_add_argmax_reduce_to_blk_kernel"): one Jacobi pass drafts B-1 slots
 * in each of N blocks; draft row r = n*(B-1) + b carries base logits and a
 * refiner bias over a vocabulary of V ids, and the readout writes
 *
 *     blk[n, 1 + b] = argmax_v  bf16( base[r, v] + bias[r, v] )
 *
 * without ever storing the [N*(B-1), V] sum.  Each sum is formed from the two
 * bf16 values and rounded once to bf16 (round-to-nearest, ties to even,
 * subnormals kept) before the comparison, as the stage-1 kernel does by
 * casting the sum back to the input dtype; values compare as reals (-0 equals
 * +0) and the lowest vocabulary id wins a tie (the first-maximum argmax of a
 * chunk followed by a strict ">" scan over chunks in ascending order).  Slot
 * 0 of every block (the verified anchor) is never written; the next pass
 * reads blk in place.  NaN inputs are outside the contract.
 *
 * Everything here is plain C: pointers, 64-bit sizes and a HIP stream.
 * No function keeps a reference to a caller buffer after it returns.
 */
#ifndef XPRESS_ARGMAX_H
#define XPRESS_ARGMAX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define XPRESS_OK 0
#define XPRESS_EINVAL 1   /* an argument describes no valid layout */
#define XPRESS_EHIP 2     /* a HIP call failed; see xpress_last_hip_error() */
#define XPRESS_ENOMEM 3   /* the library could not allocate its workspace */
#define XPRESS_ECAPTURE 4 /* the workspace would have to grow while the stream
                             is being captured into a graph; call
                             xpress_reserve() before capturing */
#define XPRESS_ESCRATCH 5 /* the call needs more than the fixed key table of
                             xpress_add_argmax_to_blk_noalloc */

/*
 * xpress_add_argmax_to_blk -- the fused readout (page and passages above).
 *
 *   base           device pointer to bf16 bit patterns, N*(B-1) rows; row r
 *                  starts at base + r*stride_base_r and holds V elements with
 *                  unit stride.  Read only.
 *   bias           device pointer, the refiner bias, laid out like base with
 *                  its own row stride.  Read only; may alias base.
 *   blk            device pointer to int64 [N, B], row-major and contiguous.
 *                  blk[n*B + 1 + b] receives the winning vocabulary id of row
 *                  n*(B-1) + b; blk[n*B] and all other memory are untouched.
 *                  Must not overlap base or bias.
 *   N              blocks, >= 0.
 *   B              slots per block (anchor + B-1 drafts), >= 1.
 *   V              vocabulary size, 1 <= V <= 2^31 - 1.
 *   stride_base_r  row stride of base in elements, >= V.
 *   stride_bias_r  row stride of bias in elements, >= V.
 *   stream         HIP stream the work is queued on (0 = the null stream).
 *
 * Asynchronous: returns once the kernels are queued; blk is valid after the
 * stream reaches that point.  N == 0 or B == 1 (no draft rows) returns
 * XPRESS_OK and queues nothing.  Any layout is accepted; rows whose starts
 * and strides are 16-byte aligned take the vector path, others a scalar path
 * with identical results.
 *
 * Errors: XPRESS_EINVAL for a negative N, B < 1, V out of range, a stride
 * below V, a null pointer when there are rows, or blk overlapping an input
 * (nothing is queued); XPRESS_ENOMEM / XPRESS_ECAPTURE when the workspace
 * cannot be provided; XPRESS_EHIP when a launch fails.  Faults inside the
 * kernels (e.g. a pointer to too small a buffer) surface at the caller's
 * next synchronisation, as for any HIP kernel.
 *
 * Workspace: when the chosen plan splits a row over several workgroups the
 * library uses a small device workspace of its own (8 bytes per row, or per
 * row and split for the two-pass plan),
 * one per (device, stream), allocated on first use and left zeroed by every
 * call, so repeated calls and graph replays need no clearing.  Calls queued
 * on different streams use different workspaces and may run concurrently.
 * When a later call needs more, the workspace grows (synchronously, outside
 * capture only) into a new allocation and the old one is retired, not freed:
 * queued work and HIP graphs captured before keep valid memory until
 * xpress_release.  The same rules hold for every entry point below that
 * uses the workspace.
 * The caller keeps every buffer alive until the queued work has finished.
 * Host threads: the library's own tables are locked, but a call holds its
 * stream's workspace from lookup to launch, so calls that queue on one
 * stream come from one host thread at a time, and xpress_release runs while
 * no other call of the library is in progress on any thread.
 */
int xpress_add_argmax_to_blk(const uint16_t* base, const uint16_t* bias,
                             int64_t* blk, int64_t N, int64_t B, int64_t V,
                             int64_t stride_base_r, int64_t stride_bias_r,
                             hipStream_t stream);

/*
 * xpress_add_argmax_to_blk_noalloc -- the same readout as
 * xpress_add_argmax_to_blk (same arguments, layout rules, result and errors)
 * for callers that cannot allocate device memory: code being captured into a
 * HIP graph without a prior xpress_reserve, tight serving loops, harnesses
 * that forbid allocation.  It never calls hipMalloc, hipFree or any other
 * allocating routine.  Rows that the plan splits over several workgroups
 * meet in two passes through a fixed key table of 4096 keys, a device array
 * built into the library (one copy per GPU, 32 KiB, held until the process
 * ends); the table holds rows x splits keys, which the automatic plan keeps
 * below 700, and a call that would need more (e.g. a split count forced with
 * xpress_set_plan) returns XPRESS_ESCRATCH and queues nothing.  Atomic and
 * balanced plans set with xpress_set_plan run as two-pass here.  Every call
 * on one GPU shares that table and overwrites it whole: calls that may run
 * at the same time on one GPU (e.g. queued on different streams) race and
 * must not overlap.  Asynchronous, like xpress_add_argmax_to_blk.  The
 * first call on a device (or xpress_reserve there) looks the table's device
 * address up with hipGetSymbolAddress; make one of them outside graph
 * capture before capturing this call.
 */
int xpress_add_argmax_to_blk_noalloc(const uint16_t* base, const uint16_t* bias,
                                     int64_t* blk, int64_t N, int64_t B, int64_t V,
                                     int64_t stride_base_r, int64_t stride_bias_r,
                                     hipStream_t stream);

/*
 * xpress_topc_argmax_to_blk -- the top-C readout (XPress kernels page,
 * "_xpress_topc_argmax_to_blk_kernel" and "fused_topc_argmax_to_blk"): each
 * draft row r = n*(B-1) + j carries C candidates; the first candidate
 * maximising bf16(base_c[r, c] + bias_c[r, c]) -- same element and tie rule
 * as above -- wins, and its vocabulary id is written:
 *
 *     blk[n, 1 + j] = cand[r, first argmax_c bf16(base_c[r, c] + bias_c[r, c])]
 *
 *   base_c, bias_c  device pointers to bf16 bit patterns, [N, B-1, C]
 *                   contiguous (row r at r*C).  Read only.
 *   cand            device pointer to int64 ids, [N, B-1, C] contiguous.
 *                   Read only; the winner's id is copied as is.
 *   blk             device pointer to int64 [N, B]; slots 1..B-1 written,
 *                   slot 0 untouched.  Must not overlap any input.
 *   N, B            as above; C >= 1 candidates per row (<= 2^31 - 1).
 *   stream          HIP stream (0 = the null stream).
 *
 * Asynchronous; same no-op and error rules as xpress_add_argmax_to_blk.
 * With the automatic plan, lists of up to 256 candidates are read by one wave
 * per row that carries the ids along (no second round trip for the gather);
 * longer lists, or any plan set with xpress_set_plan, take the streaming
 * readout with V = C and row strides C and gather the id when writing blk.
 */
int xpress_topc_argmax_to_blk(const uint16_t* base_c, const uint16_t* bias_c,
                              const int64_t* cand, int64_t* blk, int64_t N,
                              int64_t B, int64_t C, hipStream_t stream);

/*
 * xpress_readout_gemm_argmax_to_blk -- the readout with the refiner bias
 * computed in place (XPress kernels page, module description: a pass forms
 * logits = base + x @ W2 with a readout matmul and then takes the argmax; the
 * fused add + argmax consumes the matmul's bf16 result as its bias).  Here
 * the matmul runs on the matrix cores inside the readout and neither the
 * bias nor the logits are ever written:
 *
 *     bias[r, v]    = bf16( sum_k x[r, k] * w[v, k] )   (fp32 accumulation,
 *                                                         rounded once)
 *     blk[n, 1 + b] = first argmax_v bf16( base[r, v] + bias[r, v] )
 *
 *   base           device pointer, bf16 [N*(B-1), V] with row stride
 *                  stride_base_r (elements, >= V, a multiple of 8).
 *   x              device pointer, bf16 [N*(B-1), R] row-major (the latent
 *                  rows the refiner produced for the draft slots).
 *   w              device pointer, bf16 [V, R] row-major (the readout
 *                  weight, one row per vocabulary id; W2 = w^T).
 *   blk            device pointer to int64 [N, B]; slots 1..B-1 written.
 *   N, B, V        as for xpress_add_argmax_to_blk.
 *   R              latent width: 64, 128 or 256.
 *   stream         HIP stream (0 = the null stream).
 *
 * base, x and w must be 16-byte aligned (XPRESS_EINVAL otherwise).  The fp32
 * accumulation order is the matrix cores'; where every partial sum of the
 * dot products is exact (e.g. inputs on a coarse dyadic grid) the result is
 * bit-identical to rounding the exact dot product.  Asynchronous; two
 * launches; uses the (device, stream) workspace (rows x ranges keys, at most
 * rows x 512 x 8 bytes), grown on first use.  xpress_reserve does not size
 * it: before capturing this call into a HIP graph, make one call with at
 * least as many rows on the same stream outside capture (a capture that
 * would have to grow it returns XPRESS_ECAPTURE and queues nothing).  Later
 * growth retires the old table rather than freeing it, so graphs captured
 * earlier stay valid until xpress_release.
 */
int xpress_readout_gemm_argmax_to_blk(const uint16_t* base, const uint16_t* x,
                                      const uint16_t* w, int64_t* blk, int64_t N,
                                      int64_t B, int64_t V, int64_t R,
                                      int64_t stride_base_r, hipStream_t stream);

/*
 * xpress_reserve -- pre-allocate the workspace the readout would use for
 * (N, B, V) on `stream`'s device and stream, so that a later call -- e.g.
 * one being captured into a HIP graph -- allocates nothing; it also looks
 * up the device address of xpress_add_argmax_to_blk_noalloc's table.
 * Synchronous.
 * Returns XPRESS_OK, XPRESS_EINVAL, XPRESS_ENOMEM or XPRESS_EHIP.
 */
int xpress_reserve(int64_t N, int64_t B, int64_t V, hipStream_t stream);

/*
 * xpress_latent_pass -- the latent stage of one Jacobi pass (XPress kernels
 * page, module description and "_xpress_latent_kernel"), which produces the
 * rows the readout matmul consumes.  For every block n and slot b:
 *
 *     prev[b]  = am1[n] for b = 0, blk[n, b-1] otherwise
 *     x[b, :]  = xh[n, b, :] + w1[prev[b], :] @ wlat^T          (fp32)
 *     u[b, r]  = sum_{j < B} mixl[b, j, r] * x[j, r]             (fp32)
 *     g        = bf16(u[b]) @ wg^T,   v = bf16(u[b]) @ wu^T      (fp32)
 *     m        = bf16( g * sigmoid(g) * v )                      (SwiGLU)
 *     lat_out[n, b-1, :] = bf16( u[b] + m @ wd^T ),   b = 1 .. B-1
 *
 * Slot 0 is the verified anchor: its x enters the mixer of the later slots,
 * but no latent is written for it.
 *
 *   blk      device pointer, int64 [N, B] row-major: the block's tokens; slot
 *            b reads blk[n, b-1] (blk[n, B-1] is never read).  Read only.
 *   am1      device pointer, int64 [N]: the token before each block's anchor.
 *   xh       device pointer, bf16 [N, B, R]: the pass-invariant hidden cache.
 *   w1       device pointer, bf16 [V, R]: token embedding, one row per id.
 *   wlat     device pointer, bf16 [R, R]: embedding-to-latent projection,
 *            out-major (row r holds the weights of output channel r).
 *   mixl     device pointer, bf16 [B, B, R]: the folded mixer (L * tril + I)
 *            per channel; every j < B is summed, so entries above the
 *            diagonal must be zero for a causal mixer.
 *   wg, wu   device pointers, bf16 [H, R]: SwiGLU gate and up, out-major.
 *   wd       device pointer, bf16 [R, H]: SwiGLU down, out-major.
 *   lat_out  device pointer, bf16 [N, B-1, R]: written whole.  Must not
 *            overlap any input.
 *   N        blocks, >= 0 (N * B <= 2^31 - 1).
 *   B        slots per block, 2 .. 32.
 *   R        latent rank, a multiple of 64 in [64, 1024].
 *   H        MLP hidden size, a multiple of 64 in [64, 8192].
 *   V        rows of w1, >= 1.
 *   stream   HIP stream (0 = the null stream).
 *
 * xh, w1, wlat, mixl, wg, wu and wd must be 16-byte aligned; blk and am1
 * 8-byte aligned.  A token id outside [0, V) reads as a zero embedding row (no
 * out-of-bounds read; the result for that slot is then meaningless).  The
 * fp32 accumulation order is the matrix cores'; results agree with the exact
 * definition up to fp32 rounding of the sums before each bf16 rounding.
 *
 * Asynchronous; three launches on `stream`.  N == 0 queues nothing.  Uses the
 * (device, stream) workspace for u, bf16(u) and m (rows * (6R + 2H) bytes,
 * rows = N * (B-1)); grow it beforehand with xpress_latent_reserve when the
 * call will be captured into a HIP graph (growth retires the old regions
 * rather than freeing them, as for the readouts).  Errors: XPRESS_EINVAL (sizes,
 * alignment, null pointers, overlap; nothing queued), XPRESS_ENOMEM /
 * XPRESS_ECAPTURE (workspace), XPRESS_EHIP (launch).
 */
int xpress_latent_pass(const int64_t* blk, const int64_t* am1, const uint16_t* xh,
                       const uint16_t* w1, const uint16_t* wlat, const uint16_t* mixl,
                       const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                       uint16_t* lat_out, int64_t N, int64_t B, int64_t R, int64_t H,
                       int64_t V, hipStream_t stream);

/*
 * xpress_latent_reserve -- grow the (device, stream) workspace to what
 * xpress_latent_pass needs for (N, B, R, H), so that a captured call
 * allocates nothing.  Synchronous.  Returns XPRESS_OK, XPRESS_EINVAL,
 * XPRESS_ENOMEM or XPRESS_EHIP.  Growing the workspace later (a larger shape
 * on the same stream) retires the old regions, which graphs captured before
 * keep using until xpress_release.
 */
int xpress_latent_reserve(int64_t N, int64_t B, int64_t R, int64_t H, hipStream_t stream);

/*
 * xpress_latent_set_tiles -- workgroup shape override for the three latent
 * kernels, for tests and tuning.  Each workgroup computes 32 * slabs rows of
 * a 32-column tile with its four waves; slabs = 4 gives every wave its own
 * 32-row slab over the whole contraction, slabs = 2 or 1 split the
 * contraction over 2 or 4 waves and sum the partials in LDS; 8 selects the
 * LDS-staged kernels (128 rows per workgroup, operands copied to LDS in
 * coalesced 64-wide contraction chunks, up to four in flight).  Arguments are the
 * choices for the mix, gate and down kernels: 1, 2, 4 or 8, or 0 for the
 * library's choice per shape (staged from 2048 rows on, else the most slabs
 * that still give each compute unit a workgroup).  Results are identical up
 * to fp32 summation order.
 * Process-wide; returns XPRESS_OK or XPRESS_EINVAL.
 */
int xpress_latent_set_tiles(int mix, int gate, int down);

/*
 * xpress_release -- free every workspace the library holds on the current
 * device, live and retired (after synchronising that device).  Optional; for
 * tests and for callers that want the memory back.  No other call of the
 * library may be in progress meanwhile, and graphs captured before hold freed
 * workspace and must not be replayed; the next call allocates afresh.
 */
int xpress_release(void);

/*
 * xpress_set_workspace_limit -- cap, in bytes, on the workspace (live plus
 * retired) the library may hold per device; 0 (the default) means no cap.
 * A call whose workspace would have to grow past the cap returns
 * XPRESS_ENOMEM and queues nothing, exactly as when the device is out of
 * memory.  Process-wide.  Returns XPRESS_OK, or XPRESS_EINVAL for a negative
 * cap.
 */
int xpress_set_workspace_limit(int64_t bytes);

/*
 * xpress_workspace_bytes -- *live_and_retired = the bytes of workspace the
 * library holds on the current device.  Returns XPRESS_OK, XPRESS_EINVAL
 * (null pointer) or XPRESS_EHIP.
 */
int xpress_workspace_bytes(int64_t* live_and_retired);

/*
 * Plan override, for tests and tuning.  combine selects how a row's partial
 * results meet:
 *   XPRESS_COMBINE_AUTO    the library's measured choice per shape;
 *   XPRESS_COMBINE_SINGLE  one workgroup per row, no cross-workgroup step;
 *   XPRESS_COMBINE_ATOMIC  several workgroups per row; each folds its packed
 *                          (value, ~index) key into a per-row 64-bit word that
 *                          also counts arrivals, by compare-and-swap; the last
 *                          to arrive writes blk and clears the word (one
 *                          launch);
 *   XPRESS_COMBINE_TWO_PASS several workgroups per row write their packed key
 *                          to a [rows, splits] table, a second small kernel
 *                          reduces each row (two launches);
 *   XPRESS_COMBINE_BALANCED the rows' 16-byte vectors, in row-major order, are
 *                          cut into equal contiguous ranges, one per
 *                          workgroup, over a whole number of workgroups per
 *                          CU; rows shared by several ranges are folded as in
 *                          ATOMIC (one launch; needs the aligned layout and
 *                          V >= 8, else it falls back to SINGLE).
 * splits is the number of workgroups per row (0 = automatic; ignored by
 * SINGLE); for BALANCED it is the number of workgroups per CU.  block_threads
 * is the workgroup size (0 = automatic, else 64, 128, 256, 512 or 1024).  The
 * setting is process-wide and applies to later calls.  Returns XPRESS_EINVAL
 * for an unknown combine or block size.
 */
#define XPRESS_COMBINE_AUTO 0
#define XPRESS_COMBINE_SINGLE 1
#define XPRESS_COMBINE_ATOMIC 2
#define XPRESS_COMBINE_TWO_PASS 3
#define XPRESS_COMBINE_BALANCED 4
int xpress_set_plan(int combine, int splits, int block_threads);

/*
 * xpress_set_reverse_order -- a debug setting for checking that results do
 * not depend on the order in which workgroups run.  With reversed nonzero,
 * later launches of the streaming readout (every combine, and the top-C
 * readout when it takes that path) visit their (row, split) units, or their
 * balanced ranges, from last to first, and the readout with in-place bias
 * maps its workgroups to (vocabulary range, row block) pairs from last to
 * first within each XCD; the work each workgroup does is unchanged, only
 * which runs early and which late, so the combines see their keys arrive in
 * another order.  Every result must be bit-identical to the default order's.
 * Process-wide; 0 restores the default.  Always returns XPRESS_OK.
 */
int xpress_set_reverse_order(int reversed);

/*
 * xpress_describe_plan -- what a call with these sizes and alignments would
 * launch: *combine, *splits, *block_threads, *vector_path (1 = 16-byte loads)
 * and *launches.  Pure host computation.  Returns XPRESS_OK or XPRESS_EINVAL.
 */
int xpress_describe_plan(const uint16_t* base, const uint16_t* bias, int64_t N,
                         int64_t B, int64_t V, int64_t stride_base_r,
                         int64_t stride_bias_r, int* combine, int* splits,
                         int* block_threads, int* vector_path, int* launches);

/*
 * xpress_describe_gemm_plan -- the launch shape xpress_readout_gemm_argmax_to_blk
 * would use for (N, B, V): *waves per workgroup (1, 2 or 8; each wave holds
 * 64 draft rows), *ranges (the vocabulary is cut into this many contiguous
 * ranges of whole 32-id tiles, a multiple of 8), *row_wgs (workgroups per
 * range) and *tiles (ceil(V / 32)).  Any output may be null.  Pure host
 * computation on the current device's compute-unit count.  Returns
 * XPRESS_OK or XPRESS_EINVAL.
 */
int xpress_describe_gemm_plan(int64_t N, int64_t B, int64_t V, int* waves, int* ranges,
                              int* row_wgs, int* tiles);

/*
 * xpress_bf16_add_round_table -- the readout's element step alone, for
 * checking it against the definition over every input pair.  For each i in
 * [0, n_a) and each of the 65536 bf16 patterns b it writes
 * out[i*65536 + b] = bf16(a_vals[i] + b) with the same device code the
 * readout kernels use.  a_vals (n_a entries) and out (n_a*65536 entries) are
 * device pointers.  Asynchronous on stream.  Returns XPRESS_OK,
 * XPRESS_EINVAL (n_a < 0, null pointer) or XPRESS_EHIP.
 */
int xpress_bf16_add_round_table(const uint16_t* a_vals, int64_t n_a,
                                uint16_t* out, hipStream_t stream);

/*
 * xpress_read_probe -- a plain streaming read of the readout's two inputs,
 * with no arithmetic on them: the practical read ceiling against which the
 * readout's rate is reported.  Not part of the readout.  base and bias are
 * rows rows of V bf16 at row stride `stride` (elements; V and stride
 * multiples of 8, 16-byte aligned pointers).  mode XPRESS_READ_ROWS reads
 * every row's V elements with one 256-thread workgroup per row (the
 * readout's launch shape at a few hundred rows); XPRESS_READ_FLAT sweeps
 * every element from the first row's start to the last row's end (padding
 * between rows included) with two workgroups per compute unit in
 * grid-stride order.  sink is a device pointer to one uint32 that is written
 * only if the folded data happens to equal a fixed constant (it keeps the
 * loads live).  Asynchronous.  Returns XPRESS_OK, XPRESS_EINVAL or
 * XPRESS_EHIP.
 */
#define XPRESS_READ_ROWS 0
#define XPRESS_READ_FLAT 1
int xpress_read_probe(const uint16_t* base, const uint16_t* bias, int64_t rows, int64_t V,
                      int64_t stride, int mode, uint32_t* sink, hipStream_t stream);

/* The HIP error code of the last failing HIP call on this thread. */
int xpress_last_hip_error(void);

/* A static, human-readable description of a status code. */
const char* xpress_error_string(int status);

/* Library version, "major.minor.patch". */
const char* xpress_version(void);

#ifdef __cplusplus
}
#endif

#endif /* XPRESS_ARGMAX_H */
