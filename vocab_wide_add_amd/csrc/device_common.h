// device_common.h -- device helpers shared by the readout kernels of
// libxpress_argmax (gfx950, wave64): the element step bf16(a + b), the
// (value, index) order and its wave / workgroup reductions, and the packed
// order-preserving keys used to combine partial results.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace xpress {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kNoIndex = 0xFFFFFFFFu;  // "no candidate" (loses every tie)

// ---------------------------------------------------------------------------
// Element step.
// ---------------------------------------------------------------------------

// The low / high bf16 of a packed pair, widened to fp32 (exact: bf16 is the
// upper half of binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two element sums at once: a and b each pack two bf16; returns the two sums
// rounded to bf16 (round-to-nearest-even), packed the same way.  The fp32 sum
// of two bf16 values rounded to bf16 equals the exact sum rounded once to
// bf16, since fp32 carries 24 >= 2*8 + 2 significant bits.
__device__ __forceinline__ uint32_t add_round2(uint32_t a, uint32_t b)
{
    f32x2 s;
    s.x = bf16_lo(a) + bf16_lo(b);
    s.y = bf16_hi(a) + bf16_hi(b);
    bf16x2 r = __builtin_convertvector(s, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Scalar form for the unaligned path and the vocabulary tail.
__device__ __forceinline__ float add_round1(uint16_t a, uint16_t b)
{
    uint32_t p = add_round2((uint32_t)a, (uint32_t)b);
    return bf16_lo(p);
}

// ---------------------------------------------------------------------------
// (value, index) order: larger value first, then smaller index.  Float
// comparison makes -0 equal to +0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge(float& v, uint32_t& i, float ov, uint32_t oi)
{
    const bool take = (ov > v) | ((ov == v) & (oi < i));
    v = take ? ov : v;
    i = take ? oi : i;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void merge_dpp(float& v, uint32_t& i)
{
    float ov = __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
    uint32_t oi = dpp_u32<CTRL>(i);
    merge(v, i, ov, oi);
}

// Reduce over the 64 lanes of the wave; the result is wave-uniform.
__device__ __forceinline__ void wave_argmax(float& v, uint32_t& i)
{
    merge_dpp<0xB1>(v, i);   // quad_perm [1,0,3,2]: partner lane ^ 1
    merge_dpp<0x4E>(v, i);   // quad_perm [2,3,0,1]: partner lane ^ 2
    merge_dpp<0x141>(v, i);  // row_half_mirror: the other quad of each 8
    merge_dpp<0x140>(v, i);  // row_mirror: the other 8 of each 16
    // ds_swizzle bit mode, and_mask 0x1F, xor_mask 0x10: partner lane ^ 16
    float ov = __uint_as_float((uint32_t)__builtin_amdgcn_ds_swizzle(
        (int)__float_as_uint(v), 0x401F));
    uint32_t oi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)i, 0x401F);
    merge(v, i, ov, oi);
    // lanes 0..31 and 32..63 now each hold their half's result
    float v0 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
    uint32_t i0 = (uint32_t)__builtin_amdgcn_readlane((int)i, 0);
    float v1 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 32));
    uint32_t i1 = (uint32_t)__builtin_amdgcn_readlane((int)i, 32);
    merge(v0, i0, v1, i1);
    v = v0;
    i = i0;
}

// Workgroup reduction; every thread returns the workgroup's result.
template <int T>
__device__ __forceinline__ void block_argmax(float& v, uint32_t& i)
{
    constexpr int kWaves = T / 64;
    wave_argmax(v, i);
    if constexpr (kWaves > 1) {
        __shared__ float sv[kWaves];
        __shared__ uint32_t si[kWaves];
        const int wave = threadIdx.x / 64;
        if ((threadIdx.x & 63) == 0) {
            sv[wave] = v;
            si[wave] = i;
        }
        __syncthreads();
        float bv = sv[0];
        uint32_t bi = si[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            merge(bv, bi, sv[w], si[w]);
        }
        v = bv;
        i = bi;
        __syncthreads();  // sv/si may be reused by the next unit of work
    }
}

// Packed order-preserving 48-bit key: (ordered bf16 of the value) << 32 |
// ~index.  Unsigned order of keys == (value desc, index asc) order of
// candidates.  -0 is mapped to +0 first so the two compare equal.  A missing
// candidate is the key 0, below every real key (real keys have ~index >=
// 2^31).
__device__ __forceinline__ uint64_t make_key(float v, uint32_t i)
{
    if (i == kNoIndex) {
        return 0;
    }
    uint32_t h = __float_as_uint(v) >> 16;  // v is a widened bf16
    if (h == 0x8000u) {
        h = 0;
    }
    uint32_t ord = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
    return ((uint64_t)ord << 32) | (uint64_t)(kNoIndex - i);
}

__device__ __forceinline__ int64_t key_index(uint64_t key)
{
    return (int64_t)(kNoIndex - (uint32_t)(key & 0xFFFFFFFFu));
}

// ---------------------------------------------------------------------------
// Load-to-LDS and explicit wait counts, for kernels that stream operands into
// LDS with several loads in flight.
// ---------------------------------------------------------------------------

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte load-to-LDS: lane l's 16 bytes from gsrc land at LDS byte
// address lds_base + 16 l (lds_base wave-uniform, carried in M0).  Issued as
// the instructions the compiler itself emits for this load, so that its
// wait-count pass does not add a wait for every pending load before each LDS
// read; the contraction loop waits for exactly the chunk it is about to read
// (wait_vmcnt), and extra loads the compiler places after these only make
// its own waits stricter.
__device__ __forceinline__ void dma16(const uint16_t* gsrc, uint32_t lds_base)
{
    // M0 is read when the load issues; it is restored right after so that no
    // other use of M0 sees the LDS address
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gsrc), "s"(lds_base)
        : "memory");
}

// LDS byte address of a __shared__ element, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p)
{
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
    return __builtin_amdgcn_readfirstlane(a);
}

}  // namespace xpress
