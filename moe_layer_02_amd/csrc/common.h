// common.h -- device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// 8 bf16 values reordered (0,4,1,5,2,6,3,7): the order in which the int4 kernels unpack
// the 8 nibbles of a 32-bit word (nibbles i and i + 4 land in the two halves of one packed
// pair).  A pure permutation of 16-bit values.
__device__ __forceinline__ uint4 bf16x8_perm(uint4 v) {
    uint4 r;
    r.x = (v.x & 0xFFFFu) | (v.z << 16);             // elements 0, 4
    r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);         // 1, 5
    r.z = (v.y & 0xFFFFu) | (v.w << 16);             // 2, 6
    r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);         // 3, 7
    return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// SiLU(g) = g sigmoid(g) in fp32 for the gate/up epilogues: the hardware exp and reciprocal
// (each within about an ulp) in place of a correctly rounded division, which costs about ten
// dependent instructions per value where this takes two.  The result is within a few ulps of
// the exact value, far inside what the product's later rounding (h to bf16, or the fp8
// codes decided from this h) and the tolerance allow.  Large negative g: the reciprocal of
// +inf is 0 and the result -0, as the division gives; large positive g: g.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// A maximum of non-negative floats kept as their bits (which order like the floats) in one
// device word.  Atomics on one address serialise (about 16 ns each on these GPUs), so a
// caller reads the word first (amax_peek, a device-scope load that may be issued early)
// and raises it only when its value is larger: the word only grows, so a value that is
// not larger than a read can never be the maximum.
__device__ __forceinline__ uint32_t amax_peek(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void amax_raise(uint32_t *p, uint32_t seen, float v) {
    if (__float_as_uint(v) > seen) atomicMax(p, __float_as_uint(v));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
