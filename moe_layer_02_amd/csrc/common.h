// common.h -- device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// bf16 x8 -> fp16 x8 (round to nearest even), reordered (0,4,1,5,2,6,3,7): the order in
// which the int4 kernels dequantise 8 packed nibbles.
__device__ __forceinline__ uint4 bf16x8_to_f16x8_perm(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    _Float16 h[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        h[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
        h[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xFFFF0000u);
    }
    const _Float16 p[8] = {h[0], h[4], h[1], h[5], h[2], h[6], h[3], h[7]};
    uint4 r;
    r.x = (uint32_t)__builtin_bit_cast(uint16_t, p[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, p[1]) << 16);
    r.y = (uint32_t)__builtin_bit_cast(uint16_t, p[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, p[3]) << 16);
    r.z = (uint32_t)__builtin_bit_cast(uint16_t, p[4]) | ((uint32_t)__builtin_bit_cast(uint16_t, p[5]) << 16);
    r.w = (uint32_t)__builtin_bit_cast(uint16_t, p[6]) | ((uint32_t)__builtin_bit_cast(uint16_t, p[7]) << 16);
    return r;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

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
