// Device-side helpers shared by the libmoeffn kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeffn {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Packed 16-bit pair dot product with fp32 accumulation: a.lo*b.lo + a.hi*b.hi + c.
// Products of two 16-bit values are exact in fp32.
template <bool BF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a),
                                      __builtin_bit_cast(half2_t, b), c, false);
    }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b)
{
    return __builtin_bit_cast(float, b << 16);
}

template <bool BF16>
__device__ __forceinline__ float lo16_to_float(uint32_t w)
{
    if constexpr (BF16) return __builtin_bit_cast(float, w << 16);
    else return half_bits_to_float(w & 0xFFFFu);
}

template <bool BF16>
__device__ __forceinline__ float hi16_to_float(uint32_t w)
{
    if constexpr (BF16) return __builtin_bit_cast(float, w & 0xFFFF0000u);
    else return half_bits_to_float(w >> 16);
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32: round to nearest even
}

__device__ __forceinline__ uint16_t float_to_bf16_bits(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);                      // round to nearest even (finite inputs)
    return (uint16_t)(u >> 16);
}

// Sum over aligned groups of SEG lanes (SEG a power of two <= 64); every lane
// of the group receives the total.  Fixed butterfly order: bit-reproducible.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v)
{
#pragma unroll
    for (int off = SEG / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float silu(float g)
{
    return g / (1.0f + __expf(-g));
}

// Coherent (device-scope) scalar access used for the cross-workgroup
// accumulator and completion counters.
__device__ __forceinline__ float load_coherent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int load_coherent_i32(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Streaming loads for data read once (weights, partial rows): the nontemporal
// hint keeps the line out of the compute unit's vector cache, which on gfx950
// roughly doubles the bandwidth a single compute unit can draw (one workgroup
// streaming alone: about 78 GB/s against 38 GB/s with ordinary loads).
__device__ __forceinline__ uint4 load_nt16(const void *p)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load((const v4u *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_nt4(const void *p)
{
    return __builtin_nontemporal_load((const uint32_t *)p);
}

__device__ __forceinline__ float4 load_nt16f(const float *p)
{
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f v = __builtin_nontemporal_load((const v4f *)p);
    return make_float4(v.x, v.y, v.z, v.w);
}

// Asynchronous 16-byte copy global -> LDS (gfx950 global_load_lds_dwordx4):
// lane l of the wave writes its 16 bytes to lds_base + 16 l; lds_base must be
// the same for every lane.  Issued from inline assembly so that the compiler's
// wait-count pass does not treat the copy as a possible alias of every later
// LDS access (it would drain vmcnt before each): the issuing wave waits for its
// copies itself (vmcnt) before a barrier that publishes them.  m0 is saved and
// restored.
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds_base)
{
    typedef __attribute__((address_space(3))) void lvoid;
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lvoid *)lds_base);
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(m)
                 : "memory");
}

// Store one fp32 result into an output of type dt (0 f16, 1 bf16, 2 f32),
// optionally adding to what is there.
__device__ __forceinline__ void store_out(void *y, int dt, size_t i, float v, int accumulate)
{
    if (dt == 2) {
        float *p = (float *)y + i;
        *p = accumulate ? *p + v : v;
    } else if (dt == 1) {
        uint16_t *p = (uint16_t *)y + i;
        if (accumulate) v += bf16_bits_to_float(*p);
        *p = float_to_bf16_bits(v);
    } else {
        uint16_t *p = (uint16_t *)y + i;
        if (accumulate) v += half_bits_to_float(*p);
        *p = float_to_half_bits(v);
    }
}

}  // namespace moeffn
