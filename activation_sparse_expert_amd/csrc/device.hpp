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

// Strides 32 and 16 exchange whole halves (rows) of the wave: gfx950's
// v_permlane32_swap / v_permlane16_swap move lane l's `hi` to its partner
// and bring the partner's `lo` back, so one swap and one add replace two
// selects and a cross-lane LDS permute.  Lanes with bit S clear get
// lo(own) + lo(partner), the others hi(partner) + hi(own): the same sums as
// the permute form (addition commutes exactly).
template <int S>
__device__ __forceinline__ float swap_add(float lo, float hi)
{
    static_assert(S == 32 || S == 16, "row swaps");
    const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    if constexpr (S == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// The value of lane l ^ S for S < 16: a DPP quad permute for 1 and 2, an
// LDS swizzle in xor mode (no address register) for 4 and 8.
template <int S>
__device__ __forceinline__ float xor_lane(float x)
{
    const int xi = __float_as_int(x);
    if constexpr (S == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false));
    else if constexpr (S == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false));
    else return __int_as_float(__builtin_amdgcn_ds_swizzle(xi, (S << 10) | 0x1F));
}

// v + the value of lane l ^ S (every lane gets the pair's sum)
template <int S>
__device__ __forceinline__ float bfly_add(float v)
{
    if constexpr (S >= 16) return swap_add<S>(v, v);
    else return v + xor_lane<S>(v);
}

// Sum over aligned groups of SEG lanes (SEG a power of two <= 64); every lane
// of the group receives the total.  Fixed butterfly order: bit-reproducible.
template <int SEG, int S = SEG / 2>
__device__ __forceinline__ float seg_sum(float v)
{
    if constexpr (S == 0) return v;
    else return seg_sum<SEG, S / 2>(bfly_add<S>(v));
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
// restored.  NT: the nontemporal (streaming) cache policy, for data read once.
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds_base)
{
    typedef __attribute__((address_space(3))) void lvoid;
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lvoid *)lds_base);
    uint32_t saved;
    if constexpr (NT)
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                     "global_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(src), "s"(m)
                     : "memory");
    else
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
