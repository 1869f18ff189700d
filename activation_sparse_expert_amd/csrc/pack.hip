// INT2 group-64 packing of the up projection (FloE review, "混合压缩策略": up is
// the projection least sensitive to very low bit widths and is stored in INT2),
// the bf16 materialisation of those weights for the dense path, and a
// workspace fill kernel.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

__device__ __forceinline__ float load_w(const void *p, int dt, size_t i)
{
    if (dt == 2) return ((const float *)p)[i];
    const uint16_t b = ((const uint16_t *)p)[i];
    return dt == 1 ? bf16_bits_to_float(b) : half_bits_to_float(b);
}

// One thread per (channel, group of 64 inputs).  All steps are single fp32
// operations with round-to-nearest-even, in this order:
//   mn, mx;  s = fp16((mx - mn) / 3) (1 if 0);  z = fp16(-mn / s);
//   q = clamp(rint(w / s + z), 0, 3)
// Output word i of the row holds inputs 16i..16i+15: input 16i + 2m + h at
// bits 16h + 2m.
__global__ void __launch_bounds__(256)
pack_int2_kernel(const void *w, int dt, int d, int f, uint8_t *q, uint16_t *sz)
{
    const int G = d / 64;
    const size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= (size_t)f * G) return;
    const size_t j = u / G, g = u - j * G;
    const size_t base = j * d + g * 64;
    float mn = load_w(w, dt, base), mx = mn;
    for (int i = 1; i < 64; ++i) {
        const float v = load_w(w, dt, base + i);
        if (v < mn) mn = v;             // plain comparisons: a signed zero never replaces
        if (v > mx) mx = v;             // an equal earlier value
    }
    const float third = __fdiv_rn(mx - mn, 3.0f);
    uint16_t sb = float_to_half_bits(third);
    float s = half_bits_to_float(sb);
    if (s == 0.0f) { sb = 0x3C00; s = 1.0f; }
    const uint16_t zb = float_to_half_bits(__fdiv_rn(-mn, s));
    const float z = half_bits_to_float(zb);
    sz[u * 2 + 0] = sb;
    sz[u * 2 + 1] = zb;
    uint32_t words[4] = {0, 0, 0, 0};
    for (int i = 0; i < 64; ++i) {
        const float a = __fdiv_rn(load_w(w, dt, base + i), s);
        const float r = rintf(__fadd_rn(a, z));
        int c = (int)r;
        if (r < 0.0f) c = 0;
        if (r > 3.0f) c = 3;
        const int wi = i / 16, h = i & 1, m = (i & 15) >> 1;
        words[wi] |= (uint32_t)c << (16 * h + 2 * m);
    }
    *(uint4 *)(q + j * (d / 4) + g * 16) = make_uint4(words[0], words[1], words[2], words[3]);
}

// The same quantiser with L = 2^BITS - 1 levels (8, 4 or 1 bits): the codes
// of a group are packed plainly, input k at bit k*BITS of the row, least
// significant bits first; a group takes 8*BITS bytes.
template <int BITS>
__global__ void __launch_bounds__(256)
pack_bits_kernel(const void *w, int dt, int d, int f, uint8_t *q, uint16_t *sz)
{
    constexpr int L = (1 << BITS) - 1;
    constexpr int NW = 2 * BITS;                // 32-bit words per group
    const int G = d / 64;
    const size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= (size_t)f * G) return;
    const size_t j = u / G, g = u - j * G;
    const size_t base = j * d + g * 64;
    float mn = load_w(w, dt, base), mx = mn;
    for (int i = 1; i < 64; ++i) {
        const float v = load_w(w, dt, base + i);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    uint16_t sb = float_to_half_bits(__fdiv_rn(mx - mn, (float)L));
    float s = half_bits_to_float(sb);
    if (s == 0.0f) { sb = 0x3C00; s = 1.0f; }
    const uint16_t zb = float_to_half_bits(__fdiv_rn(-mn, s));
    const float z = half_bits_to_float(zb);
    sz[u * 2 + 0] = sb;
    sz[u * 2 + 1] = zb;
    uint32_t words[NW];
    for (int i = 0; i < NW; ++i) words[i] = 0;
    for (int i = 0; i < 64; ++i) {
        const float a = __fdiv_rn(load_w(w, dt, base + i), s);
        const float r = rintf(__fadd_rn(a, z));
        int c = (int)r;
        if (r < 0.0f) c = 0;
        if (r > (float)L) c = L;
        const int bit = i * BITS;
        words[bit / 32] |= (uint32_t)c << (bit % 32);
    }
    uint32_t *dst = (uint32_t *)(q + j * ((size_t)d * BITS / 8) + g * 8 * BITS);
    for (int i = 0; i < NW; ++i) dst[i] = words[i];
}

// Round a double to bfloat16, nearest-even, from its bits (finite inputs).
__device__ __forceinline__ uint16_t double_to_bf16_bits(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t sign = u >> 63;
    uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
    if (mag == 0) return (uint16_t)(sign << 15);
    // rebias exponent from double (1023) to float (127) and keep 7 mantissa bits
    int e = (int)(mag >> 52) - 1023 + 127;
    uint64_t m = (mag & 0xFFFFFFFFFFFFFull) | (1ull << 52);   // 53-bit significand
    int drop;                                                   // bits to drop to keep 8
    if (e >= 1) {
        drop = 52 - 7;
    } else {                                                   // subnormal bf16
        drop = 52 - 7 + (1 - e);
        e = 0;
        if (drop > 60) return (uint16_t)(sign << 15);
    }
    uint64_t keep = m >> drop;
    const uint64_t rem = m & ((1ull << drop) - 1);
    const uint64_t half = 1ull << (drop - 1);
    if (rem > half || (rem == half && (keep & 1))) keep++;
    uint32_t bits;
    if (e == 0) {
        bits = (uint32_t)keep;                                  // may carry into exponent 1
    } else {
        if (keep >> 8) { keep >>= 1; e++; }                     // carry out of the significand
        if (e >= 255) return (uint16_t)((sign << 15) | 0x7F80);
        bits = ((uint32_t)e << 7) | (uint32_t)(keep & 0x7F);
    }
    return (uint16_t)((sign << 15) | bits);
}

// Dense-path up weights: out = s (q - z) from the INT2 format, rounded once to
// bf16 (BF16) or fp16.  The product is exact in double (and in fp32: q - z has
// at most 13 significant bits and s 11); fp16 rounding is v_cvt_f16_f32's
// round to nearest even of that exact fp32 value.
template <bool BF16>
__global__ void __launch_bounds__(256)
materialize_kernel(const uint8_t *q, const uint16_t *sz, int d, int f, uint16_t *out)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)f * d) return;
    const size_t j = i / d, k = i - j * d;
    const int G = d / 64;
    const size_t bit = 32 * (k / 16) + 16 * (k & 1) + 2 * ((k & 15) >> 1);
    const int c = (q[j * (d / 4) + bit / 8] >> (bit % 8)) & 3;
    const double s = (double)half_bits_to_float(sz[(j * G + k / 64) * 2 + 0]);
    const double z = (double)half_bits_to_float(sz[(j * G + k / 64) * 2 + 1]);
    if constexpr (BF16) out[i] = double_to_bf16_bits(s * ((double)c - z));
    else out[i] = float_to_half_bits((float)(s * ((double)c - z)));
}

__global__ void __launch_bounds__(256)
fill_zero_kernel(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void __launch_bounds__(256)
fill_u8_kernel(uint8_t *p, size_t n, uint8_t v)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

hipError_t launch_pack_int2(const void *w, int dt, int d, int f, uint8_t *q, uint16_t *sz,
                            hipStream_t s)
{
    const size_t n = (size_t)f * (d / 64);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(pack_int2_kernel, dim3(blocks), dim3(256), 0, s, w, dt, d, f, q, sz);
    return hipGetLastError();
}

hipError_t launch_pack_bits(const void *w, int dt, int d, int f, int bits, uint8_t *q,
                            uint16_t *sz, hipStream_t s)
{
    const size_t n = (size_t)f * (d / 64);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bits == 8) hipLaunchKernelGGL(pack_bits_kernel<8>, dim3(blocks), dim3(256), 0, s, w, dt, d, f, q, sz);
    else if (bits == 4) hipLaunchKernelGGL(pack_bits_kernel<4>, dim3(blocks), dim3(256), 0, s, w, dt, d, f, q, sz);
    else if (bits == 1) hipLaunchKernelGGL(pack_bits_kernel<1>, dim3(blocks), dim3(256), 0, s, w, dt, d, f, q, sz);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_materialize16(const uint8_t *q, const uint16_t *sz, int d, int f, bool bf16,
                                uint16_t *out, hipStream_t s)
{
    const size_t n = (size_t)f * d;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL(materialize_kernel<true>, dim3(blocks), dim3(256), 0, s, q, sz, d, f, out);
    else
        hipLaunchKernelGGL(materialize_kernel<false>, dim3(blocks), dim3(256), 0, s, q, sz, d, f, out);
    return hipGetLastError();
}

namespace {

// Bit form of 0/1 channel masks (FloE review, "高效稀疏 GEMV 内核": the mask of
// Algorithm 1 as a bitmask, and its population count).  One workgroup per row
// of f channels: wave w packs the 64-channel words w, w + 4, ... by a ballot
// (channel 64 i + l at bit l of word i) and counts them; the four wave counts
// are added in LDS.  Integer work, no atomics.
constexpr int kPackThreads = 256;

__global__ void __launch_bounds__(kPackThreads)
mask_bits_kernel(const uint8_t *m, int f, uint64_t *bits, int32_t *nnz)
{
    __shared__ int cnt[kPackThreads / 64];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int words = f / 64;
    const uint8_t *src = m + (size_t)row * f;
    int n = 0;
    for (int wi = wave; wi < words; wi += kPackThreads / 64) {
        const uint64_t b = __ballot(src[(size_t)wi * 64 + lane] != 0);
        if (bits && lane == 0) bits[(size_t)row * words + wi] = b;
        n += __popcll(b);
    }
    if (lane == 0) cnt[wave] = n;
    __syncthreads();
    if (threadIdx.x == 0 && nnz) {
        int t = 0;
        for (int w = 0; w < kPackThreads / 64; ++w) t += cnt[w];
        nnz[row] = t;
    }
}

}  // namespace

hipError_t launch_mask_bits(const uint8_t *m, int rows, int f, uint64_t *bits, int32_t *nnz,
                            hipStream_t s)
{
    if (rows < 1 || f % 64 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mask_bits_kernel, dim3(rows), dim3(kPackThreads), 0, s, m, f, bits, nnz);
    return hipGetLastError();
}

hipError_t launch_fill_u8(uint8_t *p, size_t n, uint8_t v, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_u8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s)
{
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, n);
    return hipGetLastError();
}

}  // namespace moeffn
