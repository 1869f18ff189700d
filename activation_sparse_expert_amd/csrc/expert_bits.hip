// The sparse expert with the up projection at 8, 4 or 1 bits per code (FloE
// review, "敏感度分析": the up projection is also quantised to INT8, INT4 and
// INT1; the expert itself is Algorithm 1 of "高效稀疏 GEMV 内核").  The codes
// use the same group-64 scale and zero point as the INT2 format, packed plainly:
// input k of channel j at bit k*bits of row j.
//
// Two kernels and the shared reduce:
//  * upb_kernel: v = x W^up and the mask |v| > t.  The tokens' x is staged in
//    LDS as fp32, input 16 c + u at row u, column c, with per-16-input sums
//    (one token: each lane reads its own chunks into registers instead, as it
//    always takes the same ones, and no LDS is used); every wave streams 8
//    rows of codes (4 below 8 bits for one token), the loads of the rows up to
//    3 ahead in flight while one is computed, a lane taking 16 codes
//    (2*bits bytes) per step and adding s (sum q x - z sum x) per 16-code
//    chunk.  v goes to memory.
//  * gatherb_kernel: one workgroup per 64 channels.  For each token the
//    active channels of the tile are ranked (ballots in channel order) and
//    shared out by rank over the 4 waves; a wave loads its channel's gate and
//    down rows together (the next channel's while one is computed), forms the
//    gate dot product, h = SiLU(g) v (times the token scale), and adds h times
//    the down row into per-lane column sums.  The waves' sums are added in LDS in
//    wave order and written as the tile's partial row; the reduce kernel adds
//    the tiles in a fixed order.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

constexpr int kUThreads = 256;
// rows per wave: 8 at 8 bits or with several tokens (each workgroup stages
// their x), 4 for one token below 8 bits (measured on the Mixtral shape)
template <int BITS, bool ONE>
__host__ __device__ constexpr int urows() { return BITS == 8 || !ONE ? 8 : 4; }
constexpr int kUMaxSteps = 4;           // 16-code chunks per lane per row: d <= 4096
constexpr int kGThreads = 256;
constexpr int kUAhead = 3;              // rows of codes in flight ahead of the one computed

template <int BITS>
struct Chunk;                           // 16 codes of one lane
template <> struct Chunk<8> {
    uint4 w;
    __device__ void load(const uint8_t *p) { w = load_nt16(p); }
    __device__ int code(int u) const
    {
        const uint32_t x = u < 4 ? w.x : u < 8 ? w.y : u < 12 ? w.z : w.w;
        return (x >> (8 * (u & 3))) & 0xFF;
    }
};
template <> struct Chunk<4> {
    uint2 w;
    __device__ void load(const uint8_t *p)
    {
        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
        const v2u v = __builtin_nontemporal_load((const v2u *)p);
        w = make_uint2(v.x, v.y);
    }
    __device__ int code(int u) const
    {
        const uint32_t x = u < 8 ? w.x : w.y;
        return (x >> (4 * (u & 7))) & 0xF;
    }
};
template <> struct Chunk<1> {
    uint32_t w;
    __device__ void load(const uint8_t *p) { w = __builtin_nontemporal_load((const uint16_t *)p); }
    __device__ int code(int u) const { return (w >> u) & 1; }
};

// ONE: a single token, whose x chunks stay in the lane's registers (the
// lane always takes the same chunks); otherwise they are read from LDS per row
template <int BITS, bool BF16, bool ONE>
__global__ void __launch_bounds__(kUThreads)
upb_kernel(BitsArgs a)
{
    // several tokens: x staged as xs[t][u][c] = x[t][16 c + u] (fp32), so that
    // consecutive lanes (consecutive chunks c) read consecutive words, then
    // the chunk sums xc[t][c]; one token needs no staging: each lane reads its
    // own chunks below
    extern __shared__ __align__(16) float xs[];
    const int d = a.d, T = a.T, nchunk = d / 16;
    float *xc = xs + (size_t)T * d;
    for (int i = threadIdx.x; !ONE && i < T * d / 8; i += kUThreads) {
        // 8 inputs per 16-byte load (d % 512 == 0, x 16-byte aligned)
        const uint4 w = *(const uint4 *)(a.x + 8 * (size_t)i);
        const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
        const int t = (8 * i) / d, k0 = 8 * i - t * d;
        const int c = k0 / 16, u0 = k0 % 16;
        float *o = xs + (size_t)t * d + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[(size_t)(u0 + 2 * q) * nchunk] = lo16_to_float<BF16>(w4[q]);
            o[(size_t)(u0 + 2 * q + 1) * nchunk] = hi16_to_float<BF16>(w4[q]);
        }
    }
    if constexpr (!ONE) {
        __syncthreads();
        for (int i = threadIdx.x; i < T * nchunk; i += kUThreads) {
            const int t = i / nchunk, c = i - t * nchunk;
            const float *p = xs + (size_t)t * d + c;
            float s = 0.f;
            for (int u = 0; u < 16; ++u) s += p[(size_t)u * nchunk];
            xc[i] = s;
        }
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = d / 64;
    const size_t row_bytes = (size_t)d * BITS / 8;
    float xreg[ONE ? kUMaxSteps : 1][16], xcr[ONE ? kUMaxSteps : 1];
    if constexpr (ONE) {
        // the lane's chunks straight from x (two 16-byte loads each), their
        // sums in the same order as the staged form
#pragma unroll
        for (int st = 0; st < kUMaxSteps; ++st) {
            const int c = lane + 64 * st;
            uint32_t w8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (c < nchunk) {
                const uint4 p0 = *(const uint4 *)(a.x + (size_t)c * 16);
                const uint4 p1 = *(const uint4 *)(a.x + (size_t)c * 16 + 8);
                w8[0] = p0.x; w8[1] = p0.y; w8[2] = p0.z; w8[3] = p0.w;
                w8[4] = p1.x; w8[5] = p1.y; w8[6] = p1.z; w8[7] = p1.w;
            }
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                xreg[st][2 * u] = lo16_to_float<BF16>(w8[u]);
                xreg[st][2 * u + 1] = hi16_to_float<BF16>(w8[u]);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) sum += xreg[st][u];
            xcr[st] = sum;
        }
    }
    constexpr int kURows = urows<BITS, ONE>();
    const int j0 = (blockIdx.x * (kUThreads / 64) + wave) * kURows;
    // f % 64 == 0 and a workgroup takes 16 or 32 rows: all of a wave's rows
    // exist once its first does (no barrier follows)
    if (j0 >= a.f) return;
    // the row loop is unrolled; row r + kUAhead's codes are loaded while row r
    // is computed (the buffers of a row live from its load to its use)
    Chunk<BITS> ch[kURows][kUMaxSteps];
    uint32_t sz[kURows][kUMaxSteps];
    auto load_row = [&](int r) {
#pragma unroll
        for (int st = 0; st < kUMaxSteps; ++st) {
            const int c = lane + 64 * st;
            if (c < nchunk) {
                ch[r][st].load(a.up_q + (size_t)(j0 + r) * row_bytes + (size_t)c * 2 * BITS);
                sz[r][st] = load_nt4(a.up_sz + ((size_t)(j0 + r) * G + c / 4) * 2);
            }
        }
    };
#pragma unroll
    for (int r = 0; r < kUAhead && r < kURows; ++r) load_row(r);
#pragma unroll
    for (int r = 0; r < kURows; ++r) {
        const int j = j0 + r;
        if (r + kUAhead < kURows) load_row(r + kUAhead);
        for (int t = 0; t < T; ++t) {
            float acc = 0.f;
#pragma unroll
            for (int st = 0; st < kUMaxSteps; ++st) {
                const int c = lane + 64 * st;
                if (c < nchunk) {
                    const float *xp = xs + (size_t)t * d + c;
                    float dq = 0.f;
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        dq += (float)ch[r][st].code(u) *
                              (ONE ? xreg[ONE ? st : 0][u] : xp[(size_t)u * nchunk]);
                    const float s = half_bits_to_float(sz[r][st] & 0xFFFFu);
                    const float z = half_bits_to_float(sz[r][st] >> 16);
                    acc += s * (dq - z * (ONE ? xcr[ONE ? st : 0] : xc[t * nchunk + c]));
                }
            }
            acc = seg_sum<64>(acc);
            if (lane == 0) {
                a.v[(size_t)t * a.f + j] = acc;
                if (a.mask_out) a.mask_out[(size_t)t * a.f + j] = fabsf(acc) > a.thr ? 1 : 0;
            }
        }
    }
}

// NC = d / 512: lane l owns columns 8 l + 512 i, i < NC
template <bool BF16, int NC>
__global__ void __launch_bounds__(kGThreads)
gatherb_kernel(BitsArgs a)
{
    extern __shared__ __align__(16) float red[];     // [d]
    const int d = a.d;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int tile = blockIdx.x;
    const int jt = tile * kBitsTile;
    for (int t = 0; t < a.T; ++t) {
        uint4 xr[NC];
#pragma unroll
        for (int i = 0; i < NC; ++i) xr[i] = *(const uint4 *)(a.x + (size_t)t * d + 8 * lane + 512 * i);
        float acc[NC][8];
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[i][u] = 0.f;
        const float sc = a.token_scale ? a.token_scale[t] : 1.f;
        static_assert(kBitsTile == 64, "one ballot per tile");
        const int jl = jt + lane;
        const bool act = jl < a.f && fabsf(a.v[(size_t)t * a.f + jl]) > a.thr;
        unsigned long long m = __ballot(act);
        // this wave's channels: the active ones whose rank in channel order is
        // the wave's index mod 4, taken in channel order
        unsigned long long mine = 0;
        for (int rank = 0; m; ++rank) {
            if ((rank & 3) == wave) mine |= m & (~m + 1);
            m &= m - 1;
        }
        auto load_ch = [&](int j, uint4 (&g_)[NC], uint4 (&d_)[NC]) {
            const uint16_t *grow = a.gate + (size_t)j * d;
            const uint16_t *drow = a.down + (size_t)j * d;
#pragma unroll
            for (int i = 0; i < NC; ++i) g_[i] = load_nt16(grow + 8 * lane + 512 * i);
#pragma unroll
            for (int i = 0; i < NC; ++i) d_[i] = load_nt16(drow + 8 * lane + 512 * i);
        };
        // the next channel's rows are loaded while one is computed
        uint4 gw[NC], dw[NC];
        int jc = -1;
        if (mine) {
            jc = jt + __builtin_ctzll(mine);
            mine &= mine - 1;
            load_ch(jc, gw, dw);
        }
        while (jc >= 0) {
            int jn = -1;
            uint4 gn[NC], dn[NC];
            if (mine) {
                jn = jt + __builtin_ctzll(mine);
                mine &= mine - 1;
                load_ch(jn, gn, dn);
            }
            const float vj = a.v[(size_t)t * a.f + jc];
            float g = 0.f;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                g = dot2<BF16>(gw[i].x, xr[i].x, g);
                g = dot2<BF16>(gw[i].y, xr[i].y, g);
                g = dot2<BF16>(gw[i].z, xr[i].z, g);
                g = dot2<BF16>(gw[i].w, xr[i].w, g);
            }
            g = seg_sum<64>(g);
            const float h = silu(g) * vj * sc;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const uint32_t w4[4] = {dw[i].x, dw[i].y, dw[i].z, dw[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[i][2 * q] += h * lo16_to_float<BF16>(w4[q]);
                    acc[i][2 * q + 1] += h * hi16_to_float<BF16>(w4[q]);
                }
            }
            if (jn >= 0) {
#pragma unroll
                for (int i = 0; i < NC; ++i) { gw[i] = gn[i]; dw[i] = dn[i]; }
            }
            jc = jn;
        }
        // the waves' column sums, added in wave order
        for (int w = 0; w < kGThreads / 64; ++w) {
            if (wave == w) {
#pragma unroll
                for (int i = 0; i < NC; ++i)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        float *p = red + 8 * lane + 512 * i + u;
                        *p = w == 0 ? acc[i][u] : *p + acc[i][u];
                    }
            }
            __syncthreads();
        }
        float *dst = a.part + ((size_t)t * a.tiles + tile) * d;
        for (int c = threadIdx.x * 4; c < d; c += kGThreads * 4) {
            const float4 v4 = *(const float4 *)(red + c);
            typedef float v4f __attribute__((ext_vector_type(4)));
            v4f o = {v4.x, v4.y, v4.z, v4.w};
            __builtin_nontemporal_store(o, (v4f *)(dst + c));
        }
        __syncthreads();                               // red is reused by the next token
    }
}

template <int BITS>
const void *upb_for(bool bf16, bool one)
{
    if (one) return bf16 ? (const void *)upb_kernel<BITS, true, true>
                         : (const void *)upb_kernel<BITS, false, true>;
    return bf16 ? (const void *)upb_kernel<BITS, true, false> : (const void *)upb_kernel<BITS, false, false>;
}

template <int NC>
const void *gatherb_for(bool bf16)
{
    return bf16 ? (const void *)gatherb_kernel<true, NC> : (const void *)gatherb_kernel<false, NC>;
}

}  // namespace

size_t bits_lds_up(int T, int d) { return (size_t)T * d * 4 + (size_t)T * (d / 16) * 4; }

hipError_t launch_expert_bits(const BitsArgs &a, hipStream_t s)
{
    const bool one = a.T == 1;
    const void *up = a.bits == 8 ? upb_for<8>(a.bf16, one) : a.bits == 4 ? upb_for<4>(a.bf16, one)
                   : a.bits == 1 ? upb_for<1>(a.bf16, one) : nullptr;
    const int nc = a.d / 512;
    const void *ga = nc == 1 ? gatherb_for<1>(a.bf16) : nc == 2 ? gatherb_for<2>(a.bf16)
                   : nc == 4 ? gatherb_for<4>(a.bf16) : nc == 8 ? gatherb_for<8>(a.bf16) : nullptr;
    if (!up || !ga || a.d % 512 != 0 || a.d / 16 > 64 * kUMaxSteps) return hipErrorInvalidValue;
    const size_t lds_up = one ? 0 : bits_lds_up(a.T, a.d);
    if (lds_up > kBitsMaxLds) return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    if (lds_up > 0) {
        e = hipFuncSetAttribute(up, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_up);
        if (e != hipSuccess) return e;
    }
    const int urows_run = !one ? urows<8, false>() : a.bits == 8 ? urows<8, true>() : urows<4, true>();
    const int rows_per_block = (kUThreads / 64) * urows_run;   // urows<1, .> equals urows<4, .>
    void *args[] = {(void *)&a};
    e = hipLaunchKernel(up, dim3((a.f + rows_per_block - 1) / rows_per_block), dim3(kUThreads),
                        args, lds_up, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(ga, dim3(a.tiles), dim3(kGThreads), args, (size_t)a.d * 4, s);
    if (e == hipSuccess) e = hipGetLastError();
    return e;
}

}  // namespace moeffn
