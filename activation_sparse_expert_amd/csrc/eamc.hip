// Nearest stored request-level expert activation matrix (MoE-Infinity review,
// "4.5 请求级稀疏激活追踪": a new request's EAM is compared with the EAMs kept
// in the collection by the cosine distance of the flattened matrices, and the
// closest one is the match; "4.3" defines the EAM as the L x E integer matrix
// of tokens routed to each expert).
//
// Two kernels.  The first gives every stored EAM one wave: the dot product
// with the query and both squared norms are summed exactly in 64-bit integers
// (entries below 2^22 and at most 2^17 of them keep every sum below 2^61), so
// the order of the additions does not matter, and the distance
// 1 - dot / sqrt(|a|^2 |b|^2) is then formed in fp64.  The second, one
// workgroup, takes the smallest distance, the lowest index among equal ones.
// The stored EAMs are read once (nontemporal loads); the query is read by every
// wave and stays in the caches.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

constexpr int kEamThreads = 256;
constexpr int kEamWaves = kEamThreads / 64;
constexpr unsigned kEntryLimit = 1u << 22;
constexpr int kArgThreads = 1024;

typedef unsigned long long u64;

__device__ __forceinline__ u64 wave_sum_u64(u64 v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// VEC: rows read as 16-byte pieces (len % 4 == 0, 16-byte aligned bases)
template <bool VEC>
__global__ void __launch_bounds__(kEamThreads)
eamc_dist_kernel(const int32_t *eamc, int n, int len, const int32_t *query, double *dist)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * kEamWaves + (threadIdx.x >> 6);
    if (i >= n) return;                       // a whole wave; no barrier follows
    const int32_t *b = eamc + (size_t)i * len;
    // unsigned sums: exact for valid entries, defined (wrapping) for the rest,
    // which the range flags discard
    u64 dot = 0, na = 0, nb = 0;
    unsigned bad = 0;
    auto add = [&](int32_t x, int32_t y) {
        bad |= (unsigned)((unsigned)x >= kEntryLimit) | ((unsigned)((unsigned)y >= kEntryLimit) << 1);
        dot += (u64)((long long)x * y);
        na += (u64)((long long)x * x);
        nb += (u64)((long long)y * y);
    };
    if constexpr (VEC) {
        const int n4 = len / 4;
        int c = lane;
        // four 16-byte pieces of the row in flight per lane, then the tail
        for (; c + 3 * 64 < n4; c += 4 * 64) {
            uint4 bb[4];
            int4 qa[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) bb[u] = load_nt16(b + 4 * (size_t)(c + 64 * u));
#pragma unroll
            for (int u = 0; u < 4; ++u) qa[u] = *(const int4 *)(query + 4 * (size_t)(c + 64 * u));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                add(qa[u].x, (int32_t)bb[u].x);
                add(qa[u].y, (int32_t)bb[u].y);
                add(qa[u].z, (int32_t)bb[u].z);
                add(qa[u].w, (int32_t)bb[u].w);
            }
        }
        for (; c < n4; c += 64) {
            const int4 qa = *(const int4 *)(query + 4 * (size_t)c);
            const uint4 bb = load_nt16(b + 4 * (size_t)c);
            add(qa.x, (int32_t)bb.x);
            add(qa.y, (int32_t)bb.y);
            add(qa.z, (int32_t)bb.z);
            add(qa.w, (int32_t)bb.w);
        }
    } else {
        for (int c = lane; c < len; c += 64) add(query[c], (int32_t)load_nt4(b + c));
    }
    dot = wave_sum_u64(dot);
    na = wave_sum_u64(na);
    nb = wave_sum_u64(nb);
    const bool bad_any = __any(bad != 0);
    if (lane == 0) {
        double r;
        if (bad_any) r = __builtin_nan("");
        else if (na == 0 || nb == 0) r = 1.0;  // a zero vector has no direction
        else r = 1.0 - (double)dot / sqrt((double)na * (double)nb);
        dist[i] = r;
    }
}

// (d, i) is better than (bd, bi) when it is a valid entry with a smaller
// distance, or the same distance at a lower index; NaN never wins
__device__ __forceinline__ bool better(double d, int i, double bd, int bi)
{
    return i >= 0 && (bi < 0 || d < bd || (d == bd && i < bi));
}

__global__ void __launch_bounds__(kArgThreads)
eamc_argmin_kernel(const double *dist, int n, int32_t *idx_out)
{
    __shared__ double sd[kArgThreads / 64];
    __shared__ int si[kArgThreads / 64];
    double bd = 0.0;
    int bi = -1;
    for (int i = threadIdx.x; i < n; i += kArgThreads) {
        const double v = dist[i];
        if (v == v && better(v, i, bd, bi)) { bd = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double od = __shfl_xor(bd, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better(od, oi, bd, bi)) { bd = od; bi = oi; }
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { sd[wave] = bd; si[wave] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kArgThreads / 64; ++w)
            if (better(sd[w], si[w], bd, bi)) { bd = sd[w]; bi = si[w]; }
        idx_out[0] = bi;
    }
}

}  // namespace

hipError_t launch_eamc_match(const int32_t *eamc, int n, int len, const int32_t *query,
                             int32_t *idx_out, double *dist, hipStream_t s)
{
    const bool vec = len % 4 == 0 && ((uintptr_t)eamc & 15) == 0 && ((uintptr_t)query & 15) == 0;
    const unsigned blocks = (unsigned)((n + kEamWaves - 1) / kEamWaves);
    if (vec) hipLaunchKernelGGL(eamc_dist_kernel<true>, dim3(blocks), dim3(kEamThreads), 0, s,
                                eamc, n, len, query, dist);
    else hipLaunchKernelGGL(eamc_dist_kernel<false>, dim3(blocks), dim3(kEamThreads), 0, s,
                            eamc, n, len, query, dist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(eamc_argmin_kernel, dim3(1), dim3(kArgThreads), 0, s, dist, n, idx_out);
    return hipGetLastError();
}

}  // namespace moeffn
