// Sum of per-workgroup partial rows into the output (second kernel of the
// expert and layer paths; two variants by the number of contributions).  Token t's output row is the sum, in a fixed order,
// of `tiles` partials of each of its rows: one row per token for a single
// expert; for a layer, one row per routed choice (at the pair's position in the
// grouped order) and one per shared expert.  Router weights were applied when
// the partials were written.  The order of the additions is fixed, so the
// output is bit-reproducible.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

constexpr int kRedThreads = 256;
constexpr int kCols = 16;               // output columns per workgroup (4 threads x float4)
constexpr int kGroups = kRedThreads / 4;  // contribution groups per workgroup
constexpr int kBatch = 8;               // loads in flight per thread
constexpr int kMaxRowsPerTok = kMaxExpertsPerToken;

__device__ __forceinline__ int part_row(const ReduceArgs &a, int t, int ri)
{
    if (!a.layer) return t;
    if (ri < a.k) return a.pair_pos[t * a.k + ri];
    return a.T * a.k + (ri - a.k) * a.T + t;
}

// One workgroup per (token, 16 columns): about d/16 * T workgroups, so the
// partial rows are read by many compute units at once.
__global__ void __launch_bounds__(kRedThreads)
reduce_kernel(ReduceArgs a)
{
    __shared__ float4 sm[kGroups][4];
    __shared__ int rows_s[kMaxRowsPerTok];
    const int cblocks = a.d / kCols;
    const int t = blockIdx.x / cblocks;
    const int cb = blockIdx.x - t * cblocks;
    for (int ri = threadIdx.x; ri < a.rows_per_tok; ri += kRedThreads) rows_s[ri] = part_row(a, t, ri);
    __syncthreads();
    const int cq = threadIdx.x & 3, tg = threadIdx.x >> 2;
    const int col = cb * kCols + cq * 4;
    const int n = a.rows_per_tok * a.tiles;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // kBatch loads in flight per thread, then added in order
    for (int c0 = tg; c0 < n; c0 += kGroups * kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int ci = c0 + b * kGroups;
            const int cc = ci < n ? ci : tg;
            const int ri = cc / a.tiles, tile = cc - ri * a.tiles;
            v[b] = *(const float4 *)(a.part + ((size_t)rows_s[ri] * a.tiles + tile) * a.d + col);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (c0 + b * kGroups < n) {
                s.x += v[b].x; s.y += v[b].y; s.z += v[b].z; s.w += v[b].w;
            }
        }
    }
    sm[tg][cq] = s;
    __syncthreads();
    if (tg == 0) {
        float4 r = sm[0][cq];
        for (int g = 1; g < kGroups; ++g) {
            const float4 v = sm[g][cq];
            r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
        }
        const size_t base = (size_t)t * a.d + col;
        store_out(a.y, a.ydt, base + 0, r.x, a.accumulate);
        store_out(a.y, a.ydt, base + 1, r.y, a.accumulate);
        store_out(a.y, a.ydt, base + 2, r.z, a.accumulate);
        store_out(a.y, a.ydt, base + 3, r.w, a.accumulate);
    }
}

// Few contributions per output element (the dense path's split-K partials, a
// layer with many tokens): a thread owns 4 adjacent columns of one token and
// adds that token's contributions in order, all of them in flight at once.
constexpr int kRowThreads = 256;
constexpr int kRowCols = 4 * kRowThreads;   // columns per workgroup
constexpr int kRowMax = 64;                 // contributions handled this way
constexpr int kRowBatch = 16;

__global__ void __launch_bounds__(kRowThreads)
reduce_rows_kernel(ReduceArgs a)
{
    __shared__ int rows_s[kMaxRowsPerTok];
    const int cblocks = (a.d + kRowCols - 1) / kRowCols;
    const int t = blockIdx.x / cblocks;
    const int col = (blockIdx.x - t * cblocks) * kRowCols + threadIdx.x * 4;
    for (int ri = threadIdx.x; ri < a.rows_per_tok; ri += kRowThreads) rows_s[ri] = part_row(a, t, ri);
    __syncthreads();
    if (col >= a.d) return;
    const int n = a.rows_per_tok * a.tiles;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < n; c0 += kRowBatch) {
        float4 v[kRowBatch];
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            const int ci = min(c0 + b, n - 1);
            const int ri = ci / a.tiles, tile = ci - ri * a.tiles;
            v[b] = *(const float4 *)(a.part + ((size_t)rows_s[ri] * a.tiles + tile) * a.d + col);
        }
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            if (c0 + b < n) {
                s.x += v[b].x; s.y += v[b].y; s.z += v[b].z; s.w += v[b].w;
            }
        }
    }
    const size_t base = (size_t)t * a.d + col;
    store_out(a.y, a.ydt, base + 0, s.x, a.accumulate);
    store_out(a.y, a.ydt, base + 1, s.y, a.accumulate);
    store_out(a.y, a.ydt, base + 2, s.z, a.accumulate);
    store_out(a.y, a.ydt, base + 3, s.w, a.accumulate);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    if (a.d % kCols != 0 || a.rows_per_tok > kMaxRowsPerTok) return hipErrorInvalidValue;
    if (a.rows_per_tok * a.tiles <= kRowMax) {
        const int cblocks = (a.d + kRowCols - 1) / kRowCols;
        hipLaunchKernelGGL(reduce_rows_kernel, dim3(a.T * cblocks), dim3(kRowThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(reduce_kernel, dim3(a.T * (a.d / kCols)), dim3(kRedThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace moeffn
