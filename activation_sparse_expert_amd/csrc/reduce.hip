// Sum of per-workgroup partial rows into the output (second kernel of the
// expert and layer paths).  Token t's output row is the sum, in a fixed order,
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

// One workgroup per (token, 16 columns): about d/16 * T workgroups, so the
// partial rows are read by many compute units at once.
__global__ void __launch_bounds__(kRedThreads)
reduce_kernel(ReduceArgs a)
{
    __shared__ float4 sm[kGroups][4];
    const int cblocks = a.d / kCols;
    const int t = blockIdx.x / cblocks;
    const int cb = blockIdx.x - t * cblocks;
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
            int row;
            if (!a.layer) row = t;
            else if (ri < a.k) row = a.pair_pos[t * a.k + ri];
            else row = a.T * a.k + (ri - a.k) * a.T + t;
            v[b] = *(const float4 *)(a.part + ((size_t)row * a.tiles + tile) * a.d + col);
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

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    if (a.d % kCols != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reduce_kernel, dim3(a.T * (a.d / kCols)), dim3(kRedThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moeffn
