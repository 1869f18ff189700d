// Sum of per-workgroup partial rows into the output (second kernel of the
// expert and layer paths; two variants by the number of contributions).
// Token t's output row is the sum, in a fixed order, of `tiles` partials of
// each of its rows: one row per token for a single expert; for a layer, one row
// per routed choice (row t k + s for choice s) and one per shared expert.  Router weights were applied when
// the partials were written.  The order of the additions is fixed, so the
// output is bit-reproducible.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

constexpr int kRedThreads = 256;
constexpr int kCols = 32;               // output columns per workgroup: one 128-byte line of a row
constexpr int kSeg = kCols / 4;         // threads per line (float4 each)
constexpr int kGroups = kRedThreads / kSeg;  // contribution groups per workgroup
constexpr int kBatch = 8;               // loads in flight per thread
constexpr int kMaxRowsPerTok = kMaxExpertsPerToken;

__device__ __forceinline__ int part_row(const ReduceArgs &a, int t, int ri)
{
    if (!a.layer) return t;
    if (ri < a.k) return t * a.k + ri;            // routed: the pair's own row
    return a.T * a.k + (ri - a.k) * a.T + t;
}

// Partials held by row ri of token t (at least one).
__device__ __forceinline__ int part_tiles(const ReduceArgs &a, int t, int ri)
{
    if (!a.mix) return a.tiles;
    if (ri < a.k) return a.expert_dense[a.topk_idx[(size_t)t * a.k + ri]] ? a.tiles_dense : a.tiles;
    return a.shared_dense ? a.tiles_dense : a.tiles;
}

// Row table of token t in LDS: partial row, and the first contribution of
// each row (prefix over the rows' partial counts); returns the total.
__device__ int stage_rows(const ReduceArgs &a, int t, int *rows_s, int *pre_s)
{
    const int R = a.rows_per_tok;
    for (int ri = threadIdx.x; ri < R; ri += blockDim.x) {
        rows_s[ri] = part_row(a, t, ri);
        pre_s[ri + 1] = part_tiles(a, t, ri);
    }
    __syncthreads();
    if (threadIdx.x == 0) {                       // k + S <= 1024 rows: a short serial prefix
        pre_s[0] = 0;
        for (int ri = 0; ri < R; ++ri) pre_s[ri + 1] += pre_s[ri];
    }
    __syncthreads();
    return pre_s[R];
}

// Row holding contribution c (largest ri with pre_s[ri] <= c).
__device__ __forceinline__ int row_of(const int *pre_s, int R, int c)
{
    int lo = 0, hi = R - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre_s[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One workgroup per (token, 32 columns): d/32 * T workgroups, so the partial
// rows are read by many compute units at once, in whole 128-byte lines.
// Contribution c = ri * tiles + tile (row ri of the token, tile `tile`); group g
// of kSeg threads adds contributions g, g + kGroups, ... in that order, then the
// groups' sums are added by a butterfly within each wave and then wave by wave: a fixed order.  A single expert's
// token has one row (row t), so that case skips the row table.
template <bool LAYER>
__global__ void __launch_bounds__(kRedThreads)
reduce_kernel(ReduceArgs a)
{
    __shared__ float4 sm[kRedThreads / 64][kSeg];
    __shared__ int rows_s[LAYER ? kMaxRowsPerTok : 1];
    __shared__ int pre_s[LAYER ? kMaxRowsPerTok + 1 : 1];
    const int cblocks = a.d / kCols;
    const int t = blockIdx.x / cblocks;
    const int cb = blockIdx.x - t * cblocks;
    const int stride = a.stride > 0 ? a.stride : a.tiles;
    const int cq = threadIdx.x % kSeg, tg = threadIdx.x / kSeg;
    const int col = cb * kCols + cq * 4;
    int n;
    if constexpr (LAYER) n = stage_rows(a, t, rows_s, pre_s);
    else n = a.tiles;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = tg; c0 < n; c0 += kGroups * kBatch) {
        float4 v[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int c = c0 + b * kGroups;
            const bool ok = c < n;
            int row = t, tl = ok ? c : 0;
            if constexpr (LAYER) {
                const int r = ok ? row_of(pre_s, a.rows_per_tok, c) : 0;
                row = rows_s[r];
                tl = ok ? c - pre_s[r] : 0;
            }
            v[b] = load_nt16f(a.part + ((size_t)row * stride + tl) * a.d + col);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (c0 + b * kGroups < n) {
                s.x += v[b].x; s.y += v[b].y; s.z += v[b].z; s.w += v[b].w;
            }
        }
    }
    // groups of one wave by butterfly (lanes with the same column slot), then
    // the waves in order through LDS: a fixed order
    static_assert(kSeg == 8, "butterfly strides 8, 16, 32");
    s.x = bfly_add<32>(bfly_add<16>(bfly_add<8>(s.x)));
    s.y = bfly_add<32>(bfly_add<16>(bfly_add<8>(s.y)));
    s.z = bfly_add<32>(bfly_add<16>(bfly_add<8>(s.z)));
    s.w = bfly_add<32>(bfly_add<16>(bfly_add<8>(s.w)));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) < kSeg) sm[wave][cq] = s;
    __syncthreads();
    if (tg == 0) {
        float4 r = sm[0][cq];
        for (int w = 1; w < kRedThreads / 64; ++w) {
            const float4 v = sm[w][cq];
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
constexpr int kRowMax = 64;                 // contributions handled this way ...
constexpr int kRowFew = 16;                 // ... always up to this many, else only
constexpr int kRowMinBlocks = 256;          // when the grid still has this many workgroups
constexpr int kRowBatch = 16;

__global__ void __launch_bounds__(kRowThreads)
reduce_rows_kernel(ReduceArgs a)
{
    __shared__ int rows_s[kMaxRowsPerTok];
    __shared__ int pre_s[kMaxRowsPerTok + 1];
    const int cblocks = (a.d + kRowCols - 1) / kRowCols;
    const int t = blockIdx.x / cblocks;
    const int col = (blockIdx.x - t * cblocks) * kRowCols + threadIdx.x * 4;
    const int stride = a.stride > 0 ? a.stride : a.tiles;
    const int n = stage_rows(a, t, rows_s, pre_s);
    if (col >= a.d) return;
    int ri = 0, tile = 0;                       // (row, tile) of contribution c0 + b
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < n; c0 += kRowBatch) {
        float4 v[kRowBatch];
#pragma unroll
        for (int b = 0; b < kRowBatch; ++b) {
            const bool ok = c0 + b < n;
            const int r = ok ? ri : 0, tl = ok ? tile : 0;
            v[b] = load_nt16f(a.part + ((size_t)rows_s[r] * stride + tl) * a.d + col);
            if (ok && ++tile == pre_s[ri + 1] - pre_s[ri]) {   // every row holds >= 1
                tile = 0;
                ++ri;
            }
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
    const int most = a.mix && a.tiles_dense > a.tiles ? a.tiles_dense : a.tiles;
    // few contributions: a thread per 4 columns adds them all; more of them
    // over few tokens (a grid of T * d / 1024 workgroups would leave most of
    // the chip idle while each thread loads them in sequence): the 32-column
    // kernel, whose thread groups hold a token's contributions in flight at once
    const int cblocks = (a.d + kRowCols - 1) / kRowCols;
    const int contrib = a.rows_per_tok * most;
    if (contrib <= kRowMax && (contrib <= kRowFew || (long long)a.T * cblocks >= kRowMinBlocks)) {
        hipLaunchKernelGGL(reduce_rows_kernel, dim3(a.T * cblocks), dim3(kRowThreads), 0, s, a);
    } else {
        if (a.layer)
            hipLaunchKernelGGL(reduce_kernel<true>, dim3(a.T * (a.d / kCols)), dim3(kRedThreads), 0, s, a);
        else
            hipLaunchKernelGGL(reduce_kernel<false>, dim3(a.T * (a.d / kCols)), dim3(kRedThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace moeffn
