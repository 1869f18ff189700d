// Top-k router and token -> expert grouping (MoE-Infinity review, "A3 背景" and
// "4.3"; MoE-Lightning review, "MoE 模型架构").
//
// One workgroup per token computes the E logits (every expert with the same
// code path and reduction order, so identical router rows tie exactly), picks
// the top-k with ties going to the lower index, and writes the softmax
// weights.  With at most 8 experts, wave e forms logit e from x and router
// row e read straight from global memory.  When a token's router rows exceed
// 32 KB with more experts, a first kernel computes the logits that way, one
// wave per (token, expert) over many workgroups, and the per-token kernel only
// ranks them.  A second kernel of one workgroup then groups the T*k (token, slot)
// pairs by expert: counts, exclusive offsets, the pairs of each expert in
// ascending order, their grouped positions, the list of experts that received
// tokens and, for the sparse layer, the table of fixed-size token chunks that
// sets its grid.  A single token is grouped by its own workgroup.  No
// host synchronisation, atomics across workgroups or fences are involved.
#include "device.hpp"
#include "internal.hpp"
#include "route_common.hpp"

namespace moeffn {

namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / 64;

using rc::f16bits;

// x of one token into LDS as fp32, 8 elements per 16-byte unit (32 for fp32
// input), four loads in flight per thread; one copy per input type, so that no
// type test sits between the loads
template <int XT>
__device__ __forceinline__ void stage_x(const void *x, int t, int d, float *xs, int tid)
{
    const int nch = d / 8;
    if constexpr (XT == 2) {
        const float *xf = (const float *)x + (size_t)t * d;
        for (int c0 = tid; c0 < nch; c0 += 2 * kRouteThreads) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = min(c0 + u * kRouteThreads, nch - 1);
                v[2 * u] = *(const float4 *)(xf + (size_t)c * 8);
                v[2 * u + 1] = *(const float4 *)(xf + (size_t)c * 8 + 4);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = c0 + u * kRouteThreads;
                if (c < nch) {
                    *(float4 *)&xs[c * 8] = v[2 * u];
                    *(float4 *)&xs[c * 8 + 4] = v[2 * u + 1];
                }
            }
        }
    } else {
        const uint16_t *xh = (const uint16_t *)x + (size_t)t * d;
        for (int c0 = tid; c0 < nch; c0 += 4 * kRouteThreads) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = min(c0 + u * kRouteThreads, nch - 1);
                v[u] = *(const uint4 *)(xh + (size_t)c * 8);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * kRouteThreads;
                if (c < nch) {
                    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    *(float4 *)&xs[c * 8] = make_float4(f16bits<XT == 1>(w[0] & 0xFFFFu), f16bits<XT == 1>(w[0] >> 16),
                                                        f16bits<XT == 1>(w[1] & 0xFFFFu), f16bits<XT == 1>(w[1] >> 16));
                    *(float4 *)&xs[c * 8 + 4] = make_float4(f16bits<XT == 1>(w[2] & 0xFFFFu), f16bits<XT == 1>(w[2] >> 16),
                                                            f16bits<XT == 1>(w[3] & 0xFFFFu), f16bits<XT == 1>(w[3] >> 16));
                }
            }
        }
    }
}

// Logits of one token: a wave takes GE experts at a time (e = wave, wave + W,
// ...) and a lane the 16-byte units lane, lane + 64, ... of their rows, CB
// units per expert per round: GE * CB loads in flight, all issued (rows and
// units clamped to valid ones) before the products, which drop units and
// experts past the end.  Every expert's sum runs in the same order (units
// ascending within a lane, then a fixed butterfly), so identical router rows
// tie exactly.  WT: router weight type (0 fp16, 1 bf16, 2 fp32).
template <int CB, int GE, int WT>
__device__ __forceinline__ void logits(const RouteArgs &a, const float *xs, const float *bs, float *lg,
                                       int wave, int lane)
{
    const int d = a.d, E = a.E;
    constexpr int esz = WT == 2 ? 4 : 2;
    constexpr int epu = 16 / esz;                       // elements per 16-byte unit
    const int nu = d / epu;
    const unsigned char *rw = (const unsigned char *)a.rw;
    for (int e0 = wave; e0 < E; e0 += kRouteWaves * GE) {
        float p[GE];
#pragma unroll
        for (int g = 0; g < GE; ++g) p[g] = 0.f;
        for (int u0 = 0; u0 < nu; u0 += 64 * CB) {
            uint4 w[GE][CB];
#pragma unroll
            for (int g = 0; g < GE; ++g)
#pragma unroll
                for (int u = 0; u < CB; ++u) {
                    const int e = min(e0 + kRouteWaves * g, E - 1);
                    const int uu = min(u0 + lane + 64 * u, nu - 1);
                    w[g][u] = load_nt16(rw + ((size_t)e * d) * esz + (size_t)uu * 16);
                }
#pragma unroll
            for (int g = 0; g < GE; ++g)
#pragma unroll
                for (int u = 0; u < CB; ++u) {
                    const int uu = u0 + lane + 64 * u;
                    const float *xp = xs + (size_t)min(uu, nu - 1) * epu;
                    float q = p[g];
                    if constexpr (WT == 2) {
                        const float4 xv = *(const float4 *)xp;
                        q += xv.x * __uint_as_float(w[g][u].x);
                        q += xv.y * __uint_as_float(w[g][u].y);
                        q += xv.z * __uint_as_float(w[g][u].z);
                        q += xv.w * __uint_as_float(w[g][u].w);
                    } else {
                        const float4 x0 = *(const float4 *)xp, x1 = *(const float4 *)(xp + 4);
                        q += x0.x * f16bits<WT == 1>(w[g][u].x & 0xFFFFu);
                        q += x0.y * f16bits<WT == 1>(w[g][u].x >> 16);
                        q += x0.z * f16bits<WT == 1>(w[g][u].y & 0xFFFFu);
                        q += x0.w * f16bits<WT == 1>(w[g][u].y >> 16);
                        q += x1.x * f16bits<WT == 1>(w[g][u].z & 0xFFFFu);
                        q += x1.y * f16bits<WT == 1>(w[g][u].z >> 16);
                        q += x1.z * f16bits<WT == 1>(w[g][u].w & 0xFFFFu);
                        q += x1.w * f16bits<WT == 1>(w[g][u].w >> 16);
                    }
                    if (e0 + kRouteWaves * g < E && uu < nu) p[g] = q;
                }
        }
#pragma unroll
        for (int g = 0; g < GE; ++g) {
            const int e = e0 + kRouteWaves * g;
            const float v = seg_sum<64>(p[g]);
            if (lane == 0 && e < E) lg[e] = v + bs[e];
        }
    }
}

// Wide routers: logits only, one wave per (token, expert), eight experts per
// workgroup, so the router rows of a token are read by many compute units at
// once (the shared fixed-order wave dot, so identical router rows tie
// exactly).  route_kernel then ranks them.
template <int XT, int WT>
__device__ __forceinline__ float wave_logit(const RouteArgs &a, int t, int e, int lane)
{
    constexpr int xsz = XT == 2 ? 4 : 2, wsz = WT == 2 ? 4 : 2;
    const unsigned char *xr = (const unsigned char *)a.x + (size_t)t * a.d * xsz;
    const unsigned char *wr = (const unsigned char *)a.rw + (size_t)e * a.d * wsz;
    return rc::wave_row_dot<XT, WT>(xr, wr, a.d, lane) + (a.bias ? a.bias[e] : 0.f);
}

template <int XT>
__device__ __forceinline__ float wave_logit_x(const RouteArgs &a, int t, int e, int lane)
{
    if (a.rdt == 2) return wave_logit<XT, 2>(a, t, e, lane);
    if (a.rdt == 1) return wave_logit<XT, 1>(a, t, e, lane);
    return wave_logit<XT, 0>(a, t, e, lane);
}

template <int XT, int WT>
__global__ void __launch_bounds__(kRouteThreads)
route_logits_kernel(RouteArgs a)
{
    const int nblk = (a.E + kRouteWaves - 1) / kRouteWaves;
    const int t = blockIdx.x / nblk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = (blockIdx.x - t * nblk) * kRouteWaves + wave;
    if (e >= a.E) return;                               // no barriers in this kernel
    const float v = wave_logit<XT, WT>(a, t, e, lane);
    if (lane == 0) a.lg_buf[(size_t)t * a.E + e] = v;
}

// Exclusive scan over the experts of two packed 64-bit values per thread
// (experts 2 tid and 2 tid + 1): returns the exclusive prefixes and the total.
__device__ void expert_exscan(unsigned long long v0, unsigned long long v1,
                              unsigned long long &ex0, unsigned long long &ex1,
                              unsigned long long &total)
{
    __shared__ unsigned long long wsum[kRouteWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long incl = v0 + v1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    unsigned long long base = 0ull;
    total = 0ull;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) {
        if (w < wave) base += wsum[w];
        total += wsum[w];
    }
    ex0 = base + incl - v0 - v1;
    ex1 = ex0 + v0;
    __syncthreads();                                 // wsum is reused by the next scan
}

// Chunk ci of a table whose experts start at chunks cst[0..E] belongs to the
// last expert whose first chunk is <= ci (experts without chunks share the
// next one's start): entry = expert << 16 | first grouped position.
__device__ void write_chunks(const int *cst, const int *run, int E, int csize, int32_t *tab)
{
    const int nc = cst[E];
    for (int ci = threadIdx.x; ci < nc; ci += kRouteThreads) {
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cst[mid] <= ci) lo = mid;
            else hi = mid - 1;
        }
        tab[ci] = (lo << 16) | (run[lo] + (ci - cst[lo]) * csize);
    }
}

// Counting sort of the T*k pairs by expert, stable in pair order.  Reads the
// top-k indices through coherent loads (they were written by this or an
// earlier kernel).  With a.chunk > 0 it also lists every expert's pairs in
// chunks of a.chunk consecutive grouped positions (the last one shorter),
// experts in ascending order: entry = expert << 16 | first position.  With
// a.dense_min > 0 (a layer call that chooses the path per expert) experts with
// at least dense_min pairs are listed instead in chunks of a.dense_chunk in a
// second table (chunk_tab2 / n_chunks2) and flagged in expert_dense.
__device__ void group_pairs(const RouteArgs &a, unsigned char *smem, bool reg, int my_e, float my_w)
{
    // reg: every pair is p = tid and this thread's pair chose expert my_e with
    // weight my_w (a single token with k <= kRouteThreads, known in
    // registers); else the choices are read from memory
    const int tid = threadIdx.x;
    const int E = a.E;
    int *cnt = (int *)smem;                          // [E] counts
    int *run = cnt + E;                              // [E] running placement base
    int *cst = run + E;                              // [E+1] first chunk of each expert
    int *cst2 = cst + E + 1;                         // [E+1] first dense chunk of each expert
    // [E][kRouteWaves] lanes of each wave whose pair of the batch chose expert e
    unsigned long long *msk = (unsigned long long *)(cnt + ((4 * E + 2 + 1) & ~1));
    const int P = a.T * a.k;
    // the experts of this thread's first kHeld pairs (p = tid + kRouteThreads i)
    // are loaded once, all in flight together, and kept for the placement
    constexpr int kHeld = 8;
    int held[kHeld];
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
        const int p = tid + kRouteThreads * i;
        held[i] = p >= P ? -1 : reg ? (i == 0 ? my_e : -1) : load_coherent_i32(a.topk_idx + p);
    }
    for (int e = tid; e < E; e += kRouteThreads) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHeld; ++i)
        if (held[i] >= 0) atomicAdd(&cnt[held[i]], 1);
    for (int p = tid + kRouteThreads * kHeld; p < P; p += kRouteThreads)
        atomicAdd(&cnt[load_coherent_i32(a.topk_idx + p)], 1);
    __syncthreads();
    // one exclusive scan over the experts gives, packed in 64 bits, the pair
    // offset (bits 0-23), the first chunk (24-47) and the position in the
    // active list (48-63) of every expert; no field can overflow (at most
    // 65536 pairs, chunks or experts).  A second scan gives the first dense
    // chunk when the path is chosen per expert.
    {
        auto is_dense = [&](int e) { return a.dense_min > 0 && cnt[e] >= a.dense_min; };
        auto pack = [&](int e) -> unsigned long long {
            if (e >= E) return 0ull;
            const unsigned long long c = (unsigned)cnt[e];
            const unsigned long long nch =
                a.chunk > 0 && !is_dense(e) ? (c + a.chunk - 1) / a.chunk : 0ull;
            return c | (nch << 24) | ((unsigned long long)(c > 0) << 48);
        };
        const int e0 = 2 * tid;                      // this thread's experts: e0, e0 + 1 (E <= 1024)
        unsigned long long ex0, ex1, total;
        expert_exscan(pack(e0), pack(e0 + 1), ex0, ex1, total);
        const unsigned long long ex[2] = {ex0, ex1};
        if (a.dense_min > 0) {
            auto dpack = [&](int e) -> unsigned long long {
                return e < E && is_dense(e) ? (unsigned long long)((cnt[e] + a.dense_chunk - 1) /
                                                                   a.dense_chunk) : 0ull;
            };
            unsigned long long d0, d1, dtot;
            expert_exscan(dpack(e0), dpack(e0 + 1), d0, d1, dtot);
            if (e0 < E) cst2[e0] = (int)d0;
            if (e0 + 1 < E) cst2[e0 + 1] = (int)d1;
            if (tid == 0) {
                cst2[E] = (int)dtot;
                *a.n_chunks2 = (int)dtot;
            }
        }
        if (a.expert_dense)
            for (int e = tid; e < E; e += kRouteThreads) a.expert_dense[e] = is_dense(e) ? 1 : 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = e0 + i;
            if (e < E) {
                const int off = (int)(ex[i] & 0xFFFFFFull);
                a.offset[e] = off;
                run[e] = off;
                cst[e] = (int)((ex[i] >> 24) & 0xFFFFFFull);
                a.count[e] = cnt[e];
                if (a.eam_row) a.eam_row[e] += cnt[e];   // request-level EAM row
                if (a.active && cnt[e] > 0) a.active[(int)(ex[i] >> 48)] = e;
            }
        }
        if (tid == 0) {
            a.offset[E] = (int)(total & 0xFFFFFFull);
            cst[E] = (int)((total >> 24) & 0xFFFFFFull);
            if (a.n_active) *a.n_active = (int)(total >> 48);
            if (a.chunk > 0) *a.n_chunks = cst[E];
        }
    }
    __syncthreads();
    if (a.chunk > 0) write_chunks(cst, run, E, a.chunk, a.chunk_tab);
    if (a.dense_min > 0) write_chunks(cst2, run, E, a.dense_chunk, a.chunk_tab2);
    __syncthreads();
    // stable placement, one chunk of pairs at a time: a pair's rank among the
    // chunk's earlier pairs of its expert is the count of set bits below it in
    // that expert's lane masks (its own wave's, then the earlier waves')
    const int lane = tid & 63, wave = tid >> 6;
    for (int b = 0, bi = 0; b < P; b += kRouteThreads, ++bi) {
        const int p = b + tid;
        int e = -1;                                  // expert of pair p (held, else loaded)
        if (p < P) {
            if (bi < kHeld) {
                e = held[0];
#pragma unroll
                for (int j = 1; j < kHeld; ++j) e = bi == j ? held[j] : e;
            } else {
                e = load_coherent_i32(a.topk_idx + p);
            }
        }
        for (int i = tid; i < E * kRouteWaves; i += kRouteThreads) msk[i] = 0ull;
        __syncthreads();
        if (e >= 0) atomicOr(&msk[e * kRouteWaves + wave], 1ull << lane);
        __syncthreads();
        if (e >= 0) {
            int rank = __popcll(msk[e * kRouteWaves + wave] & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w) rank += __popcll(msk[e * kRouteWaves + w]);
            const int pos = run[e] + rank;
            a.pairs[pos] = p;
            if (a.chunk_rec) {
                // single-token chunks: chunk pos holds pair p; its record lets
                // the expert kernel start from one load
                const float w = reg ? my_w : a.topk_w[p];
                *(int4 *)(a.chunk_rec + 4 * (size_t)pos) = make_int4(e, p, __float_as_int(w), pos);
            }
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kRouteThreads) {   // the batch's pairs of ee follow these
            int c = 0;
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) c += __popcll(msk[ee * kRouteWaves + w]);
            run[ee] += c;
        }
        __syncthreads();
    }
}

template <int CB, int GE>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(RouteArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    float *xs = (float *)smem;                        // [d]
    float *lg = xs + a.d;                             // [E rounded up to 4]
    float *bs = lg + ((a.E + 3) & ~3);                // [E] router bias (0 without one)
    int *sel = (int *)(bs + a.E);                     // [k]
    float *wsel = (float *)(sel + a.k);               // [k] weights of the choices
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = a.d, E = a.E, k = a.k;

    if (a.lg_buf) {
        // logits (bias included) from route_logits_kernel
        for (int e = tid; e < E; e += kRouteThreads) lg[e] = a.lg_buf[(size_t)t * E + e];
        __syncthreads();
    } else if (E <= kRouteWaves) {
        // few experts: wave e forms logit e as the logits kernel does
        if (wave < E) {
            const float v = a.xdt == 2 ? wave_logit_x<2>(a, t, wave, lane)
                          : a.xdt == 1 ? wave_logit_x<1>(a, t, wave, lane)
                                       : wave_logit_x<0>(a, t, wave, lane);
            if (lane == 0) lg[wave] = v;
        }
        __syncthreads();
    } else {
        if (a.xdt == 2) stage_x<2>(a.x, t, d, xs, tid);
        else if (a.xdt == 1) stage_x<1>(a.x, t, d, xs, tid);
        else stage_x<0>(a.x, t, d, xs, tid);
        for (int e = tid; e < E; e += kRouteThreads) bs[e] = a.bias ? a.bias[e] : 0.f;
        __syncthreads();

        if (a.rdt == 2) logits<CB, GE, 2>(a, xs, bs, lg, wave, lane);
        else if (a.rdt == 1) logits<CB, GE, 1>(a, xs, bs, lg, wave, lane);
        else logits<CB, GE, 0>(a, xs, bs, lg, wave, lane);
        __syncthreads();
    }

    // top-k in one ranking pass: the rank of expert e is the number of experts
    // ahead of it in the order (larger logit, then lower index; a NaN logit
    // counts as -inf), and the experts of rank < k are the choices in rank
    // order.  The logits are padded to a multiple of 4 with -inf, which never
    // ranks ahead of a real expert.
    {
        const int E4 = (E + 3) & ~3;
        for (int e = E + tid; e < E4; e += kRouteThreads) lg[e] = -INFINITY;
        __syncthreads();
        rc::rank_topk(lg, E, k, sel, tid, kRouteThreads);
        __syncthreads();
    }
    if (wave == 0) {
        // weights
        const float m = lg[sel[0]];
        const float den = rc::gate_den(lg, sel, E, k, a.renorm, m, lane);
        for (int s = lane; s < k; s += 64) {
            const int e = sel[s];
            const float w = __expf(lg[e] - m) / den;
            a.topk_idx[(size_t)t * k + s] = e;
            a.topk_w[(size_t)t * k + s] = w;
            wsel[s] = w;
        }
        if (a.logits)
            for (int e = lane; e < E; e += 64) a.logits[(size_t)t * E + e] = lg[e];
    }

    if (!a.count || gridDim.x != 1) return;
    __syncthreads();            // one token: its own workgroup groups it
    const int my_e = tid < k ? sel[tid] : 0;      // read before the grouping reuses LDS
    const float my_w = tid < k ? wsel[tid] : 0.f;
    __syncthreads();
    group_pairs(a, smem, k <= kRouteThreads, my_e, my_w);
}

// Grouping of all T*k pairs by one workgroup (after the per-token kernel).
__global__ void __launch_bounds__(kRouteThreads)
group_kernel(RouteArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    group_pairs(a, smem, false, 0, 0.f);
}

}  // namespace

bool route_split(int d, int E, int rdt)
{
    // up to kRouteWaves experts the per-token kernel forms the logits the same way itself
    return E > kRouteWaves && (size_t)E * d * (rdt == 2 ? 4 : 2) > (32u << 10);
}

namespace {
template <int XT>
const void *logits_kernel_for(int rdt)
{
    if (rdt == 2) return (const void *)route_logits_kernel<XT, 2>;
    if (rdt == 1) return (const void *)route_logits_kernel<XT, 1>;
    return (const void *)route_logits_kernel<XT, 0>;
}
}  // namespace

hipError_t launch_route_logits(const RouteArgs &a, hipStream_t s)
{
    const void *lk = a.xdt == 2 ? logits_kernel_for<2>(a.rdt)
                   : a.xdt == 1 ? logits_kernel_for<1>(a.rdt) : logits_kernel_for<0>(a.rdt);
    const int nblk = (a.E + kRouteWaves - 1) / kRouteWaves;
    void *largs[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(lk, dim3((unsigned)a.T * nblk), dim3(kRouteThreads), largs, 0, s);
    if (e == hipSuccess) e = hipGetLastError();
    return e;
}

hipError_t launch_route(const RouteArgs &a, hipStream_t s)
{
    if (a.lg_buf) {
        const hipError_t e = launch_route_logits(a, s);
        if (e != hipSuccess) return e;
    }
    size_t lds = (size_t)a.d * 4 + (size_t)a.E * 8 + (size_t)a.k * 8 + 32;
    // counts, bases and chunk starts (4 E + 2 ints), then the lane masks
    // ([E][8] u64)
    const size_t lds_group = (size_t)a.E * 16 + 16 + (size_t)a.E * kRouteWaves * 8 + 64;
    if (lds_group > lds) lds = lds_group;
    // 16-byte units per lane of one router row (64 lanes): CB (<= 8) of them per
    // expert and round, GE = 16 / CB experts per wave at a time
    const int nu = a.d * (a.rdt == 2 ? 4 : 2) / 16;
    const int cpl = (nu + 63) / 64;
    const void *kern;
    if (cpl > 4) kern = (const void *)route_kernel<8, 2>;
    else if (cpl > 2) kern = (const void *)route_kernel<4, 4>;
    else if (cpl > 1) kern = (const void *)route_kernel<2, 8>;
    else kern = (const void *)route_kernel<1, 16>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    void *args[] = {(void *)&a};
    hipError_t e = hipLaunchKernel(kern, dim3(a.T), dim3(kRouteThreads), args, lds, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess || !a.count || a.T == 1) return e;
    if (lds_group > 64 * 1024) {
        e = hipFuncSetAttribute((const void *)group_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds_group);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kRouteThreads), lds_group, s, a);
    return hipGetLastError();
}

}  // namespace moeffn
