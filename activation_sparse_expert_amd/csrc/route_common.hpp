// Router steps shared by the routing kernels and by the expert kernel, which
// routes a single token itself (MoE-Infinity review, "A3 背景": top-k gating
// over the router's logits; MoE-Lightning review, "MoE 模型架构").  One code
// path per step, so that both callers form bit-identical logits, choices and
// weights.
#pragma once
#include "device.hpp"

namespace moeffn {
namespace rc {

// 16-bit float bits to float (bf16 or fp16), chosen at compile time
template <bool BF>
__device__ __forceinline__ float f16bits(uint32_t b)
{
    return BF ? bf16_bits_to_float((uint16_t)b) : half_bits_to_float((uint16_t)b);
}

// 8 elements of a 16-bit (T_ 0 fp16, 1 bf16) or fp32 (2) array at element
// offset 8 g, as floats (one or two 16-byte loads)
template <int T_>
__device__ __forceinline__ void load8(const void *base, size_t g, float (&v)[8])
{
    if constexpr (T_ == 2) {
        const float4 a = *((const float4 *)base + 2 * g), b = *((const float4 *)base + 2 * g + 1);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 u = *((const uint4 *)base + g);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = f16bits<T_ == 1>(w[i] & 0xFFFFu);
            v[2 * i + 1] = f16bits<T_ == 1>(w[i] >> 16);
        }
    }
}

// x_row . w_row over d elements by one wave: lane l takes the 8-element groups
// l, l + 64, ... (4 of each in flight), in ascending order, and the lanes'
// sums are added by a fixed butterfly, so identical router rows give
// identical logits.  XT / WT: element types (0 fp16, 1 bf16, 2 fp32).
template <int XT, int WT>
__device__ __forceinline__ float wave_row_dot(const void *x_row, const void *w_row, int d, int lane)
{
    const int ng = d / 8;
    constexpr int CB = 4;                               // groups per lane per round
    float acc = 0.f;
    for (int g0 = 0; g0 < ng; g0 += 64 * CB) {
        float xv[CB][8], wv[CB][8];
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int g = min(g0 + lane + 64 * i, ng - 1);
            load8<XT>(x_row, g, xv[i]);
            load8<WT>(w_row, g, wv[i]);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            float q = acc;
#pragma unroll
            for (int j = 0; j < 8; ++j) q += xv[i][j] * wv[i][j];
            if (g0 + lane + 64 * i < ng) acc = q;
        }
    }
    return seg_sum<64>(acc);
}

// Logit of expert e for one token: the row dot plus the router bias.
template <int XT>
__device__ __forceinline__ float wave_logit_rows(const void *x_row, const void *rw, int rdt, int d,
                                                 const float *bias, int e, int lane)
{
    float v;
    if (rdt == 2) v = wave_row_dot<XT, 2>(x_row, (const float *)rw + (size_t)e * d, d, lane);
    else if (rdt == 1) v = wave_row_dot<XT, 1>(x_row, (const uint16_t *)rw + (size_t)e * d, d, lane);
    else v = wave_row_dot<XT, 0>(x_row, (const uint16_t *)rw + (size_t)e * d, d, lane);
    return v + (bias ? bias[e] : 0.f);
}

// Top-k in one ranking pass over lg [E4] (padded with -inf to a multiple of
// 4): the rank of expert e is the number of experts ahead of it (larger
// logit, then lower index; a NaN logit counts as -inf), and sel[r] = the
// expert of rank r < k.  Threads tid, tid + nthr, ... take the experts.
__device__ __forceinline__ void rank_topk(const float *lg, int E, int k, int *sel, int tid, int nthr)
{
    const int E4 = (E + 3) & ~3;
    for (int e = tid; e < E; e += nthr) {
        const float le = lg[e] != lg[e] ? -INFINITY : lg[e];
        int r = 0;
#pragma unroll 4
        for (int e2 = 0; e2 < E4; e2 += 4) {
            const float4 l4 = *(const float4 *)&lg[e2];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float l2 = lv[j] != lv[j] ? -INFINITY : lv[j];
                // branch-free: ahead if larger, or equal with a lower index
                r += (int)(l2 > le) | ((int)(l2 == le) & (int)(e2 + j < e));
            }
        }
        if (r < k) sel[r] = e;
    }
}

// Softmax denominator of the gate weights, formed by one wave: over the k
// chosen logits (renorm) or over all E, each term exp(l - m) with m the
// largest chosen logit; lanes add their terms in order, then a fixed
// butterfly.  Weight of choice s = exp(lg[sel[s]] - m) / den.
__device__ __forceinline__ float gate_den(const float *lg, const int *sel, int E, int k, int renorm,
                                          float m, int lane)
{
    float den = 0.f;
    if (renorm) {
        for (int s = lane; s < k; s += 64) den += __expf(lg[sel[s]] - m);
    } else {
        for (int e = lane; e < E; e += 64) den += __expf(lg[e] - m);
    }
    return seg_sum<64>(den);
}

}  // namespace rc
}  // namespace moeffn
