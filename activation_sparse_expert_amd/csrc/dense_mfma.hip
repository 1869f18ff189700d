// Dense grouped-GEMM path on bf16 MFMA for batched tokens (threshold off).
// MoE-Lightning review, "层次化屋顶模型": the MoE FFN's operational intensity
// grows with the micro-batch, so with many tokens per expert the expert FFN is
// a real contraction; FloE review, "MoE 专家前向计算" gives what it computes:
//   H_e = SiLU(X_e W^gate) (.) (X_e W^up),   Y_e = H_e W^down,
// and the layer adds each token's rows with its router weight (shared experts
// with weight 1).
//
// Kernel 1 (gate/up): a workgroup of 4 waves owns 128 intermediate channels of
// one expert (32 per wave) and loops over the expert's tokens in 64-row
// chunks.  v_mfma_f32_32x32x16_bf16 runs with the tokens as rows (A) and the
// weight rows as columns (B); weights are read once, straight from HBM into
// registers with 16-byte loads.  The reduction index k is permuted inside
// every 64-wide block (lane half h takes k = 32h + 8s + 0..7 at step s); A and
// B use the same permutation, which leaves the sum unchanged.  Epilogue:
// h = SiLU(g) * u in fp32 to the workspace.
// Kernel 2 (down): a workgroup owns 128 output columns and one quarter of the
// intermediate channels (split-K); A = H split into bf16 hi + lo parts (so H
// keeps ~16 significant bits), B = W^down.  Results are scaled by the router
// weight and stored as partial rows; the shared reduction kernel sums them.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kDenseThreads = 256;
constexpr int kNB = 128;        // columns per workgroup (4 waves x 32)
constexpr int kKSplit = kDenseKSplit;

__device__ __forceinline__ floatx16 mfma(const uint4 &a, const uint4 &b, const floatx16 &c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Slot -> (expert, token count, first pair) as in the sparse kernel.
struct SlotInfo {
    int e, ntok, pair0, hrow0;
    bool shared;
    bool valid;
};

__device__ __forceinline__ SlotInfo slot_info(const DenseArgs &a, int slot)
{
    SlotInfo s{};
    if (slot < a.S) {
        s.e = a.E + slot;
        s.ntok = a.T;
        s.shared = true;
        s.pair0 = 0;
        s.hrow0 = a.T * a.k + slot * a.T;
        s.valid = true;
    } else {
        const int ai = slot - a.S;
        s.valid = ai < *a.n_active;
        if (!s.valid) return s;
        s.e = a.active[ai];
        s.pair0 = a.offset[s.e];
        s.ntok = a.offset[s.e + 1] - s.pair0;
        s.shared = false;
        s.hrow0 = s.pair0;
    }
    return s;
}

__device__ __forceinline__ int token_of(const DenseArgs &a, const SlotInfo &s, int m)
{
    return s.shared ? m : a.pairs[s.pair0 + m] / a.k;
}

__global__ void __launch_bounds__(kDenseThreads)
gateup_kernel(DenseArgs a)
{
    const int nblk = a.f / kNB;
    const int slot = blockIdx.x / nblk;
    const int nb = blockIdx.x - slot * nblk;
    const SlotInfo si = slot_info(a, slot);
    if (!si.valid) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, li = lane & 31;
    const int d = a.d;
    const int j = nb * kNB + wave * 32 + li;                       // this lane's B column
    const uint16_t *grow = a.gate + (size_t)si.e * a.f * d + (size_t)j * d + 32 * h;
    const uint16_t *urow = a.up + (size_t)si.e * a.f * d + (size_t)j * d + 32 * h;

    for (int m0 = 0; m0 < si.ntok; m0 += 64) {
        const uint16_t *xrow[2];
        bool xv[2];
        for (int mt = 0; mt < 2; ++mt) {
            const int m = m0 + 32 * mt + li;
            xv[mt] = m < si.ntok;
            xrow[mt] = a.x + (size_t)(xv[mt] ? token_of(a, si, m) : 0) * d + 32 * h;
        }
        floatx16 ag[2], au[2];
        for (int mt = 0; mt < 2; ++mt)
            for (int r = 0; r < 16; ++r) { ag[mt][r] = 0.f; au[mt][r] = 0.f; }
        const bool two = (m0 + 32) < si.ntok;
        for (int kb = 0; kb < d; kb += 64) {
            uint4 bg[4], bu[4], ax[2][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bg[s] = *(const uint4 *)(grow + kb + 8 * s);
                bu[s] = *(const uint4 *)(urow + kb + 8 * s);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    ax[mt][s] = xv[mt] ? *(const uint4 *)(xrow[mt] + kb + 8 * s) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ag[0] = mfma(ax[0][s], bg[s], ag[0]);
                au[0] = mfma(ax[0][s], bu[s], au[0]);
                if (two) {
                    ag[1] = mfma(ax[1][s], bg[s], ag[1]);
                    au[1] = mfma(ax[1][s], bu[s], au[1]);
                }
            }
        }
        // D layout: value r of lane l is row 8(r/4) + 4h + r%4, column l%32
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * h + (r & 3);
                const int m = m0 + 32 * mt + i;
                if (m < si.ntok)
                    a.h[(size_t)(si.hrow0 + m) * a.f + j] = silu(ag[mt][r]) * au[mt][r];
            }
        }
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

__global__ void __launch_bounds__(kDenseThreads)
down_kernel(DenseArgs a)
{
    const int nblk = a.d / kNB;
    const int per_slot = nblk * kKSplit;
    const int slot = blockIdx.x / per_slot;
    const int rem = blockIdx.x - slot * per_slot;
    const int nb = rem / kKSplit, ks = rem - nb * kKSplit;
    const SlotInfo si = slot_info(a, slot);
    if (!si.valid) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, li = lane & 31;
    const int d = a.d, f = a.f;
    const int c = nb * kNB + wave * 32 + li;                        // this lane's output column
    const int kspan = f / kKSplit;
    const int k_beg = ks * kspan, k_end = k_beg + kspan;
    const uint16_t *dcol = a.down + (size_t)si.e * f * d + c;

    __shared__ int row_s[64];
    __shared__ float sc_s[64];

    for (int m0 = 0; m0 < si.ntok; m0 += 64) {
        const int nm = min(64, si.ntok - m0);
        if (threadIdx.x < 64) {
            const int m = m0 + threadIdx.x;
            int row = 0;
            float sc = 0.f;
            if (threadIdx.x < nm) {
                row = si.hrow0 + m;
                sc = si.shared ? 1.f : a.topk_w[a.pairs[si.pair0 + m]];
            }
            row_s[threadIdx.x] = row;
            sc_s[threadIdx.x] = sc;
        }
        __syncthreads();
        floatx16 acc[2];
        for (int mt = 0; mt < 2; ++mt)
            for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
        const bool two = 32 < nm;
        const float *hrow[2];
        bool hv[2];
        for (int mt = 0; mt < 2; ++mt) {
            const int m = 32 * mt + li;
            hv[mt] = m < nm;
            hrow[mt] = a.h + (size_t)(si.hrow0 + m0 + (hv[mt] ? m : 0)) * f + 32 * h;
        }
        for (int kb = k_beg; kb < k_end; kb += 64) {
            uint4 b[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint16_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = dcol[(size_t)(kb + 32 * h + 8 * s + e) * d];
                b[s] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                if (mt == 1 && !two) break;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    float hv8[8];
                    if (hv[mt]) {
                        const float4 p0 = *(const float4 *)(hrow[mt] + kb + 8 * s);
                        const float4 p1 = *(const float4 *)(hrow[mt] + kb + 8 * s + 4);
                        hv8[0] = p0.x; hv8[1] = p0.y; hv8[2] = p0.z; hv8[3] = p0.w;
                        hv8[4] = p1.x; hv8[5] = p1.y; hv8[6] = p1.z; hv8[7] = p1.w;
                    } else {
                        for (int e = 0; e < 8; ++e) hv8[e] = 0.f;
                    }
                    uint16_t hi[8], lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        hi[e] = float_to_bf16_bits(hv8[e]);
                        lo[e] = float_to_bf16_bits(hv8[e] - bf16_bits_to_float(hi[e]));
                    }
                    const uint4 ahi = make_uint4(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                                                 pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7]));
                    const uint4 alo = make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                                 pack_bf16x2(lo[4], lo[5]), pack_bf16x2(lo[6], lo[7]));
                    acc[mt] = mfma(ahi, b[s], acc[mt]);
                    acc[mt] = mfma(alo, b[s], acc[mt]);
                }
            }
        }
        // scaled partial rows: [row][ks][d]
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
                if (i < nm)
                    a.part[((size_t)row_s[i] * kKSplit + ks) * d + c] = sc_s[i] * acc[mt][r];
            }
        }
        __syncthreads();
    }
}

}  // namespace

size_t dense_h_bytes(int T, int f, int k, int S)
{
    return (size_t)T * (k + S) * f * 4;
}

hipError_t launch_dense_layer(const DenseArgs &a, hipStream_t s)
{
    if (a.f % kNB != 0 || a.d % kNB != 0 || (a.f / kKSplit) % 64 != 0) return hipErrorInvalidValue;
    const int slots = a.S + (a.E < a.T * a.k ? a.E : a.T * a.k);
    hipLaunchKernelGGL(gateup_kernel, dim3(slots * (a.f / kNB)), dim3(kDenseThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(down_kernel, dim3(slots * (a.d / kNB) * kKSplit), dim3(kDenseThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moeffn
