// Dense grouped-GEMM path on bf16 MFMA for batched tokens (threshold off).
// MoE-Lightning review, "层次化屋顶模型": the MoE FFN's operational intensity
// grows with the micro-batch, so with many tokens per expert the expert FFN is
// a real contraction; FloE review, "MoE 专家前向计算" gives what it computes:
//   H_e = SiLU(X_e W^gate) (.) (X_e W^up),   Y_e = H_e W^down,
// and the layer adds each token's rows with its router weight (shared experts
// with weight 1).
//
// Kernel 1 (gate/up): a workgroup of 8 waves owns 128 intermediate channels of
// one expert and loops over the expert's tokens in 64-row chunks; wave w takes
// token half w & 1 and channel quarter w >> 1.  v_mfma_f32_32x32x16_bf16 runs
// with the tokens as rows (A) and the weight rows as columns (B).  Each
// 128-wide k block of the gate, up and x tiles is copied straight from global
// memory into LDS (whole 256-byte row pieces, four rows per instruction), one
// block ahead of the one being multiplied, in two 80 KB stages; weights are
// read from HBM once.  The reduction index k is permuted inside
// every 64-wide block (lane half h takes k = 32h + 8s + 0..7 at step s); A and
// B use the same permutation, which leaves the sum unchanged.  Epilogue:
// h = SiLU(g) * u in fp32 to the workspace.  When experts average more than
// 64 tokens, gateup128_kernel takes 128 tokens per pass instead (64-wide k
// blocks in three 48 KB stages, two in flight), so each staged weight block
// feeds twice the products and the weights stream half as often.
// Kernel 2 (down): a workgroup owns 128 output columns and one quarter of the
// intermediate channels (split-K); A = H split into bf16 hi + lo parts (so H
// keeps ~16 significant bits), B = W^down.  W^down is stored channel-major
// ([f][d], the layout the sparse path gathers rows from), so a 64 x 128 tile
// is loaded with coalesced row reads into LDS and each lane collects its 8
// consecutive k values of one column from there; H is staged in LDS as bf16
// hi and lo tiles once per workgroup.  Both are double-buffered, one k block
// ahead.  Results are scaled by the router weight and stored as partial rows;
// the shared reduction kernel sums them.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));    // register-friendly 16-byte value

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

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi)
{
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

constexpr int kXP = 72;         // halves per LDS row of a 64-wide k block (16-byte pad)

// gate/up tiles per 128-wide k block, copied global -> LDS: 64 gate rows, 64
// up rows and 64 x rows of 256 bytes (a long run per weight row, which HBM
// serves far better than 128-byte pieces).  A row's sixteen 16-byte chunks are
// stored with the low three bits of the chunk index XOR-swizzled by (row & 7),
// so a fragment read (32 rows, one chunk each) is free of bank conflicts.
constexpr int kGuThreads = 512;
constexpr int kGuWaves = kGuThreads / 64;
constexpr int kGuBN = 128;                                          // channels per workgroup
constexpr int kGuStages = 2;
constexpr int kGuRows = 2 * kGuBN + 64;                             // gate, up and x rows of a stage
constexpr size_t kGuStage = (size_t)kGuRows * 256;                  // bytes
constexpr size_t kGuLds = kGuStages * kGuStage;                     // 160 KB
constexpr int kGuCopies = kGuRows * 16 / 64 / kGuWaves;            // 16-byte copies per lane per stage (10)

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + 16 * (chunk ^ (row & 7)); }

__global__ void __launch_bounds__(kGuThreads)
gateup_kernel(DenseArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int nblk = a.f / kGuBN;
    const int slot = blockIdx.x / nblk;
    const int nb = blockIdx.x - slot * nblk;
    const SlotInfo si = slot_info(a, slot);
    if (!si.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, li = lane & 31;
    const int mt = wave & 1, nt = wave >> 1;                        // token half, channel quarter
    const int d = a.d;
    const int j = nb * kGuBN + nt * 32 + li;                        // this lane's B column
    const size_t wbase = (size_t)si.e * a.f * d + (size_t)nb * kGuBN * d;
    const int nkb = d / 128;

    for (int m0 = 0; m0 < si.ntok; m0 += 64) {
        // copy q of wave w covers tile rows 4 (w kGuCopies + q) .. + 3
        const uint16_t *src[kGuCopies];
#pragma unroll
        for (int q = 0; q < kGuCopies; ++q) {
            const int p = (wave * kGuCopies + q) * 64 + lane;           // 16-byte position in the stage
            const int row = p >> 4, c = (p & 15) ^ (row & 7);           // tile row, source chunk
            const uint16_t *rp;
            if (row < kGuBN) {
                rp = a.gate + wbase + (size_t)row * d;
            } else if (row < 2 * kGuBN) {
                rp = a.up + wbase + (size_t)(row - kGuBN) * d;
            } else {
                const int m = m0 + row - 2 * kGuBN;                     // rows past the chunk read
                rp = a.x + (size_t)(m < si.ntok ? token_of(a, si, m) : 0) * d;   // a valid token
            }
            src[q] = rp + 8 * c;
        }
        auto issue = [&](int kb, int stage) {
            unsigned char *base = smem + (size_t)stage * kGuStage;
#pragma unroll
            for (int q = 0; q < kGuCopies; ++q)
                copy16_to_lds(src[q] + (size_t)kb * 128, base + (size_t)(wave * kGuCopies + q) * 1024);
        };

        floatx16 ag, au;
        for (int r = 0; r < 16; ++r) { ag[r] = 0.f; au[r] = 0.f; }
        const bool mine = m0 + 32 * mt < si.ntok;                   // this wave's token half has tokens

        issue(0, 0);
        for (int kb = 0; kb < nkb; ++kb) {
            // block kb's copies are the only ones in flight
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            // the stage written next held block kb - 1, which every wave has finished
            if (kb + 1 < nkb) issue(kb + 1, (kb + 1) % kGuStages);
            if (mine) {
                const unsigned char *st = smem + (size_t)(kb % kGuStages) * kGuStage;
                const int gr = nt * 32 + li, ur = kGuBN + nt * 32 + li, xr = 2 * kGuBN + mt * 32 + li;
#pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) {
                    const int c = 8 * h + s8;                       // k = 64h + 8 s8 + 0..7
                    const uint4 bg = *(const uint4 *)(st + swz(gr, c));
                    const uint4 bu = *(const uint4 *)(st + swz(ur, c));
                    const uint4 ax = *(const uint4 *)(st + swz(xr, c));
                    ag = mfma(ax, bg, ag);
                    au = mfma(ax, bu, au);
                }
            }
        }
        __syncthreads();        // the stages are reused by the next token chunk
        // D layout: value r of lane l is row 8(r/4) + 4h + r%4, column l%32
        if (mine) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 8 * (r >> 2) + 4 * h + (r & 3);
                const int m = m0 + 32 * mt + i;
                if (m < si.ntok)
                    a.h[(size_t)(si.hrow0 + m) * a.f + j] = silu(ag[r]) * au[r];
            }
        }
    }
}

// gate/up for experts with many tokens: 128 tokens per pass, so each weight
// block staged in LDS feeds twice the products.  Stage = one 64-wide k block:
// 128 gate, 128 up and 128 x rows of 128 bytes (48 KB), three stages, two
// blocks in flight.  Wave w owns channel quarter w >> 1 and token quarters
// 2 (w & 1) and 2 (w & 1) + 1.  Chunks are XOR-swizzled by (row & 7) as above.
constexpr int kG2Rows = 2 * kGuBN + 128;
constexpr size_t kG2Stage = (size_t)kG2Rows * 128;                 // 48 KB
constexpr int kG2Stages = 3;
constexpr size_t kG2Lds = kG2Stages * kG2Stage;                    // 144 KB
constexpr int kG2Copies = kG2Rows * 8 / 64 / kGuWaves;            // 16-byte copies per lane per stage (6)

__device__ __forceinline__ int swz2(int row, int chunk) { return row * 128 + 16 * (chunk ^ (row & 7)); }

__global__ void __launch_bounds__(kGuThreads)
gateup128_kernel(DenseArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int nblk = a.f / kGuBN;
    const int slot = blockIdx.x / nblk;
    const int nb = blockIdx.x - slot * nblk;
    const SlotInfo si = slot_info(a, slot);
    if (!si.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, li = lane & 31;
    const int mp = wave & 1, nt = wave >> 1;                        // token-quarter pair, channel quarter
    const int d = a.d;
    const int j = nb * kGuBN + nt * 32 + li;                        // this lane's B column
    const size_t wbase = (size_t)si.e * a.f * d + (size_t)nb * kGuBN * d;
    const int nkb = d / 64;

    for (int m0 = 0; m0 < si.ntok; m0 += 128) {
        // copy q of wave w covers tile rows 8 (w kG2Copies + q) .. + 7
        const uint16_t *src[kG2Copies];
#pragma unroll
        for (int q = 0; q < kG2Copies; ++q) {
            const int p = (wave * kG2Copies + q) * 64 + lane;           // 16-byte position in the stage
            const int row = p >> 3, c = (p & 7) ^ (row & 7);            // tile row, source chunk
            const uint16_t *rp;
            if (row < kGuBN) {
                rp = a.gate + wbase + (size_t)row * d;
            } else if (row < 2 * kGuBN) {
                rp = a.up + wbase + (size_t)(row - kGuBN) * d;
            } else {
                const int m = m0 + row - 2 * kGuBN;                     // rows past the chunk read
                rp = a.x + (size_t)(m < si.ntok ? token_of(a, si, m) : 0) * d;   // a valid token
            }
            src[q] = rp + 8 * c;
        }
        auto issue = [&](int kb, int stage) {
            unsigned char *base = smem + (size_t)stage * kG2Stage;
#pragma unroll
            for (int q = 0; q < kG2Copies; ++q)
                copy16_to_lds(src[q] + (size_t)kb * 64, base + (size_t)(wave * kG2Copies + q) * 1024);
        };

        floatx16 ag[2], au[2];
        for (int i = 0; i < 2; ++i)
            for (int r = 0; r < 16; ++r) { ag[i][r] = 0.f; au[i][r] = 0.f; }
        bool mine[2];
        for (int i = 0; i < 2; ++i) mine[i] = m0 + 32 * (2 * mp + i) < si.ntok;

        issue(0, 0);
        if (nkb > 1) issue(1, 1);
        for (int kb = 0; kb < nkb; ++kb) {
            // this wave's copies of block kb are done once at most the next
            // block's remain in flight
            if (kb + 1 < nkb) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kG2Copies) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            // the stage written next held block kb - 1, which every wave has finished
            if (kb + 2 < nkb) issue(kb + 2, (kb + 2) % kG2Stages);
            const unsigned char *st = smem + (size_t)(kb % kG2Stages) * kG2Stage;
            const int gr = nt * 32 + li, ur = kGuBN + nt * 32 + li;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int c = 4 * h + s4;                           // k = 32h + 8 s4 + 0..7
                const uint4 bg = *(const uint4 *)(st + swz2(gr, c));
                const uint4 bu = *(const uint4 *)(st + swz2(ur, c));
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (mine[i]) {
                        const int xr = 2 * kGuBN + 32 * (2 * mp + i) + li;
                        const uint4 ax = *(const uint4 *)(st + swz2(xr, c));
                        ag[i] = mfma(ax, bg, ag[i]);
                        au[i] = mfma(ax, bu, au[i]);
                    }
                }
            }
        }
        __syncthreads();        // the stages are reused by the next pass
        // D layout: value r of lane l is row 8(r/4) + 4h + r%4, column l%32
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (!mine[i]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * (2 * mp + i) + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < si.ntok)
                    a.h[(size_t)(si.hrow0 + m) * a.f + j] = silu(ag[i][r]) * au[i][r];
            }
        }
    }
}

constexpr int kBP = 136;        // halves per LDS row of a down-weight tile (128 columns + pad)
constexpr size_t kDownHs = (size_t)2 * 64 * kXP;                  // hi + lo H tiles (halves)
constexpr size_t kDownBs = (size_t)64 * kBP;                      // one weight tile (halves)
constexpr size_t kDownLds = (2 * kDownHs + 2 * kDownBs) * 2 + 64 * 8;

__global__ void __launch_bounds__(kDenseThreads)
down_kernel(DenseArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *hs = (uint16_t *)smem;                                // [2 buf][hi, lo][64][kXP]
    uint16_t *bs = hs + 2 * kDownHs;                                // [2 buf][64 k][kBP]
    int *row_s = (int *)(bs + 2 * kDownBs);                         // [64]
    float *sc_s = (float *)(row_s + 64);                            // [64]
    const int nblk = a.d / kNB;
    const int per_slot = nblk * kKSplit;
    const int slot = blockIdx.x / per_slot;
    const int rem = blockIdx.x - slot * per_slot;
    const int nb = rem / kKSplit, ks = rem - nb * kKSplit;
    const SlotInfo si = slot_info(a, slot);
    if (!si.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, li = lane & 31;
    const int d = a.d, f = a.f;
    const int c = nb * kNB + wave * 32 + li;                        // this lane's output column
    const int kspan = f / kKSplit;
    const int k_beg = ks * kspan, k_end = k_beg + kspan;
    const uint16_t *dtile = a.down + (size_t)si.e * f * d + nb * kNB;
    // loaders: H tile 64 x 64 fp32 (4 float4 per thread), weight tile 64 x 128
    // bf16 (4 uint4 per thread)
    const int hm = tid >> 4, hc = tid & 15;                         // H rows hm + 16q, k 4hc..
    const int bk = tid >> 4, bc = tid & 15;                         // W rows bk + 16q, cols 8bc..

    for (int m0 = 0; m0 < si.ntok; m0 += 64) {
        const int nm = min(64, si.ntok - m0);
        if (tid < 64) {
            int row = 0;
            float sc = 0.f;
            if (tid < nm) {
                // partial rows: routed ones by pair t k + s, shared ones after them
                if (si.shared) {
                    row = si.hrow0 + m0 + tid;
                    sc = 1.f;
                } else {
                    const int p = a.pairs[si.pair0 + m0 + tid];
                    row = p;
                    sc = a.topk_w[p];
                }
            }
            row_s[tid] = row;
            sc_s[tid] = sc;
        }
        // rows past the chunk read row 0 and are zeroed when stored
        const float *hbase = a.h + (size_t)(si.hrow0 + m0) * f + 4 * hc;
        int hoff[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) hoff[q] = (hm + 16 * q < nm ? hm + 16 * q : 0) * f;

        floatx16 acc[2];
        for (int mt = 0; mt < 2; ++mt)
            for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
        const bool two = 32 < nm;

#define DOWN_LOAD(KB)                                                                          \
    for (int q = 0; q < 4; ++q) {                                                              \
        hv[q] = *(const float4 *)(hbase + hoff[q] + (KB));                                     \
        wv[q] = *(const u32x4 *)(dtile + (size_t)((KB) + bk + 16 * q) * d + 8 * bc);           \
    }
#define DOWN_STORE(BUF)                                                                        \
    for (int q = 0; q < 4; ++q) {                                                              \
        const bool ok = hm + 16 * q < nm;                                                      \
        const float v[4] = {ok ? hv[q].x : 0.f, ok ? hv[q].y : 0.f, ok ? hv[q].z : 0.f,        \
                            ok ? hv[q].w : 0.f};                                               \
        uint16_t hi[4], lo[4];                                                                 \
        for (int e = 0; e < 4; ++e) {                                                          \
            hi[e] = float_to_bf16_bits(v[e]);                                                  \
            lo[e] = float_to_bf16_bits(v[e] - bf16_bits_to_float(hi[e]));                      \
        }                                                                                      \
        uint16_t *hhi = hs + (size_t)(BUF) * kDownHs;                                          \
        const int o = (hm + 16 * q) * kXP + 4 * hc;                                            \
        *(uint2 *)&hhi[o] = make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));  \
        *(uint2 *)&hhi[64 * kXP + o] = make_uint2(pack_bf16x2(lo[0], lo[1]),                   \
                                                  pack_bf16x2(lo[2], lo[3]));                  \
        *(u32x4 *)&bs[(size_t)(BUF) * kDownBs + (bk + 16 * q) * kBP + 8 * bc] = wv[q];         \
    }
        float4 hv[4];
        u32x4 wv[4];
#pragma unroll
        DOWN_LOAD(k_beg)
#pragma unroll
        DOWN_STORE(0)
        __syncthreads();
        int cur = 0;
        for (int kb = k_beg; kb < k_end; kb += 64) {
            const bool more = kb + 64 < k_end;
            if (more) {                                             // in flight during the products
#pragma unroll
                DOWN_LOAD(kb + 64)
            }
            const uint16_t *hhi = hs + (size_t)cur * kDownHs;
            const uint16_t *hlo = hhi + 64 * kXP;
            const uint16_t *bt = bs + (size_t)cur * kDownBs;
#pragma unroll 2
            for (int s4 = 0; s4 < 4; ++s4) {
                // B fragment: k = 32h + 8 s4 + 0..7 of this lane's column, read across rows
                const int kr = 32 * h + 8 * s4;
                uint16_t bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[e] = bt[(kr + e) * kBP + wave * 32 + li];
                const uint4 b = make_uint4(pack_bf16x2(bv[0], bv[1]), pack_bf16x2(bv[2], bv[3]),
                                           pack_bf16x2(bv[4], bv[5]), pack_bf16x2(bv[6], bv[7]));
                const uint4 ahi0 = *(const uint4 *)&hhi[li * kXP + kr];
                const uint4 alo0 = *(const uint4 *)&hlo[li * kXP + kr];
                acc[0] = mfma(ahi0, b, acc[0]);
                acc[0] = mfma(alo0, b, acc[0]);
                if (two) {
                    const uint4 ahi1 = *(const uint4 *)&hhi[(32 + li) * kXP + kr];
                    const uint4 alo1 = *(const uint4 *)&hlo[(32 + li) * kXP + kr];
                    acc[1] = mfma(ahi1, b, acc[1]);
                    acc[1] = mfma(alo1, b, acc[1]);
                }
            }
            if (more) {         // the other buffers were last read before the previous barrier
#pragma unroll
                DOWN_STORE(cur ^ 1)
            }
            __syncthreads();
            cur ^= 1;
        }
#undef DOWN_LOAD
#undef DOWN_STORE
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
    if (a.f % kNB != 0 || a.d % kNB != 0 || (a.f / kKSplit) % 64 != 0 || a.f % kGuBN != 0)
        return hipErrorInvalidValue;
    const int slots = a.S + (a.E < a.T * a.k ? a.E : a.T * a.k);
    // experts averaging more than 64 tokens take the 128-token passes
    const bool wide = (long long)a.T * a.k > 64ll * a.E;
    const void *gk = wide ? (const void *)gateup128_kernel : (const void *)gateup_kernel;
    const size_t glds = wide ? kG2Lds : kGuLds;
    hipError_t e = hipFuncSetAttribute(gk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)glds);
    if (e != hipSuccess) return e;
    if (wide)
        hipLaunchKernelGGL(gateup128_kernel, dim3(slots * (a.f / kGuBN)), dim3(kGuThreads), glds, s, a);
    else
        hipLaunchKernelGGL(gateup_kernel, dim3(slots * (a.f / kGuBN)), dim3(kGuThreads), glds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void *)down_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kDownLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(down_kernel, dim3(slots * (a.d / kNB) * kKSplit), dim3(kDenseThreads), kDownLds, s, a);
    return hipGetLastError();
}

}  // namespace moeffn
